// kernels.hpp -- launch interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdr {

enum { IO_F32 = 0, IO_BF16 = 1 };
enum { DECAY_NONE = 0, DECAY_SCALAR = 1, DECAY_CHANNEL = 2 };

constexpr int kChunk = 64;

struct DecodeArgs {
    const void *q, *k, *v;   // [B,Hqk,D], [B,Hqk,D], [B,Hv,D]
    const float *g;          // [B,Hv] or [B,Hv,D] or null
    const float *beta;       // [B,Hv] or null
    const void *bg, *wg;     // [B,Hv,D] or null
    float *S;                // [B,Hv,D,D] in/out
    void *o;                 // [B,Hv,D]
    int B, Hqk, Hv, decay;
    float scale;
};

struct ChunkArgs {
    const void *q, *k, *v;   // [B,T,Hqk,D], [B,T,Hqk,D], [B,T,Hv,D]
    const float *g;          // [B,T,Hv] or [B,T,Hv,D] or null
    const float *beta;       // [B,T,Hv] or null
    const void *bg, *wg;     // [B,T,Hv,D] or null
    const float *S0;         // [B,Hv,D,D] or null
    void *o;                 // [B,T,Hv,D]
    float *ST;               // [B,Hv,D,D]
    void *ws_io;             // per chunk unit: Y, Q~ (C x D), Kend^T, U_z^T (D x C), A (C x C), io dtype
    float *ws_gamma;         // per chunk unit: end-of-chunk decay, D floats
    int B, T, Hqk, Hv, decay, NC;
    float scale;
};

// Elements of the io-dtype workspace per chunk unit, and the byte layout.
__host__ __device__ inline size_t chunk_ws_io_elems(int D) { return (size_t)4 * kChunk * D + (size_t)kChunk * kChunk; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t chunk_ws_bytes(int B, int Hv, int NC, int D, int io) {
    const size_t units = (size_t)B * Hv * NC;
    const size_t esz = io == IO_BF16 ? 2 : 4;
    return align256(units * chunk_ws_io_elems(D) * esz) + units * D * sizeof(float);
}

hipError_t launch_decode(int io, int D, const DecodeArgs &a, hipStream_t s);
hipError_t launch_chunk(int io, int D, const ChunkArgs &a, hipStream_t s);
hipError_t launch_state_fill(float *dst, const float *src, size_t n, hipStream_t s);
bool chunk_supported(int io, int D);

}  // namespace gdr
