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
    void *ws_io;             // per chunk unit, io dtype, matrix-core fragment order: Y (C x D); with
                             // per-channel decay also Q~ (C x D) and Kend^T (D x C); U_z^T (D x C); A (C x C)
    float *ws_tab;           // per chunk unit, kTab floats: per-channel decay: gamma (D);
                             // otherwise exp(G_t) and exp(G_end - G_t) (C each)
    void *ws_kT;             // scalar or no decay: k^T (D x C, fragment order) per (sequence, QK head, chunk)
    int B, T, Hqk, Hv, decay, NC;
    float scale;
};

constexpr int kTab = 2 * kChunk;  // floats per chunk unit in ws_tab (>= D for every supported D)

// Workspace layout. With a scalar decay (or none) the queries and the
// end-of-chunk keys are not stored per V head: the sweep reads q directly and
// one k^T per QK head, and applies the per-token decay factors itself.
__host__ __device__ inline size_t chunk_ws_io_elems(int D, bool chan) {
    return (size_t)(chan ? 4 : 2) * kChunk * D + (size_t)kChunk * kChunk;
}
__host__ __device__ inline size_t ws_off_uz(int D, bool chan) { return (size_t)(chan ? 3 : 1) * kChunk * D; }
__host__ __device__ inline size_t ws_off_a(int D, bool chan) { return (size_t)(chan ? 4 : 2) * kChunk * D; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
struct ChunkWsLayout {
    size_t io_bytes, tab_bytes, kT_bytes;
    size_t total() const { return io_bytes + tab_bytes + kT_bytes; }
};
inline ChunkWsLayout chunk_ws_layout(int B, int Hqk, int Hv, int NC, int D, int io, bool chan) {
    const size_t units = (size_t)B * Hv * NC;
    const size_t esz = io == IO_BF16 ? 2 : 4;
    ChunkWsLayout L;
    L.io_bytes = align256(units * chunk_ws_io_elems(D, chan) * esz);
    L.tab_bytes = align256(units * kTab * sizeof(float));
    L.kT_bytes = chan ? 0 : align256((size_t)B * Hqk * NC * D * kChunk * esz);
    return L;
}

hipError_t launch_decode(int io, int D, const DecodeArgs &a, hipStream_t s);
hipError_t launch_chunk(int io, int D, const ChunkArgs &a, hipStream_t s);
hipError_t launch_state_fill(float *dst, const float *src, size_t n, hipStream_t s);
bool chunk_supported(int io, int D);

}  // namespace gdr
