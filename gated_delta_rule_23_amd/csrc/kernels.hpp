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

// Multi-token recurrent forward: the prefill layouts and gate modes, no workspace.
struct RecurArgs {
    const void *q, *k, *v;   // [B,T,Hqk,D], [B,T,Hqk,D], [B,T,Hv,D]
    const float *g;          // [B,T,Hv] or [B,T,Hv,D] or null
    const float *beta;       // [B,T,Hv] or null
    const void *bg, *wg;     // [B,T,Hv,D] or null
    const float *S0;         // [B,Hv,D,D] or null (zeros)
    float *ST;               // [B,Hv,D,D]; may equal S0
    void *o;                 // [B,T,Hv,D]
    int B, T, Hqk, Hv, decay;
    float scale;
    // Input stage (conv_w non-null): q, k, v are raw projections and the
    // gate and decay arrays hold their inputs before the activations.
    const float *conv_w;     // [(2 Hqk + Hv) D, 4] taps
    const void *conv_in;     // [B, 3, (2 Hqk + Hv) D] or null (zeros)
    void *conv_out;          // same layout, or null
    const float *decay_scale;  // [Hv] or null (1)
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
    void *ws_kT;             // scalar or no decay: k^T (D x C) then q (C x D), fragment order, per
                             // (sequence, QK head, chunk)
    float *ws_seg;           // segmented sweep (P > 1): per (sequence, V head, segment < P - 1) the
                             // segment's transition M (D x D), its end state from zero N (D x D; for
                             // segment 0, a copy of S0 once the scan has read N), and the entry state of
                             // the next segment (D x D), fp32
    int B, T, Hqk, Hv, decay, NC;
    int P, L;                // sweep segments and their length in chunks (P = 1: one pass)
    float scale;
    // Input stage (conv_w non-null), as in RecurArgs.
    const float *conv_w;
    const void *conv_in;
    void *conv_out;
    const float *decay_scale;
    // chunk_prep: V heads of one QK head that a work item runs back to back
    // (divides Hv / Hqk; chosen by the launcher, 0 from callers).
    int prep_grp;
    // Per-channel decay with the input stage: q, k, v come convolved and
    // normalised from the stage pass, while g, beta, b and w are the raw
    // inputs of their activations, which the prep applies as it loads them
    // (decay_scale as for the input stage).
    int raw_gates;
};

constexpr int kTab = 2 * kChunk;  // floats per chunk unit in ws_tab (>= D for every supported D)

// Workspace layout. With a scalar decay (or none) the queries and the
// end-of-chunk keys are not stored per V head: the sweep reads one k^T and one
// q per QK head and applies the per-token decay factors itself.
__host__ __device__ inline size_t chunk_ws_io_elems(int D, bool chan) {
    return (size_t)(chan ? 4 : 2) * kChunk * D + (size_t)kChunk * kChunk;
}
__host__ __device__ inline size_t ws_off_uz(int D, bool chan) { return (size_t)(chan ? 3 : 1) * kChunk * D; }
__host__ __device__ inline size_t ws_off_a(int D, bool chan) { return (size_t)(chan ? 4 : 2) * kChunk * D; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
struct ChunkWsLayout {
    size_t io_bytes, tab_bytes, kT_bytes, seg_bytes;
    size_t total() const { return io_bytes + tab_bytes + kT_bytes + seg_bytes; }
};
// Segments of the sequential sweep. When few (sequence, head, value tile)
// work items would leave most of the device idle and the sequence is long,
// the chunks are split into P segments that run in parallel from their true
// entry states, found by a short scan over the segments' transitions. The
// policy depends only on the shapes (sized for MI355X's 256 compute units),
// so the workspace size needs no device query. The sweep is split when its
// 32-column work items would fill at most half the device. With bf16 io at
// d = 128 the split sweep then runs 64-column work items (half as many per
// segment) and the segment pass runs three 32-column items per CU, so half
// again as many segments fit: P = 1 + 384 / items (measured: on 16 heads of
// 64k tokens 7 segments beat 5 and 8).
constexpr int kSegCUs = 256, kSegMinChunks = 16, kSegMax = 8;
inline void chunk_segments(int B, int Hv, int D, int NC, int io, int &P, int &L) {
    const long long items = (long long)B * Hv * (D / 32);
    long long p = items > 0 ? kSegCUs / items : 1;
    p = p < NC / kSegMinChunks ? p : NC / kSegMinChunks;
    p = p < kSegMax ? p : kSegMax;
    if (p < 2) { P = 1; L = NC; return; }
    if (io == IO_BF16 && D == 128) {
        p = 1 + 3 * kSegCUs / (2 * items);
        p = p < NC / kSegMinChunks ? p : NC / kSegMinChunks;
        p = p < kSegMax ? p : kSegMax;
    }
    L = (int)((NC + p - 1) / p);
    P = (NC + L - 1) / L;
}

inline ChunkWsLayout chunk_ws_layout(int B, int Hqk, int Hv, int NC, int D, int io, bool chan) {
    const size_t units = (size_t)B * Hv * NC;
    const size_t esz = io == IO_BF16 ? 2 : 4;
    ChunkWsLayout L;
    L.io_bytes = align256(units * chunk_ws_io_elems(D, chan) * esz);
    L.tab_bytes = align256(units * kTab * sizeof(float));
    L.kT_bytes = chan ? 0 : align256((size_t)2 * B * Hqk * NC * D * kChunk * esz);
    int P, Ls;
    chunk_segments(B, Hv, D, NC, io, P, Ls);
    L.seg_bytes = P > 1 ? align256((size_t)3 * B * Hv * (P - 1) * D * D * sizeof(float)) : 0;
    return L;
}

// Gradients of the recurrence (recurrent form). Work items are (sequence, V
// head, tile of kBwdCols value columns); the state is checkpointed every
// kBwdBlock tokens by a forward pass, and each block is replayed before it is
// walked in reverse.
constexpr int kBwdBlock = 4, kBwdCols = 32;
struct BwdArgs {
    const void *q, *k, *v;   // [B,T,Hqk,D], [B,T,Hqk,D], [B,T,Hv,D] (io dtype)
    const float *g;          // [B,T,Hv] or [B,T,Hv,D] or null
    const float *beta;       // [B,T,Hv] or null
    const void *bg, *wg;     // [B,T,Hv,D] or null
    const float *S0;         // [B,Hv,D,D] or null (zeros)
    const void *dO;          // [B,T,Hv,D] (io dtype)
    const float *dST;        // [B,Hv,D,D] or null (zeros)
    float *dq, *dk;          // [B,T,Hqk,D]
    float *dv;               // [B,T,Hv,D]
    float *dg;               // shape of g, or null
    float *dbeta;            // [B,T,Hv] (tied gates) or null
    float *db, *dw;          // [B,T,Hv,D] (decoupled gates) or null
    float *dS0;              // [B,Hv,D,D] or null (not written)
    float *ws_ck;            // state entering every block of kBwdBlock tokens: [NB][B][Hv][D][D]
    float *ws_part;          // per-tile partial sums over the tile's value columns, [B][T][Hv][D] each:
                             // s S_t do, dS u, -Sbar du, rowsum(dSbar . S_{t-1}) for every tile; then
                             // v . dz per tile, [B][T][Hv]
    int B, T, Hqk, Hv, decay;
    float scale;
};
struct BwdWsLayout {
    size_t ck_bytes, part_bytes;
    size_t total() const { return ck_bytes + part_bytes; }
};
inline BwdWsLayout bwd_ws_layout(int B, int T, int Hv, int D) {
    const size_t NB = ((size_t)T + kBwdBlock - 1) / kBwdBlock, tiles = (size_t)D / kBwdCols;
    const size_t th = (size_t)B * T * Hv;
    BwdWsLayout L;
    L.ck_bytes = align256(NB * B * Hv * D * D * sizeof(float));
    L.part_bytes = align256((4 * tiles * th * D + tiles * th) * sizeof(float));
    return L;
}

// The input stage as a pass of its own (stage.hip), used by the chunked
// prefill of per-channel-decay layers: raw projections and gate inputs in,
// processed q, k, v, activated gates and the decay g out (prefill layouts).
struct StageArgs {
    const void *q, *k, *v;       // raw [B,T,Hqk,D], [B,T,Hqk,D], [B,T,Hv,D] (io)
    const float *conv_w;         // [(2 Hqk + Hv) D, 4]
    const void *conv_in;         // [B, 3, (2 Hqk + Hv) D] (io) or null (zeros)
    void *conv_out;              // same layout, or null
    void *qo, *ko, *vo;          // processed q, k, v (io)
    int B, T, Hqk, Hv;
};
// Bytes of each processed array in the workspace, in this order, each on a
// 256-byte boundary: q, k, v (io). The gates and the decay stay in the
// caller's arrays: the prefill's load stage applies their activations.
struct StageWsLayout {
    size_t qk, v;                // bytes of q (= k) and of v
    size_t total() const { return 2 * qk + v; }
};
inline StageWsLayout stage_ws_layout(int B, int T, int Hqk, int Hv, int D, int io) {
    const size_t esz = io == IO_BF16 ? 2 : 4, tok = (size_t)B * T;
    StageWsLayout L;
    L.qk = align256(tok * Hqk * D * esz);
    L.v = align256(tok * Hv * D * esz);
    return L;
}
hipError_t launch_stage(int io, int D, const StageArgs &a, hipStream_t s);

hipError_t launch_decode(int io, int D, const DecodeArgs &a, hipStream_t s);
// Chunked backward (chunk_bwd.hip). Per chunk unit u = (b * Hv + h) * NC + c
// the workspace holds fp32 arrays, row-major:
struct ChunkBwdArgs {
    const void *q, *k, *v;   // as BwdArgs
    const float *g, *beta;
    const void *bg, *wg;
    const float *S0;
    const void *dO;
    const float *dST;
    float *dq, *dk, *dv, *dg, *dbeta, *db, *dw, *dS0;
    float *wUz;                   // [units][C][D]: U_z = L Z
    float *wQt;                   // [units][D][C]: Q~^T
    float *wU, *wdU;              // [units][C][D]: U of the chunk; dU, then dR = L^T dU
    float *wdE, *wdQ, *wdK;       // [units][C][D]: -dR S^T, s dO S^T, U dS_next^T
    float *wA, *wT, *wdA, *wdT;   // [units][C][C]
    float *wS, *wdS;              // [units][D][D]: state entering the chunk; dL/d(state leaving it)
    float *wG;                    // [units][C][D] (per-channel decay) or [units][C]: in-chunk log-decay sums
    float *wGam, *wdGam;          // [units][D]: exp(G_end); rowsum(dS_next . S)
    float *wdq, *wdk;             // [B][T][Hv][D] per-V-head parts (grouped heads), else null
    float *wYt, *wKet;            // [units][D][C]: Y^T (Y = L E~), Kend^T
    // Not separate arrays: p = s A^T dO and b = s (Q~ - A Y)^T dO of the
    // backward sweep, from its first kernel to its last reader, live where
    // cb_grad_s later writes -dR S^T (wP = wdE) and s dO S^T, U dS_next^T
    // (wB = wdQ, which with wdK after it holds 2 C D >= D D floats per unit).
    float *wP, *wB;
    int B, T, Hqk, Hv, decay, NC;
    float scale;
};
// The workspace is carved into kChunkBwdArrays arrays in the order of the
// pointer fields wUz .. wKet above, each starting on a 256-byte boundary.
constexpr int kChunkBwdArrays = 20;
struct ChunkBwdWsLayout {
    size_t floats[kChunkBwdArrays];
    size_t total() const {
        size_t t = 0;
        for (int i = 0; i < kChunkBwdArrays; ++i) t += align256(floats[i] * 4);
        return t;
    }
};
inline ChunkBwdWsLayout chunk_bwd_ws_layout(int B, int T, int Hqk, int Hv, int D) {
    const size_t units = (size_t)B * Hv * ((T + kChunk - 1) / kChunk);
    const size_t cd = units * kChunk * D, cc = units * kChunk * kChunk, dd = units * D * D, vd = units * D;
    const size_t part = Hv > Hqk ? (size_t)B * T * Hv * D : 0;
    return ChunkBwdWsLayout{{cd, cd, cd, cd, cd, cd, cd, cc, cc, cc, cc, dd, dd, cd, vd, vd, part, part, cd, cd}};
}

hipError_t launch_backward(int io, int D, const BwdArgs &a, hipStream_t s);
hipError_t launch_chunk_backward(int io, int D, const ChunkBwdArgs &a, hipStream_t s);
hipError_t launch_chunk(int io, int D, const ChunkArgs &a, hipStream_t s);
hipError_t launch_recurrent(int io, int D, const RecurArgs &a, hipStream_t s);
hipError_t launch_state_fill(float *dst, const float *src, size_t n, hipStream_t s);
bool chunk_supported(int io, int D);

}  // namespace gdr
