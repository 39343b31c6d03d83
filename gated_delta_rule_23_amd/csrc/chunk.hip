// chunk.hip -- chunkwise-parallel prefill of the gated delta-rule mixer.
//
// The chunked schedule: "Chunkwise KDA: reorganizando a recorrência como
// multiplicações de matrizes" and "Pipeline Triton da versão por chunks"
// (page "Uma análise das variantes de atenção linear da família DeltaNet"),
// generalised to decoupled erase/write gates as in "Treinamento Paralelo
// Eficiente por Blocos" (page "Resumo Técnico: Gated DeltaNet-2"). For a
// chunk of C = 64 tokens with entry state S_c (d_k x d_v), G_i the in-chunk
// inclusive prefix sum of g = log(alpha), e the erase key and z the gated value:
//
//   E~ = e . exp(G)     Q~ = q . exp(G)     Kend = k . exp(G_end - G)
//   gamma = exp(G_end)
//   T_ij = sum_c e_ic k_jc exp(G_ic - G_jc)  (j < i)
//   A_ij = sum_c q_ic k_jc exp(G_ic - G_jc)  (j <= i)
//   L = (I + T)^-1                 (unit lower triangular; no dense solve)
//   Y = L E~        U_z = L Z      (erase side / write side of the WY form)
//   U = U_z - Y S_c                (the resolved errors)
//   O = s (Q~ S_c + A U)
//   S_{c+1} = Diag(gamma) S_c + Kend^T U
//
// Two kernels. chunk_prep is parallel over every (sequence, V head, chunk):
// it does everything that does not depend on the state -- prefix sums, decay
// absorption, both Gram products (never as E~ times k . exp(-G), which
// overflows once a channel decays by more than about 88 inside a chunk; see
// the block-referenced factors below), the triangular solve for Y and U_z -- and
// stores Y, U_z^T and A (with per-channel decay also Q~, Kend^T and gamma;
// with a scalar decay per-token decay factors and one k^T per QK head) in a
// workspace, each matrix in the order the sweep's matrix-core operand loads
// read it. chunk_sweep is the
// single sequential pass over chunks: per (sequence, V head, value tile) it
// keeps the fp32 state in matrix-core accumulator registers and per chunk
// does U = U_z - Y S_c, O = s (Q~ S_c + A U) and
// S_{c+1} = gamma . S_c + Kend^T U. Value columns of the state evolve
// independently, so the sweep is split over value tiles. When few work items
// would leave the device idle on a long sequence, the sweep is also split
// over time: chunk_seg_state forms each segment's affine map (transition and
// end state from zero), chunk_seg_combine chains the maps into each
// segment's entry state, and chunk_sweep runs the segments side by side.
//
// Matrix products run on gfx950 MFMA: bf16 operands with fp32 accumulation
// for bfloat16 io, fp32 operands for float32 io. The triangular inverse is
// formed in fp32 from 16 x 16 diagonal blocks, then block forward
// substitution (the 16-token diagonal blocks first, then the off-diagonal
// blocks, as the pages' pipeline does).
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr int C = kChunk;
#ifndef SWEEP_PF
#define SWEEP_PF 3
#endif
#ifndef SWEEP_NCT128
#define SWEEP_NCT128 2
#endif


__host__ __device__ constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t a16(size_t x) { return (x + 15) & ~(size_t)15; }

// Workspace matrices are stored in "fragment order": the data one wave's
// matrix-core operand load needs is contiguous. For a row-major R x K matrix
// read as A (or B^T) operand fragments, the fragment (row tile rt, K step ks)
// is one block of 64 lanes x FE elements (FE = KS / 4: 8 for bf16, 1 for
// fp32), lane l holding row 16 rt + l % 16, columns KS ks + FE (l / 16) ...
template <typename IO>
__device__ __forceinline__ size_t frag_slot(int rt, int ks, int K) {
    constexpr int KS = Mma<IO>::KS, FE = KS / 4;
    return ((size_t)(rt * (K / KS) + ks) * 64 + (threadIdx.x & 63)) * FE;
}
template <typename IO>
__device__ __forceinline__ typename Mma<IO>::Frag load_frag(const IO *M, int rt, int ks, int K) {
    return *reinterpret_cast<const typename Mma<IO>::Frag *>(M + frag_slot<IO>(rt, ks, K));
}
// NT: a non-temporal store, for workspaces far larger than the memory-side
// cache (the per-channel prefill's), which it would only churn; a smaller
// one (the Qwen-shaped layer's 161 MB) stays cached for the sweep.
template <typename IO, bool NT = false>
__device__ __forceinline__ void store_frag(IO *M, int rt, int ks, int K, typename Mma<IO>::Frag f) {
    auto *p = reinterpret_cast<typename Mma<IO>::Frag *>(M + frag_slot<IO>(rt, ks, K));
    if constexpr (NT) __builtin_nontemporal_store(f, p);
    else *p = f;
}
// Four consecutive values to a workspace in the io dtype, as store_frag.
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
template <bool NT>
__device__ __forceinline__ void store4_ws(float *p, f32x4 x) {
    if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
    else store4f(p, x);
}
template <bool NT>
__device__ __forceinline__ void store4_ws(bf16_t *p, f32x4 x) {
    const u32x2 v{f2bf2(x[0], x[1]), f2bf2(x[2], x[3])};
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
    else *reinterpret_cast<u32x2 *>(p) = v;
}
// ... and a token-contiguous D x C matrix read in accumulator layout (lane
// l = col % 16 + 16 (tok % 16) / 4 holds 4 consecutive tokens of one column)
// is stored as one block of 64 lanes x 4 elements per (token tile, column tile).
template <int D>
__device__ __forceinline__ size_t cfrag_off(int col, int tok) {
    const int lane = (col & 15) + 16 * ((tok & 15) >> 2);
    return ((size_t)((tok >> 4) * (D / 16) + (col >> 4)) * 64 + lane) * 4 + (tok & 3);
}

// The 10 lower-triangular 16 x 16 tiles of a 64 x 64 matrix.
__device__ __forceinline__ void lower_tile(int idx, int &ti, int &tj) {
    ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    tj = idx - ti * (ti + 1) / 2;
}

// exp(x) = 2^(x log2 e) on the hardware exp2 (v_exp_f32, ~1 ulp).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// Per-channel decay inside a chunk, referenced block by block so that no
// factor exceeds 1 (the pages' pipeline forms the 16-token diagonal blocks
// first, then the off-diagonal ones). For the 16-token block b of a chunk let
// B_b be its per-channel sum of g, R_b = B_0 + ... + B_{b-1} the sum before it
// (R_0 = 0, R_4 = G_end), and Gb_i = G_i - R_b the in-block inclusive prefix of
// token i in block b. The tiles hold
//   Q^ = q . exp(Gb),  E^ = e . exp(Gb),  K^ = k . exp(B_b - Gb)   (all <= |x|).
// For tokens i in block bi and j in block bj <= bi,
//   exp(G_i - G_j) = exp(Gb_i) . exp(R_bi - R_{bj+1}) . exp(B_bj - Gb_j),
// so a Gram tile is E^ (or Q^) rows times K^ rows with one per-channel factor
// exp(R_bi - R_{bj+1}) on the K^ operand: 1 for bj = bi - 1, <= 1 further
// below the diagonal, and exp(-B_bi) >= 1 on the diagonal, where the K^ rows
// are read from a tile already scaled by it (k . exp(-Gb), at most
// exp(kDiagRange)). A diagonal block whose decay exceeds kDiagRange on some
// channel is instead formed entry by entry, sum_c e_ic k_jc exp(Gb_ic - Gb_jc),
// so no factor can overflow or vanish at any decay. The chunk-referenced
// operands follow by factors <= 1:
//   Q~ = Q^ . exp(R_b),  E~ = E^ . exp(R_b),  Kend = K^ . exp(G_end - R_{b+1}).
// kDecRows rows of per-channel factors (written by the wave of the block
// whose sums give them):
//   0-3   exp(R_b)                      (Q~, E~ of block b)
//   4-6   exp(B_1), exp(B_2), exp(B_1 + B_2)   (Gram tiles (2,0), (3,1), (3,0))
//   7-10  exp(-B_b), capped at exp(kDiagRange)   (diagonal Gram tile of block b)
//   11-14 exp(G_end - R_{b+1})          (Kend of block b)
//   15    exp(G_end)                    (Kend of a mild chunk)
// With bfloat16 io, phase A writes the diagonal K operand, E~ and Kend as
// tiles of their own, so that no bfloat16 operand is unpacked and rescaled
// on the matrix-core path; with float32 io (whose tiles are twice as large)
// the operands are scaled as they are read, one multiply per element.
constexpr int kDecRows = 16;
constexpr float kDiagRange = 40.f;
// A chunk whose every 16-token block decays by less than kMildBlock on every
// channel keeps the chunk-referenced factors of the plain form (E~ and Q~ as
// above, K~ = k . exp(-G) <= exp(4 kMildBlock), Kend = K~ . exp(G_end)): the
// decays of ordinary layers stay far inside that range, and their chunks
// then need neither the block factors nor their extra tiles.
constexpr float kMildBlock = 15.f;
__host__ __device__ constexpr int dec_row_far(int bi, int bj) {  // factor row of Gram tile (bi, bj), bi - bj >= 2
    return bi == 2 ? 4 : bj == 1 ? 5 : 6;
}

// Orders this wave's shared-memory accesses around a point where lanes read
// what other lanes of the same wave wrote (a wave executes its LDS accesses
// in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Operands from shared memory in either orientation. Mma<IO>::load reads a
// fragment from storage where the operand's K index is contiguous. Km<IO>
// reads the same fragment from "K-major" storage, where element (row r, k)
// sits at M[k * ld + r]. For bfloat16 that is the gfx950 LDS transpose read
// ds_read_b64_tr_b16, whose lane layout (checked on the device) is: inside
// each group of 16 lanes, lane s supplies the address of 4 consecutive 16-bit
// elements, and lane j receives element j % 4 of the words supplied by lanes
// j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4, in that order. Lane s pointing
// at rows 4 (s % 4) .. 4 (s % 4) + 3 of K-row k0 + s / 4 therefore hands lane
// j row j of K-rows k0 .. k0 + 3.
__device__ __forceinline__ s16x4 ds_tr16(const bf16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

template <typename IO> struct Km;
template <> struct Km<bf16_t> {
    // 16 x 32 fragment (the operand of v_mfma_f32_16x16x32_bf16).
    __device__ __forceinline__ static u16x8 frag(const bf16_t *M, int ld) {
        const int l = lane_id(), s = l & 15, g = l >> 4;
        const bf16_t *p = M + (8 * g + (s >> 2)) * ld + 4 * (s & 3);
        const s16x4 lo = ds_tr16(p), hi = ds_tr16(p + 4 * ld);
        return __builtin_bit_cast(u16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // acc += A * Bt^T for 16 x 16 blocks: A K-major at A, Bt with K contiguous.
    __device__ __forceinline__ static f32x4 mma16(f32x4 acc, const bf16_t *A, int lda, const bf16_t *Bt, int ldb) {
        const int l = lane_id(), s = l & 15, g = l >> 4;
        const s16x4 av = ds_tr16(A + (4 * g + (s >> 2)) * lda + 4 * (s & 3));
        const s16x4 bv = *reinterpret_cast<const s16x4 *>(Bt + s * ldb + 4 * g);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
    }
    // Multiply the 8 elements of a fragment (8 consecutive K indices) by f[0..7].
    __device__ __forceinline__ static u16x8 scale(u16x8 x, const float *f) {
        const f32x4 f0 = load4f(f), f1 = load4f(f + 4);
        const u32x4 r = {f2bf2(bf2f(x[0]) * f0[0], bf2f(x[1]) * f0[1]), f2bf2(bf2f(x[2]) * f0[2], bf2f(x[3]) * f0[3]),
                         f2bf2(bf2f(x[4]) * f1[0], bf2f(x[5]) * f1[1]), f2bf2(bf2f(x[6]) * f1[2], bf2f(x[7]) * f1[3])};
        return __builtin_bit_cast(u16x8, r);
    }
    __device__ __forceinline__ static u16x8 scale(u16x8 x, float f) {
        const u32x4 r = {f2bf2(bf2f(x[0]) * f, bf2f(x[1]) * f), f2bf2(bf2f(x[2]) * f, bf2f(x[3]) * f),
                         f2bf2(bf2f(x[4]) * f, bf2f(x[5]) * f), f2bf2(bf2f(x[6]) * f, bf2f(x[7]) * f)};
        return __builtin_bit_cast(u16x8, r);
    }
};
template <> struct Km<float> {
    __device__ __forceinline__ static float frag(const float *M, int ld) {
        const int l = lane_id();
        return M[(l >> 4) * ld + (l & 15)];
    }
    __device__ __forceinline__ static f32x4 mma16(f32x4 acc, const float *A, int lda, const float *Bt, int ldb) {
        const int l = lane_id(), s = l & 15, g = l >> 4;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(4 * ks + g) * lda + s], Bt[s * ldb + 4 * ks + g], acc, 0, 0, 0);
        return acc;
    }
    __device__ __forceinline__ static float scale(float x, const float *f) { return x * f[0]; }
    __device__ __forceinline__ static float scale(float x, float f) { return x * f; }
};

// 16 bytes of stored elements (8 bf16 or 4 fp32) kept raw in registers, so a
// prefetch does not wait for its data; widened to float at use.
template <typename IO> struct Raw16;
template <> struct Raw16<bf16_t> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void widen(uint4 r, float *f) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return uint4{f2bf2(f[0], f[1]), f2bf2(f[2], f[3]), f2bf2(f[4], f[5]), f2bf2(f[6], f[7])};
    }
    __device__ __forceinline__ static float at(uint4 r, int i) {  // element i (i a constant after unrolling)
        const uint32_t w = i < 2 ? r.x : i < 4 ? r.y : i < 6 ? r.z : r.w;
        return __uint_as_float(i % 2 ? w & 0xffff0000u : w << 16);
    }
};
template <> struct Raw16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void widen(uint4 r, float *f) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y); f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
    __device__ __forceinline__ static float at(uint4 r, int i) {
        return __uint_as_float(i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w);
    }
};
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
// 16-byte store with a non-temporal hint, for outputs nothing here reads back.
__device__ __forceinline__ void st16_stream(void *p, uint4 x) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x), reinterpret_cast<u32x4 *>(p));
}

// ---------------------------------------------------------------------------
// chunk_prep: everything in a chunk that does not depend on the state, for
// every (sequence, V head, chunk) unit; persistent over units, with the next
// unit's inputs prefetched into registers while the current one is processed.
//
// Shared memory holds the chunk's token-major tiles (row t = token, 16-byte
// channel groups): q, k and z = gated v; for decoupled gates or per-channel
// decay also the erase key; for per-channel decay the tiles carry the decay
// referenced to their 16-token block (Q^, K^, E^ above), and the per-channel
// factors between blocks are applied where the tiles are read. With a scalar
// decay the tiles stay undecayed and the decay is applied where they are
// read: to Gram entries as exp(G_i - G_j) (no factor can overflow), and per
// token to the E~ and Kend operands.
//  A. prefix sums of g, token tables, the tiles; gamma.
//  B. Gram products T = E~ K~^T, A = Q~ K~^T on the matrix cores (20 lower
//     16 x 16 tiles); T and A kept column-major; Q~ and Kend^T go to the
//     workspace straight from the tiles.
//  C. A to the workspace; L = (I + T)^-1: the 16 x 16 diagonal blocks by fp32
//     substitution, then column block j by block forward substitution,
//     X_i = -D_i sum_{j <= k < i} T_ik X_k, one wave per column block.
//  D. [Y | U_z] = L [E~ | Z] on the matrix cores, each wave a slice of the
//     2 d columns; U_z^T goes to the workspace from the accumulators, Y
//     through a column-major staging tile.
//  E. Y to the workspace.
template <typename IO, int D>
struct PrepCfg {
    static constexpr int NW = 4, NT = 64 * NW;
    static constexpr int V = 16 / sizeof(IO);  // elements per 16-byte access
    static constexpr int CO = D / V;           // 16-byte channel groups per token row
    static constexpr int NGRP = NT / CO;       // token groups in phase A
    static constexpr int TPT = C / NGRP;       // tokens per thread in phase A
    static constexpr int KS = Mma<IO>::KS;
    static constexpr int PD = D + V;           // token-major tile row stride
    static constexpr int LC = C + V;           // column-major 64 x 64 stride (T, A, L)
    static constexpr int LY = C + V;           // column-major Y staging stride
    static constexpr int LT = 16 + V;          // per-wave 16 x 16 temporary stride
    static constexpr int WC = 2 * D / NW;      // columns of [E~ | Z] per wave in phase D
    static constexpr int NCTS = WC / 16;
    static constexpr size_t TILE = a16((size_t)C * PD * sizeof(IO));
    static constexpr size_t R1 = a16(cmax((size_t)C * PD, (size_t)D * LY) * sizeof(IO));
    static constexpr size_t MAT = a16((size_t)C * LC * sizeof(IO));
    static constexpr size_t TMP = a16((size_t)NW * 16 * LT * sizeof(IO));
    static constexpr size_t TD = a16((size_t)4 * 16 * 17 * 4);
    static constexpr size_t TAB = a16((size_t)5 * C * 4);
    static constexpr size_t PART = a16((size_t)NGRP * D * 4);
    static constexpr size_t DEC = a16((size_t)kDecRows * D * 4) + 32;  // decay factor rows + 4 block flags
    static_assert(NT % CO == 0 && NGRP * TPT == C && WC % 16 == 0, "phase mappings");
    // Phase A: each wave holds the tokens of one 16-token block.
    static_assert(TPT * (64 / CO) == 16 && C / 16 == NW, "one 16-token block per wave in phase A");
    static_assert(PART <= MAT, "the per-group sums share the T tile's space");
    // Per-channel decay: the diagonal K operand, E~ and Kend as tiles (bfloat16 io only).
    static constexpr bool DTILES = sizeof(IO) == 2;
    static constexpr size_t bytes(bool has_e, bool chan) {
        return R1 + TILE * (2 + (has_e ? 1 : 0) + (chan && DTILES ? 3 : 0)) + 2 * MAT + TMP + TD + TAB + (chan ? DEC : 0);
    }
};

// Input stage (raw projections in): q and k are normalised as
// x / sqrt(sum x^2 + kStageNormEps); the gates are logistic functions of
// their inputs, and the decay is g = -c softplus(x).
constexpr float kStageNormEps = 1e-12f;
__device__ __forceinline__ float sigmoidf(float x) { return act_sigmoid(x); }
template <bool RAW>
__device__ __forceinline__ float stage_decay(float x, float c) {
    if constexpr (RAW) return -c * act_softplus(x);
    else return x;
}

// One thread's raw inputs for a chunk: TPT tokens x one 16-byte channel group
// of q, k, v (and b, w, per-channel g); lane l of wave 0 also holds token l's
// beta and scalar g.
template <typename IO, int D, bool CHAN, bool BW, bool RAW>
struct PrepIn {
    using Cfg = PrepCfg<IO, D>;
    static constexpr int TPT = Cfg::TPT, V = Cfg::V;
    uint4 q[TPT], k[TPT], v[TPT], bg[BW ? TPT : 1], wg[BW ? TPT : 1];
    f32x4 g[CHAN ? TPT * V / 4 : 1];
    float betal, gs;
    // Input stage: token c*C - 3 + grp of the raw q, k, v (groups 0-2), the
    // chunk's convolution window before its first token.
    uint4 halo_q, halo_k, halo_v;

    // The loads are issued in three parts (PART 0: q, k; 1: v, per-channel g;
    // 2: b, w, beta, scalar g) at different points of the previous unit, so
    // the memory queue drains behind computation instead of stalling a burst.
    // qk false: q and k are already in registers (the same QK head's chunk),
    // so the convolution window of neither is fetched.
    template <int PART>
    __device__ __forceinline__ void load(const ChunkArgs &a, int u, int co, int grp, bool qk = true) {
        const int NC = a.NC, c = u % NC, bh = u / NC, b = bh / a.Hv, h = bh - b * a.Hv;
        const int hq = h / (a.Hv / a.Hqk), t0 = c * C, n = min(C, a.T - t0);
        const int l = threadIdx.x & 63;
        const size_t row0 = (size_t)b * a.T + t0;  // first token row of the chunk
        const size_t qko = (row0 * a.Hqk + hq) * D + V * co;
        const size_t vo = (row0 * a.Hv + h) * D + V * co;
        const size_t sqk = (size_t)a.Hqk * D, sv = (size_t)a.Hv * D;  // token strides (elements)
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const int t = min(TPT * grp + j, n - 1);  // clamped: padded tokens are zeroed at use
            if constexpr (PART == 0) {
                q[j] = ld16(static_cast<const IO *>(a.q) + qko + t * sqk);
                k[j] = ld16(static_cast<const IO *>(a.k) + qko + t * sqk);
            }
            if constexpr (PART == 1) {
                v[j] = ld16(static_cast<const IO *>(a.v) + vo + t * sv);
                if constexpr (CHAN)
#pragma unroll
                    for (int i = 0; i < V / 4; ++i) g[j * (V / 4) + i] = load4f(a.g + vo + t * sv + 4 * i);
            }
            if constexpr (PART == 2 && BW) {
                bg[j] = ld16(static_cast<const IO *>(a.bg) + vo + t * sv);
                wg[j] = ld16(static_cast<const IO *>(a.wg) + vo + t * sv);
            }
        }
        if constexpr (RAW && PART == 2)  // late: short live range for the window registers
            if (grp < 3) {
                const int th = t0 - 3 + grp;  // < 0: from the incoming convolution state (zeros without one)
                const size_t ch = 2 * sqk + sv;
                const IO *cin = th < 0 && a.conv_in ? static_cast<const IO *>(a.conv_in) + ((size_t)b * 3 + 3 + th) * ch
                                                    : nullptr;
                const uint4 zero = uint4{0u, 0u, 0u, 0u};
                const size_t cq = (size_t)hq * D + V * co;
                if (qk) {
                    halo_q = th >= 0 ? ld16(static_cast<const IO *>(a.q) + qko + (ptrdiff_t)(th - t0) * (ptrdiff_t)sqk)
                                     : cin ? ld16(cin + cq) : zero;
                    halo_k = th >= 0 ? ld16(static_cast<const IO *>(a.k) + qko + (ptrdiff_t)(th - t0) * (ptrdiff_t)sqk)
                                     : cin ? ld16(cin + sqk + cq) : zero;
                }
                halo_v = th >= 0 ? ld16(static_cast<const IO *>(a.v) + vo + (ptrdiff_t)(th - t0) * (ptrdiff_t)sv)
                                 : cin ? ld16(cin + 2 * sqk + (size_t)h * D + V * co) : zero;
            }
        if constexpr (PART == 2)
            if (threadIdx.x < 64) {  // wave 0: one token per lane
                const size_t tl = (row0 + min(l, n - 1)) * a.Hv + h;
                if constexpr (!BW) betal = a.beta[tl];
                if constexpr (!CHAN) gs = a.decay == DECAY_SCALAR ? a.g[tl] : 0.f;
            }
    }
    __device__ __forceinline__ void load_all(const ChunkArgs &a, int u, int co, int grp) {
        load<0>(a, u, co, grp);
        load<1>(a, u, co, grp);
        load<2>(a, u, co, grp);
    }
};

// Workgroups per CU the prep is compiled for: two where two fit in shared
// memory and the variant keeps few tiles, else one (which lets the compiler
// use the whole register file).
template <typename IO, int D, bool CHAN, bool BW>
constexpr int prep_occupancy() {
    return (CHAN || BW || 2 * PrepCfg<IO, D>::bytes(false, false) > (size_t)160 * 1024) ? 1 : 2;
}

template <typename IO, int D, bool CHAN, bool BW, bool RAW>
__global__ __launch_bounds__(256, (prep_occupancy<IO, D, CHAN, BW>())) void chunk_prep(ChunkArgs a) {
    using M = Mma<IO>;
    using K = Km<IO>;
    using R = Raw16<IO>;
    using Frag = typename M::Frag;
    using Cfg = PrepCfg<IO, D>;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, V = Cfg::V, CO = Cfg::CO, NGRP = Cfg::NGRP, TPT = Cfg::TPT;
    constexpr int KS = M::KS, FE = KS / 4, PD = Cfg::PD, LC = Cfg::LC, LY = Cfg::LY, LT = Cfg::LT;
    constexpr int WC = Cfg::WC, NCTS = Cfg::NCTS;
    constexpr bool HAS_E = CHAN || BW;
    // RAW: the gates and the decay arrive before their activations. Without a
    // per-channel decay q, k and v arrive raw as well, and the whole input
    // stage runs here; with one, the convolution and the normalisation of q,
    // k and v ran as a pass of their own before this kernel.
    constexpr bool RQKV = RAW && !CHAN;
    static_assert(NT == 256, "launch bounds");

    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char *sp = smem;
    IO *tQ = reinterpret_cast<IO *>(sp);  sp += Cfg::R1;    // q (Q~), token-major; later Y staging [D][LY]
    IO *tK = reinterpret_cast<IO *>(sp);  sp += Cfg::TILE;  // k (K~)
    IO *tZ = reinterpret_cast<IO *>(sp);  sp += Cfg::TILE;  // z
    IO *tE = reinterpret_cast<IO *>(sp);  sp += HAS_E ? Cfg::TILE : 0;  // erase key (E~)
    constexpr bool DT = CHAN && Cfg::DTILES;
    IO *tKd = reinterpret_cast<IO *>(sp); sp += DT ? Cfg::TILE : 0;     // per-channel decay: k . exp(-Gb)
    IO *tEt = reinterpret_cast<IO *>(sp); sp += DT ? Cfg::TILE : 0;     //   E~ (chunk-referenced)
    IO *tKe = reinterpret_cast<IO *>(sp); sp += DT ? Cfg::TILE : 0;     //   Kend
    IO *sTc = reinterpret_cast<IO *>(sp); sp += Cfg::MAT;   // T(i, j) at sTc[j * LC + i], blocks below the diagonal
    IO *sAc = reinterpret_cast<IO *>(sp); sp += Cfg::MAT;   // A, same layout; then L
    IO *sLc = sAc;
    IO *sTmp = reinterpret_cast<IO *>(sp); sp += Cfg::TMP;  // per-wave 16 x 16 temporaries
    float *sTd = reinterpret_cast<float *>(sp); sp += Cfg::TD;  // T's diagonal blocks, fp32, [blk][col][17]
    float *sG = reinterpret_cast<float *>(sp); sp += Cfg::TAB;  // per token: G,
    float *sEG = sG + C;                                          //   exp(G),
    float *sBt = sG + 3 * C;                                      //   beta,
    float *sSE = sG + 4 * C;                                      //   the E~ factor of a raw erase-key tile
    float *sBlk = reinterpret_cast<float *>(sTmp);                // [4][D] block sums of g (phase A only)
    float *sPart = reinterpret_cast<float *>(sTc);                // [NGRP][D] token-group sums of g (phase A only)
    float *sDec = reinterpret_cast<float *>(sp);                  // [kDecRows][D] per-channel decay factors
    int *sSlow = reinterpret_cast<int *>(sDec + kDecRows * D);    // [4]: diagonal block formed entry by entry
    IO *sYc = tQ;                                                 // Y(t, c) at sYc[c * LY + t]

    // The wave index is uniform across the wave: keep it in a scalar register
    // so that per-wave choices below are scalar branches, not masked ones.
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lr = l & 15,
              lg = l >> 4;
    const int co = tid % CO, grp = tid / CO;
    // With the input stage, a scalar decay and tied gates, a work item is a
    // (sequence, chunk) and PG consecutive V heads of one QK head, run one
    // after another: q and k are loaded, convolved and normalised once and
    // stay in registers for the later heads. Otherwise a work item is one
    // unit: without the input stage the shared q and k would only save
    // loads, and the register-bound per-channel and decoupled-gate variants
    // measured slower with the grouped loop.
    constexpr bool GROUPED = RAW && !CHAN && !BW;
    const int grpsz = a.Hv / a.Hqk, PG = GROUPED ? a.prep_grp : 1, HG = a.Hv / PG, gunits = a.B * HG * a.NC;
    const auto unit_of = [&](int gu, int hh) {
        if constexpr (!GROUPED) return gu;
        const int c = gu % a.NC, bq = gu / a.NC, b = bq / HG, hg = bq - b * HG;
        return (b * a.Hv + hg * PG + hh) * a.NC + c;
    };

    PrepIn<IO, D, CHAN, BW, RQKV> in;
    if ((int)blockIdx.x < gunits) in.load_all(a, unit_of(blockIdx.x, 0), co, grp);

    for (int gu = blockIdx.x, hh = 0; gu < gunits;) {
        const int u = unit_of(gu, hh);
        const bool first = !GROUPED || hh == 0;  // q and k are not yet formed for this work item
        // The next unit: the item's next V head, else the next item's first.
        const int gun = gu + (int)gridDim.x;
        const bool next_same = GROUPED && hh + 1 < PG;
        const bool has_next = next_same || gun < gunits;
        const int un = next_same ? unit_of(gu, hh + 1) : unit_of(gun, 0);
        const int NC = a.NC, c = u % NC, bh = u / NC, h = bh % a.Hv;
        const int n = min(C, a.T - c * C);
        IO *ws = static_cast<IO *>(a.ws_io) + (size_t)u * chunk_ws_io_elems(D, CHAN);
        IO *wY = ws, *wQ = ws + C * D, *wUzT = ws + ws_off_uz(D, CHAN), *wA = ws + ws_off_a(D, CHAN);
        // Kend^T per unit (per-channel decay), or k^T once per QK head, written by its first V head.
        IO *wKT = CHAN ? ws + 2 * C * D
                       : static_cast<IO *>(a.ws_kT) + ((size_t)(bh / a.Hv * a.Hqk + h / grpsz) * NC + c) * (2 * D * C);
        IO *wQh = wKT + D * C;
        const bool write_kT = CHAN || h % grpsz == 0;
        float *tab = a.ws_tab + (size_t)u * kTab;
        // Input stage: g holds the decay's input x, g = -dsc softplus(x).
        const float dsc = RAW && a.decay_scale ? a.decay_scale[h] : 1.f;
        __syncthreads();  // the previous unit is done with shared memory

        // ---- A. prefix sums, token tables, tiles ----
        // Input stage: this thread's convolution taps (q, k and v channels).
        // The one-workgroup-per-CU variants have the registers to request
        // them first, so that their latency hides behind phase A; the others
        // load each tensor's taps where they are used.
        constexpr bool EARLY_TAPS = RQKV && prep_occupancy<IO, D, CHAN, BW>() == 1;
        f32x4 taps[EARLY_TAPS ? 3 * V : 1];
        if constexpr (EARLY_TAPS) {
            const size_t sqk = (size_t)a.Hqk * D;
            const size_t cq = (size_t)(h / grpsz) * D + V * co;
            const size_t cb[3] = {cq, sqk + cq, 2 * sqk + (size_t)h * D + V * co};
#pragma unroll
            for (int x = 0; x < 3; ++x)
                if (x == 2 || first)
#pragma unroll
                    for (int c4 = 0; c4 < V; ++c4) taps[x * V + c4] = load4f(a.conv_w + (cb[x] + c4) * 4);
        }
        float G[CHAN ? TPT : 1][V];
        float Bmy[CHAN ? V : 1];  // per-channel decay sum of this thread's 16-token block (the wave's block)
        if constexpr (CHAN) {
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int ch = 0; ch < V; ++ch)
                    G[j][ch] = (TPT * grp + j < n ? stage_decay<RAW>(in.g[j * (V / 4) + ch / 4][ch % 4], dsc) : 0.f) +
                               (j > 0 ? G[j - 1][ch] : 0.f);
            // The wave holds one 16-token block: its groups' totals, exchanged
            // through shared memory inside the wave, give the offset that turns
            // each local prefix into the in-block prefix Gb and the block's sum
            // B, which goes to sBlk for the other waves.
#pragma unroll
            for (int i = 0; i < V / 4; ++i)
                store4f(sPart + grp * D + V * co + 4 * i,
                        f32x4{G[TPT - 1][4 * i], G[TPT - 1][4 * i + 1], G[TPT - 1][4 * i + 2], G[TPT - 1][4 * i + 3]});
            wave_sync();
            constexpr int GPB = NGRP / 4;
            float Bw[V], off[V];
#pragma unroll
            for (int ch = 0; ch < V; ++ch) Bw[ch] = off[ch] = 0.f;
#pragma unroll
            for (int gg = 0; gg < GPB; ++gg)
#pragma unroll
                for (int i = 0; i < V / 4; ++i) {
                    const f32x4 p = load4f(sPart + (w * GPB + gg) * D + V * co + 4 * i);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Bw[4 * i + r] += p[r];
                        if (w * GPB + gg < grp) off[4 * i + r] += p[r];
                    }
                }
#pragma unroll
            for (int ch = 0; ch < V; ++ch)
#pragma unroll
                for (int j = 0; j < TPT; ++j) G[j][ch] += off[ch];
            if (l < CO)
#pragma unroll
                for (int i = 0; i < V / 4; ++i)
                    store4f(sBlk + w * D + V * co + 4 * i, f32x4{Bw[4 * i], Bw[4 * i + 1], Bw[4 * i + 2], Bw[4 * i + 3]});
#pragma unroll
            for (int ch = 0; ch < V; ++ch) Bmy[ch] = Bw[ch];
        }
        if (w == 0) {
            float eg = 1.f;
            if constexpr (!CHAN) {
                // Scalar decay: lane = token; inclusive scan of g over the chunk.
                float Gl = l < n && a.decay == DECAY_SCALAR ? stage_decay<RAW>(in.gs, dsc) : 0.f;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(Gl, off);
                    if (l >= off) Gl += y;
                }
                eg = fast_exp(Gl);
                const float er = fast_exp(__shfl(Gl, 63) - Gl);
                sG[l] = Gl;
                sEG[l] = eg;
                tab[l] = eg;       // per-token decay factors for the sweep
                tab[C + l] = er;
            }
            const float bt = BW ? 0.f : RAW ? sigmoidf(in.betal) : in.betal;
            if constexpr (!BW) sBt[l] = bt;
            sSE[l] = BW ? eg : bt * eg;
        }
        IO *sHalo = sTmp;  // input stage: [3 tokens][q, k, v][D], the window before the chunk
        if constexpr (RQKV) {
            // The raw rows go to the tiles (token-major, as the processed
            // ones will) and the 3 tokens before the chunk to sHalo, so that
            // each thread can read the 3 rows before its own.
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int o = (TPT * grp + j) * PD + V * co;
                if (first) {
                    *reinterpret_cast<uint4 *>(tQ + o) = in.q[j];
                    *reinterpret_cast<uint4 *>(tK + o) = in.k[j];
                }
                *reinterpret_cast<uint4 *>(tZ + o) = in.v[j];
            }
            if (grp < 3) {
                if (first) {
                    *reinterpret_cast<uint4 *>(sHalo + (3 * grp + 0) * D + V * co) = in.halo_q;
                    *reinterpret_cast<uint4 *>(sHalo + (3 * grp + 1) * D + V * co) = in.halo_k;
                }
                *reinterpret_cast<uint4 *>(sHalo + (3 * grp + 2) * D + V * co) = in.halo_v;
            }
        }
        __syncthreads();
        if constexpr (RQKV) {
            const size_t sqk = (size_t)a.Hqk * D, ch = 2 * sqk + (size_t)a.Hv * D;
            const int hq = h / grpsz, b = bh / a.Hv;
            const size_t cq = (size_t)hq * D + V * co, ck = sqk + cq, cv = 2 * sqk + (size_t)h * D + V * co;
            // Raw row of token t of this chunk (t >= -3) for tensor x (0 q, 1 k, 2 v).
            const auto raw_row = [&](int x, int t) -> uint4 {
                const IO *tile = x == 0 ? tQ : x == 1 ? tK : tZ;
                return t >= 0 ? *reinterpret_cast<const uint4 *>(tile + t * PD + V * co)
                              : *reinterpret_cast<const uint4 *>(sHalo + (3 * (3 + t) + x) * D + V * co);
            };
            // The convolution state after the last chunk: its last 3 raw tokens.
            if (a.conv_out && c == NC - 1 && grp < 3) {
                IO *cout = static_cast<IO *>(a.conv_out) + ((size_t)b * 3 + grp) * ch;
                const int t = n - 3 + grp;
                if (h % grpsz == 0) {
                    *reinterpret_cast<uint4 *>(cout + cq) = raw_row(0, t);
                    *reinterpret_cast<uint4 *>(cout + ck) = raw_row(1, t);
                }
                *reinterpret_cast<uint4 *>(cout + cv) = raw_row(2, t);
            }
            // Convolve this thread's tokens (window: 3 rows before them, then
            // their own), normalise q and k over the head, and keep the
            // results in place of the raw rows.
            const auto stage = [&](uint4(&x)[TPT], int xi, size_t cbase, bool norm) {
                uint4 wnd[TPT + 3];  // raw, widened one channel at a time
                float out[TPT][V];
#pragma unroll
                for (int r = 0; r < 3; ++r) wnd[r] = raw_row(xi, TPT * grp - 3 + r);
#pragma unroll
                for (int j = 0; j < TPT; ++j) wnd[3 + j] = x[j];
#pragma unroll
                for (int c4 = 0; c4 < V; ++c4) {
                    f32x4 tp;
                    if constexpr (EARLY_TAPS) tp = taps[xi * V + c4];
                    else tp = load4f(a.conv_w + (cbase + c4) * 4);
                    float xc[TPT + 3];
#pragma unroll
                    for (int r = 0; r < TPT + 3; ++r) xc[r] = R::at(wnd[r], c4);
#pragma unroll
                    for (int j = 0; j < TPT; ++j)
                        out[j][c4] = tp[0] * xc[j] + tp[1] * xc[j + 1] + tp[2] * xc[j + 2] + tp[3] * xc[j + 3];
                }
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    if (norm) {
                        float ss = 0.f;
#pragma unroll
                        for (int c4 = 0; c4 < V; ++c4) ss += out[j][c4] * out[j][c4];
                        ss = lanes_allreduce<CO>(ss);
                        const float f = 1.f / sqrtf(ss + kStageNormEps);
#pragma unroll
                        for (int c4 = 0; c4 < V; ++c4) out[j][c4] *= f;
                    }
                    x[j] = R::pack(out[j]);
                }
            };
            if (first) {
                stage(in.q, 0, cq, true);
                stage(in.k, 1, ck, true);
            }
            stage(in.v, 2, cv, false);
            __syncthreads();  // every window read before the tiles are overwritten
        }
        // exp(B), exp(R) and exp(G_end - R_{b+1}) of that block; exp(G_end)
        float eB[CHAN ? V : 1], eR[CHAN ? V : 1], eG1[CHAN ? V : 1], eGe[CHAN ? V : 1];
        bool mild = true;  // the chunk keeps the chunk-referenced factors (uniform over the workgroup)
        if constexpr (CHAN) {
            // Sums over the blocks before this thread's block (R_b), its block
            // (B_b), the blocks after it (G_end - R_{b+1}) and the block just
            // before it; the wave's block is b = w, uniform over the wave.
            // Every wave reads all four block sums of every channel, so the
            // mild test (a ballot over them) agrees across the workgroup. The
            // block index is taken per lane (grp / GPB, equal to w) so that
            // the selects below stay branch-free.
            constexpr int GPB = NGRP / 4;
            const int myb = grp / GPB;
            float Rb[V], Pv[V], Af[V];
            bool steep = false;
#pragma unroll
            for (int ch = 0; ch < V; ++ch) Rb[ch] = Pv[ch] = Af[ch] = 0.f;
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2)
#pragma unroll
                for (int i = 0; i < V / 4; ++i) {
                    const f32x4 p = load4f(sBlk + b2 * D + V * co + 4 * i);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = p[r];
                        steep = steep || x <= -kMildBlock;
                        Rb[4 * i + r] += b2 < myb ? x : 0.f;
                        Af[4 * i + r] += b2 > myb ? x : 0.f;
                        Pv[4 * i + r] = b2 == myb - 1 ? x : Pv[4 * i + r];
                    }
                }
            mild = __ballot(steep) == 0;
#pragma unroll
            for (int ch = 0; ch < V; ++ch) {
                eR[ch] = fast_exp(Rb[ch]);
                eGe[ch] = fast_exp(Rb[ch] + Bmy[ch] + Af[ch]);
            }
            if (!mild)
#pragma unroll
                for (int ch = 0; ch < V; ++ch) {
                    eB[ch] = fast_exp(Bmy[ch]);
                    eG1[ch] = fast_exp(Af[ch]);
                }
            // The decay factor table: the first group of each wave writes the
            // rows its block's sums give.
            const auto put_row = [&](int row, const float(&f)[V]) {
#pragma unroll
                for (int i = 0; i < V / 4; ++i)
                    store4f(sDec + row * D + V * co + 4 * i, f32x4{f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]});
            };
            if (!Cfg::DTILES && w == 3 && l < CO) put_row(15, eGe);  // exp(G_end)
            if (!mild && l < CO) {
                put_row(w, eR);                                  // exp(R_b)
                if (w == 1 || w == 2) put_row(3 + w, eB);        // exp(B_1), exp(B_2)
                if (w == 2) {                                    // exp(B_1 + B_2)
                    float f[V];
#pragma unroll
                    for (int ch = 0; ch < V; ++ch) f[ch] = fast_exp(Pv[ch] + Bmy[ch]);
                    put_row(6, f);
                }
                if constexpr (!Cfg::DTILES) {
                    float f[V];
#pragma unroll
                    for (int ch = 0; ch < V; ++ch) f[ch] = fast_exp(fminf(-Bmy[ch], kDiagRange));
                    put_row(7 + w, f);                           // exp(-B_b)
                    put_row(11 + w, eG1);                        // exp(G_end - R_{b+1})
                }
            }
            if (grp == NGRP - 1)  // gamma per channel for the sweep
#pragma unroll
                for (int i = 0; i < V / 4; ++i)
                    store4f(tab + V * co + 4 * i, f32x4{eGe[4 * i], eGe[4 * i + 1], eGe[4 * i + 2], eGe[4 * i + 3]});
        }
        // Per-channel decay: a block whose decay exceeds kDiagRange on some
        // channel ("slow"; the flag is uniform over the wave that holds it)
        // keeps its raw q, k and e in the tiles until its diagonal Gram tiles
        // have been formed entry by entry below; every other block's diagonal
        // tiles read k . exp(-Gb) = K^ . exp(-B).
        bool slow = false;
        if constexpr (CHAN) {
            bool big = false;
#pragma unroll
            for (int ch = 0; ch < V; ++ch) big = big || Bmy[ch] < -kDiagRange;
            slow = __ballot(big) != 0;
            if (l == 0) sSlow[w] = slow ? 1 : 0;
        }
        // The tiles: mode 0 a mild chunk (chunk-referenced factors), 1 the
        // block-referenced factors, 2 a slow block (raw q, k and e).
        const auto write_tiles = [&](auto mode_c) {
            constexpr int MODE = decltype(mode_c)::value;
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const int t = TPT * grp + j;
            const bool valid = t < n;
            float qq[V], kk[V], vv[V], eb[V], wz[V];
            R::widen(in.q[j], qq);
            R::widen(in.k[j], kk);
            R::widen(in.v[j], vv);
            if constexpr (BW) {
                R::widen(in.bg[j], eb);
                R::widen(in.wg[j], wz);
                if constexpr (RAW)
#pragma unroll
                    for (int ch = 0; ch < V; ++ch) {
                        eb[ch] = sigmoidf(eb[ch]);
                        wz[ch] = sigmoidf(wz[ch]);
                    }
            } else {
                const float bt = sBt[t];
#pragma unroll
                for (int ch = 0; ch < V; ++ch) eb[ch] = wz[ch] = bt;
            }
            float oq[V], ok[V], oz[V], oe[V], okd[CHAN ? V : 1], oet[CHAN ? V : 1], oke[CHAN ? V : 1];
#pragma unroll
            for (int ch = 0; ch < V; ++ch) {
                const float kv = valid ? kk[ch] : 0.f, qv = valid ? qq[ch] : 0.f;
                oz[ch] = valid ? wz[ch] * vv[ch] : 0.f;
                if constexpr (CHAN) {
                    // Q^, E^ and K^ of the in-block prefix Gb, every factor <= 1
                    // (raw values in a slow block, scaled once its diagonal is
                    // formed); k . exp(-Gb) for the diagonal tiles, at most
                    // exp(kDiagRange) outside slow blocks; E~ = E^ . exp(R) and
                    // Kend = K^ . exp(G_end - R_{b+1}) (a slow block's Kend
                    // is written once its K^ is).
                    const float egt = fast_exp(G[j][ch]), ev = eb[ch] * kv;
                    if constexpr (MODE == 0) {
                        const float eg = egt * eR[ch], emg = __builtin_amdgcn_rcpf(eg);
                        oq[ch] = qv * eg;
                        ok[ch] = okd[ch] = kv * emg;
                        oe[ch] = oet[ch] = ev * eg;
                        oke[ch] = ok[ch] * eGe[ch];
                    } else if constexpr (MODE == 2) {
                        oq[ch] = qv;
                        ok[ch] = okd[ch] = oke[ch] = kv;
                        oe[ch] = ev;
                        oet[ch] = ev * egt * eR[ch];
                    } else {
                        okd[ch] = kv * __builtin_amdgcn_rcpf(egt);
                        ok[ch] = okd[ch] * eB[ch];
                        oke[ch] = ok[ch] * eG1[ch];
                        oq[ch] = qv * egt;
                        oe[ch] = ev * egt;
                        oet[ch] = oe[ch] * eR[ch];
                    }
                } else {
                    oq[ch] = qv;
                    ok[ch] = kv;
                    oe[ch] = eb[ch] * kv;
                }
            }
            const int o = t * PD + V * co;
            *reinterpret_cast<uint4 *>(tQ + o) = R::pack(oq);
            *reinterpret_cast<uint4 *>(tK + o) = R::pack(ok);
            *reinterpret_cast<uint4 *>(tZ + o) = R::pack(oz);
            if constexpr (HAS_E) *reinterpret_cast<uint4 *>(tE + o) = R::pack(oe);
            if constexpr (DT) {
                if constexpr (MODE != 0) {
                    *reinterpret_cast<uint4 *>(tKd + o) = R::pack(okd);
                    *reinterpret_cast<uint4 *>(tEt + o) = R::pack(oet);
                }
                *reinterpret_cast<uint4 *>(tKe + o) = R::pack(oke);
            }
        }
        };
        if constexpr (CHAN) {
            if (mild) write_tiles(std::integral_constant<int, 0>{});
            else if (slow) write_tiles(std::integral_constant<int, 2>{});
            else write_tiles(std::integral_constant<int, 1>{});
        } else {
            write_tiles(std::integral_constant<int, 0>{});
        }
        if constexpr (CHAN) {
            if (slow) {
                // The block's diagonal Gram tiles entry by entry,
                //   T_ij = sum_c e_ic k_jc exp(Gb_ic - Gb_jc) (j < i), A_ij likewise with q (j <= i),
                // from the raw rows of the tiles. Each lane sums its channel
                // group over the pairs (own token i, token j of the block); the
                // prefix Gb_j of its channel group comes from the lane holding
                // token j, and the partial sums are added over the channel groups.
                constexpr int GPB = NGRP / 4;
                const int gi = grp - w * GPB;
                wave_sync();  // the wave's raw rows are in the tiles
#pragma unroll
                for (int ii = 0; ii < TPT; ++ii) {
                    const int ti = TPT * grp + ii;
                    float qq[V], ee[V];
                    R::widen(*reinterpret_cast<const uint4 *>(tQ + ti * PD + V * co), qq);
                    R::widen(*reinterpret_cast<const uint4 *>(tE + ti * PD + V * co), ee);
#pragma unroll 1
                    for (int sg = 0; sg < GPB; ++sg) {
                        const int src = sg * CO + co;
#pragma unroll
                        for (int jj = 0; jj < TPT; ++jj) {
                            float kk[V];
                            R::widen(*reinterpret_cast<const uint4 *>(tK + (16 * w + TPT * sg + jj) * PD + V * co), kk);
                            float pt = 0.f, pa = 0.f;
#pragma unroll
                            for (int ch = 0; ch < V; ++ch) {
                                const float kf = kk[ch] * fast_exp(fminf(G[ii][ch] - __shfl(G[jj][ch], src), 0.f));
                                pt += ee[ch] * kf;
                                pa += qq[ch] * kf;
                            }
                            pt = lanes_allreduce<CO>(pt);
                            pa = lanes_allreduce<CO>(pa);
                            const int il = TPT * gi + ii, jl = TPT * sg + jj;
                            if ((ii * TPT + jj) % CO == co) {
                                sTd[(w * 16 + jl) * 17 + il] = jl < il ? pt : 0.f;
                                sAc[(16 * w + jl) * LC + 16 * w + il] = Elem<IO>::to(jl <= il ? pa : 0.f);
                            }
                        }
                    }
                }
                wave_sync();  // every raw row read: scale this thread's rows to Q^, K^, E^
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    const int o = (TPT * grp + j) * PD + V * co;
                    float qq[V], kk[V], ee[V];
                    R::widen(*reinterpret_cast<const uint4 *>(tQ + o), qq);
                    R::widen(*reinterpret_cast<const uint4 *>(tK + o), kk);
                    R::widen(*reinterpret_cast<const uint4 *>(tE + o), ee);
                    float ke[V];
#pragma unroll
                    for (int ch = 0; ch < V; ++ch) {
                        const float eg = fast_exp(G[j][ch]), ek = fast_exp(fminf(Bmy[ch] - G[j][ch], 0.f));
                        qq[ch] *= eg;
                        ee[ch] *= eg;
                        kk[ch] *= ek;
                        ke[ch] = kk[ch] * eG1[ch];
                    }
                    *reinterpret_cast<uint4 *>(tQ + o) = R::pack(qq);
                    *reinterpret_cast<uint4 *>(tK + o) = R::pack(kk);
                    *reinterpret_cast<uint4 *>(tE + o) = R::pack(ee);
                    if constexpr (DT) *reinterpret_cast<uint4 *>(tKe + o) = R::pack(ke);
                }
            }
        }
        // The raw inputs are consumed: start fetching the next unit's.
        if (has_next && !next_same) in.template load<0>(a, un, co, grp);
        __syncthreads();

        // ---- B. Gram products: 20 lower 16 x 16 tiles, 10 of T and 10 of A ----
        // (Instantiated apart for mild chunks, which need no factor table.)
        const auto gram = [&](auto mild_c) {
            constexpr bool MILD = decltype(mild_c)::value;
            const IO *TL = HAS_E ? tE : tK;  // left factor of T (raw k times beta for tied gates)
            constexpr int KD = D / KS;
            f32x4 x[5];
#pragma unroll
            for (int s = 0; s < 5; ++s) {
                const int p = w + NW * s, kind = p / 10;
                int ti, tj;
                lower_tile(p - kind * 10, ti, tj);
                const IO *X = (kind == 0 ? TL : tQ) + ti * 16 * PD;
                const IO *Y = (DT && !MILD && ti == tj ? tKd : tK) + tj * 16 * PD;
                Frag fa[KD], fb[KD];
#pragma unroll
                for (int ks = 0; ks < KD; ++ks) {
                    fa[ks] = M::load(X + ks * KS, PD);
                    fb[ks] = M::load(Y + ks * KS, PD);
                }
                if constexpr (CHAN && !MILD)  // the tile's per-channel factor (the diagonal's is in tKd with bfloat16 io)
                    if (ti - tj >= 2 || (!DT && ti == tj)) {
                        const float *f = sDec + (ti == tj ? 7 + ti : dec_row_far(ti, tj)) * D + FE * lg;
#pragma unroll
                        for (int ks = 0; ks < KD; ++ks) fb[ks] = K::scale(fb[ks], f + ks * KS);
                    }
                x[s] = zero4();
#pragma unroll
                for (int ks = 0; ks < KD; ++ks) x[s] = M::mma(x[s], fa[ks], fb[ks]);
            }
#pragma unroll
            for (int s = 0; s < 5; ++s) {
                const int p = w + NW * s, kind = p / 10;
                int ti, tj;
                lower_tile(p - kind * 10, ti, tj);
                const int col = tj * 16 + lr, row0 = ti * 16 + 4 * lg;
                f32x4 y = x[s];
                if constexpr (!CHAN) {
                    const f32x4 Gr = load4f(sG + row0);
                    const float Gc = sG[col];
                    f32x4 f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) f[r] = fast_exp(fminf(Gr[r] - Gc, 0.f));
                    if constexpr (!BW)
                        if (kind == 0) f *= load4f(sBt + row0);
                    y *= f;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = kind == 0 ? col < row0 + r : col <= row0 + r;
                    y[r] = keep ? y[r] : 0.f;
                }
                // (Diagonal tiles of a block formed entry by entry in phase A are kept.)
                if (CHAN && !MILD && ti == tj && sSlow[ti]) {
                } else if (kind == 0 && ti == tj) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sTd[(ti * 16 + lr) * 17 + 4 * lg + r] = y[r];
                } else {
                    store4f((kind == 0 ? sTc : sAc) + col * LC + row0, y);
                }
            }
            // A is zero above its diagonal tiles.
            for (int z = w; z < 6; z += NW) {
                const int ti = z < 3 ? 0 : z < 5 ? 1 : 2, tj = z < 3 ? z + 1 : z < 5 ? z - 1 : 3;
                store4f(sAc + (tj * 16 + lr) * LC + ti * 16 + 4 * lg, zero4());
            }
            // Q~ (or raw q once per QK head) fragments; per-channel decay: Q~ = Q^ . exp(R_b), b = rt.
            if (write_kT)
                for (int f = w; f < (C / 16) * (D / KS); f += NW) {
                    const int rt = f / (D / KS), ks = f - rt * (D / KS);
                    Frag x = M::load(tQ + rt * 16 * PD + ks * KS, PD);
                    if constexpr (CHAN && !MILD) x = K::scale(x, sDec + rt * D + ks * KS + FE * lg);
                    store_frag<IO, CHAN>(CHAN ? wQ : wQh, rt, ks, D, x);
                }
            // Kend^T (or raw k^T) fragments: rows = channels, K = tokens, read K-major from the tiles.
            if (write_kT)
                for (int f = w; f < (D / 16) * (C / KS); f += NW) {
                    const int rt = f / (C / KS), ks = f - rt * (C / KS);
                    Frag x = K::frag((DT ? tKe : tK) + ks * KS * PD + rt * 16, PD);
                    if constexpr (CHAN && !DT)  // Kend = K^ . exp(G_end - R_{b+1}), b = the fragment's token block
                        x = K::scale(x, sDec[(MILD ? 15 : 11 + ((ks * KS + FE * lg) >> 4)) * D + rt * 16 + lr]);
                    store_frag<IO, CHAN>(wKT, rt, ks, C, x);
                }
        };
        if (!CHAN || mild) gram(std::true_type{});
        else if constexpr (CHAN) gram(std::false_type{});
        __syncthreads();

        if (has_next) in.template load<1>(a, un, co, grp);

        // ---- C. A to the workspace; L = (I + T)^-1 ----
        for (int f = w; f < (C / 16) * (C / KS); f += NW) {
            const int rt = f / (C / KS), ks = f - rt * (C / KS);
            store_frag<IO, CHAN>(wA, rt, ks, C, K::frag(sAc + ks * KS * LC + rt * 16, LC));
        }
        // Diagonal block w of L: (I + T_ww)^-1 by fp32 substitution, lane lr < 16 forms column lr.
        float xd[16];
        if (l < 16) {
            const float *Tb = sTd + w * 16 * 17;  // T(i, m) of the block at Tb[m * 17 + i]
#pragma unroll
            for (int i = 0; i < 16; ++i) xd[i] = i == lr ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                float col[16];
#pragma unroll
                for (int i = m + 1; i < 16; ++i) col[i] = Tb[m * 17 + i];
#pragma unroll
                for (int i = m + 1; i < 16; ++i) xd[i] -= col[i] * xd[m];
            }
        }
        __syncthreads();  // A has been read out: its space becomes L
        if (l < 16) {
            IO *dst = sLc + (16 * w + lr) * LC + 16 * w;
#pragma unroll
            for (int i = 0; i < 16; i += 4) store4f(dst + i, f32x4{xd[i], xd[i + 1], xd[i + 2], xd[i + 3]});
        } else if (l < 32 && (w == 1 || w == 3)) {
            // Blocks (0,1) and (2,3) above the diagonal: phase D's 32-wide K steps read them.
            IO *dst = sLc + (16 * w + lr) * LC + 16 * (w - 1);
#pragma unroll
            for (int i = 0; i < 16; i += 4) store4f(dst + i, zero4());
        }
        __syncthreads();
        if (w < 3) {  // column block w: X_i = -D_i sum_{w <= k < i} T_ik X_k
            IO *tmp = sTmp + w * 16 * LT;
            for (int i = w + 1; i < 4; ++i) {
                f32x4 acc = zero4();
                for (int k = w; k < i; ++k)
                    acc = K::mma16(acc, sTc + 16 * k * LC + 16 * i, LC, sLc + 16 * w * LC + 16 * k, LC);
                store4f(tmp + lr * LT + 4 * lg, acc);
                wave_sync();
                const f32x4 x = K::mma16(zero4(), sLc + 16 * i * LC + 16 * i, LC, tmp, LT);
                store4f(sLc + (16 * w + lr) * LC + 16 * i + 4 * lg, -x);
                wave_sync();
            }
        }
        __syncthreads();

        if (has_next) in.template load<2>(a, un, co, grp, !next_same);

        // ---- D. [Y | U_z] = L [E~ | Z] ----
        {
            constexpr int NKS = C / KS;
            Frag la[4][NKS];
#pragma unroll
            for (int ri = 0; ri < 4; ++ri)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    if (ks * KS < 16 * ri + 16) la[ri][ks] = K::frag(sLc + ks * KS * LC + 16 * ri, LC);
#pragma unroll
            for (int ct = 0; ct < NCTS; ++ct) {
                const int c0 = WC * w + 16 * ct;
                const bool zside = c0 >= D;
                const IO *src = zside ? tZ + (c0 - D) : (DT && !mild ? tEt : HAS_E ? tE : tK) + c0;
                Frag bf[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    bf[ks] = K::frag(src + ks * KS * PD, PD);
                    if (!zside) {
                        if constexpr (!CHAN)
                            bf[ks] = K::scale(bf[ks], sSE + ks * KS + FE * lg);
                        else if constexpr (!DT) {  // E~ = E^ . exp(R_b), b = the fragment's token block
                            if (!mild) bf[ks] = K::scale(bf[ks], sDec[((ks * KS + FE * lg) >> 4) * D + c0 + lr]);
                        }
                    }
                }
#pragma unroll
                for (int ri = 0; ri < 4; ++ri) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        if (ks * KS < 16 * ri + 16) acc = M::mma(acc, la[ri][ks], bf[ks]);
                    if (zside) store4_ws<CHAN>(wUzT + cfrag_off<D>(c0 - D + lr, 16 * ri + 4 * lg), acc);
                    else store4f(sYc + (c0 + lr) * LY + 16 * ri + 4 * lg, acc);
                }
            }
        }
        __syncthreads();

        // ---- E. Y to the workspace ----
        for (int f = w; f < (C / 16) * (D / KS); f += NW) {
            const int rt = f / (D / KS), ks = f - rt * (D / KS);
            store_frag<IO, CHAN>(wY, rt, ks, D, K::frag(sYc + ks * KS * LY + rt * 16, LY));
        }
        if (!GROUPED || ++hh == PG) {
            hh = 0;
            gu += (int)gridDim.x;
        }
    }
}

// Sequential sweep over chunks for one (sequence, V head, value tile of BV =
// 16*NCT columns), with two kinds of waves. NWC = D/32 "chain" waves carry
// the state: chain wave w keeps state rows 32w..32w+31 in accumulator layout
// and per chunk forms P = Y S_c and U = U_z - P for its token tiles
// [w*TPW, (w+1)*TPW), then S_{c+1} = gamma . S_c + Kend^T U. NWC "output"
// waves form O = s (Q~ S_c + A U) for the same token tiles. Both kinds meet
// at two barriers per chunk: once S_c^T is in shared memory (the output waves
// then form Q~ S_c while the chain forms U) and once U^T is (the output waves
// then add A U and store O while the chain updates the state), so the output
// work and its loads stay off the state's critical path. Every wave
// prefetches its own slice of the chunk factors PF chunks ahead.
//
// With a scalar decay (CHAN false) the workspace holds neither Q~ nor Kend^T
// per V head: the output waves read the QK head's q and scale the rows of
// q S_c by exp(G_t), and the chain waves read its k^T and use the rows of U
// scaled by exp(G_end - G_t) for the state update
// (Kend^T U = k^T Diag(exp(G_end - G)) U).
template <typename IO, int D, int NCT>
struct SweepShape {
    using M = Mma<IO>;
    static constexpr int NWC = D / 32, TPW = 4 / NWC, KD = D / M::KS, KC = C / M::KS;
    static constexpr int BV = 16 * NCT, LS = D + 8, LU = C + 8, LO = BV + 8;
};

// Where one sweep work item finds its chunk factors.
template <typename IO>
struct SweepSrc {
    const IO *ws;     // io workspace
    const float *tab; // per-unit float tables
    const IO *kT;     // k^T and q of this QK head, chunk 0 (scalar decay)
    size_t u0;        // unit of chunk 0
};

template <typename IO, int D, int NCT, bool CHAN>
struct ChainOps {  // Y rows and U_z columns of the wave's token tiles; Kend^T (k^T) rows of its state rows; decay
    using Sh = SweepShape<IO, D, NCT>;
    using F = typename Sh::M::Frag;
    using R4 = Raw4<IO>;
    F ya[Sh::TPW][Sh::KD], ka[2][Sh::KC];
    typename R4::type uz[Sh::TPW][NCT];
    f32x4 g4[2];                     // gamma of the wave's state rows
    f32x4 er[CHAN ? 1 : Sh::TPW];    // exp(G_end - G) of the wave's token rows (scalar decay)

    __device__ __forceinline__ void load(const SweepSrc<IO> &src, int c, int w, int col0) {
        load_a(src, c, w, col0);
        load_b(src, c, w);
    }
    // The operands of U = U_z - Y S_c.
    __device__ __forceinline__ void load_a(const SweepSrc<IO> &src, int c, int w, int col0) {
        const int l = threadIdx.x & 63, lq = l >> 4;
        const size_t u = src.u0 + c;
        const IO *Y = src.ws + u * chunk_ws_io_elems(D, CHAN), *UzT = Y + ws_off_uz(D, CHAN);
        const float *tab = src.tab + u * kTab;
#pragma unroll
        for (int tt = 0; tt < Sh::TPW; ++tt) {
            const int rt = w * Sh::TPW + tt;
#pragma unroll
            for (int ks = 0; ks < Sh::KD; ++ks) ya[tt][ks] = load_frag(Y, rt, ks, D);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                uz[tt][ct] = R4::load(UzT + ((size_t)(rt * (D / 16) + col0 / 16 + ct) * 64 + l) * 4);
            if constexpr (!CHAN) er[tt] = load4f(tab + C + rt * 16 + 4 * lq);
        }
    }
    // The operands of the state update.
    __device__ __forceinline__ void load_b(const SweepSrc<IO> &src, int c, int w) {
        const int l = threadIdx.x & 63, lq = l >> 4;
        const size_t u = src.u0 + c;
        const IO *Y = src.ws + u * chunk_ws_io_elems(D, CHAN);
        const IO *KT = CHAN ? Y + 2 * C * D : src.kT + (size_t)c * 2 * D * C;
        const float *tab = src.tab + u * kTab;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int ch0 = 32 * w + 16 * rt;
#pragma unroll
            for (int ks = 0; ks < Sh::KC; ++ks) ka[rt][ks] = load_frag(KT, ch0 / 16, ks, C);
            if constexpr (CHAN) g4[rt] = load4f(tab + ch0 + 4 * lq);
            else { const float gm = tab[C - 1]; g4[rt] = f32x4{gm, gm, gm, gm}; }
        }
    }
};

template <typename IO, int D, int NCT, bool CHAN>
struct OutOps {  // Q~ (q) and A rows of the wave's token tiles
    using Sh = SweepShape<IO, D, NCT>;
    using F = typename Sh::M::Frag;
    F qa[Sh::TPW][Sh::KD], aa[Sh::TPW][Sh::KC];
    float eg[CHAN ? 1 : Sh::TPW];    // exp(G) of this lane's token in each of the wave's tiles (scalar decay)

    __device__ __forceinline__ void load(const SweepSrc<IO> &src, int c, int w) {
        load_a(src, c, w);
        load_b(src, c, w);
    }
    // The operands of Q~ S_c.
    __device__ __forceinline__ void load_a(const SweepSrc<IO> &src, int c, int w) {
        const int lr = threadIdx.x & 15;
        const size_t u = src.u0 + c;
        const IO *unit = src.ws + u * chunk_ws_io_elems(D, CHAN);
#pragma unroll
        for (int tt = 0; tt < Sh::TPW; ++tt) {
            const int rt = w * Sh::TPW + tt;
            if constexpr (CHAN) {
#pragma unroll
                for (int ks = 0; ks < Sh::KD; ++ks) qa[tt][ks] = load_frag(unit + C * D, rt, ks, D);
            } else {
                const IO *Qf = src.kT + (size_t)c * 2 * D * C + D * C;
#pragma unroll
                for (int ks = 0; ks < Sh::KD; ++ks) qa[tt][ks] = load_frag(Qf, rt, ks, D);
                eg[tt] = src.tab[u * kTab + rt * 16 + lr];
            }
        }
    }
    // The operand of A U.
    __device__ __forceinline__ void load_b(const SweepSrc<IO> &src, int c, int w) {
        const size_t u = src.u0 + c;
        const IO *A = src.ws + u * chunk_ws_io_elems(D, CHAN) + ws_off_a(D, CHAN);
#pragma unroll
        for (int tt = 0; tt < Sh::TPW; ++tt)
#pragma unroll
            for (int ks = 0; ks < Sh::KC; ++ks) aa[tt][ks] = load_frag(A, w * Sh::TPW + tt, ks, C);
    }
};

// One chunk on a chain wave.
// With RELOAD, the wave refills op with chunk cn's operands as soon as each
// part has been consumed (the U operands before the second barrier, the
// state-update operands at the end), spreading its loads over the chunk.
template <typename IO, int D, int NCT, bool CHAN, bool RELOAD = false>
__device__ __forceinline__ void chain_chunk(ChainOps<IO, D, NCT, CHAN> &op, f32x4 (&S)[2][NCT], IO *sST,
                                            IO *sUT, IO *sUK, int w, bool zero_uz = false,
                                            const SweepSrc<IO> *src = nullptr, int cn = 0, int col0 = 0) {
    using Sh = SweepShape<IO, D, NCT>;
    using M = typename Sh::M;
    using F = typename M::Frag;
    constexpr int KS = M::KS, LS = Sh::LS, LU = Sh::LU;
    const int l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            store4f(sST + (16 * ct + lr) * LS + 32 * w + 16 * rt + 4 * lq, S[rt][ct]);
    __syncthreads();  // S_c^T is shared
#pragma unroll
    for (int tt = 0; tt < Sh::TPW; ++tt) {
        const int T0 = (w * Sh::TPW + tt) * 16;
        f32x4 accP[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accP[ct] = zero4();
#pragma unroll
        for (int ks = 0; ks < Sh::KD; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                accP[ct] = M::mma(accP[ct], op.ya[tt][ks], M::load(sST + 16 * ct * LS + ks * KS, LS));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 U = (zero_uz ? zero4() : Raw4<IO>::widen(op.uz[tt][ct])) - accP[ct];
            store4f(sUT + (16 * ct + lr) * LU + T0 + 4 * lq, U);
            if constexpr (!CHAN) store4f(sUK + (16 * ct + lr) * LU + T0 + 4 * lq, U * op.er[tt]);
        }
    }
    if constexpr (RELOAD) op.load_a(*src, cn, w, col0);
    __syncthreads();  // U^T is shared
    const IO *sU = CHAN ? sUT : sUK;
    F ub[Sh::KC][NCT];
#pragma unroll
    for (int ks = 0; ks < Sh::KC; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) ub[ks][ct] = M::load(sU + 16 * ct * LU + ks * KS, LU);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= op.g4[rt];
#pragma unroll
        for (int ks = 0; ks < Sh::KC; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = M::mma(S[rt][ct], op.ka[rt][ks], ub[ks][ct]);
    }
    if constexpr (RELOAD) op.load_b(*src, cn, w);
}

// One chunk on an output wave (w = its index among the output waves). The
// wave forms its token tiles of O transposed, O^T = S_c^T Q~^T + U^T A^T (the
// matrix-core operands swapped), so each lane holds 4 consecutive value
// columns of one token: they go to the staging rows as one 8- or 16-byte
// write. With RELOAD the wave refills op with chunk cn's Q~ once the second
// barrier has passed and its A at the end. TAIL = the chunk may hold fewer
// than C tokens (only the last one), so output rows are stored under a
// predicate; every other chunk stores unconditionally, which keeps the number
// of memory operations in flight static.
template <typename IO, int D, int NCT, bool CHAN, bool TAIL, bool RELOAD = false>
__device__ __forceinline__ void out_chunk(OutOps<IO, D, NCT, CHAN> &op, const IO *sST, const IO *sUT, IO *sO,
                                          IO *orow0, size_t orow_stride, int n_valid, float scale, int w,
                                          const SweepSrc<IO> *src = nullptr, int cn = 0) {
    using Sh = SweepShape<IO, D, NCT>;
    using M = typename Sh::M;
    using F = typename M::Frag;
    constexpr int KS = M::KS, LS = Sh::LS, LU = Sh::LU, LO = Sh::LO, BV = Sh::BV;
    const int l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
    f32x4 accR[Sh::TPW][NCT];
    __syncthreads();  // S_c^T is shared
#pragma unroll
    for (int tt = 0; tt < Sh::TPW; ++tt) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) accR[tt][ct] = zero4();
#pragma unroll
        for (int ks = 0; ks < Sh::KD; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                accR[tt][ct] = M::mma(accR[tt][ct], M::load(sST + 16 * ct * LS + ks * KS, LS), op.qa[tt][ks]);
        if constexpr (!CHAN)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) accR[tt][ct] *= op.eg[tt];
    }
    __syncthreads();  // U^T is shared
    if constexpr (RELOAD) op.load_a(*src, cn, w);
    F ub[Sh::KC][NCT];
#pragma unroll
    for (int ks = 0; ks < Sh::KC; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) ub[ks][ct] = M::load(sUT + 16 * ct * LU + ks * KS, LU);
#pragma unroll
    for (int tt = 0; tt < Sh::TPW; ++tt) {
        const int T0 = (w * Sh::TPW + tt) * 16;
        // All K steps (A is zero above its diagonal tiles): a trip count that
        // depends on the wave would put branches around the prefetch
        // bookkeeping and force a full drain of the loads in flight.
#pragma unroll
        for (int ks = 0; ks < Sh::KC; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) accR[tt][ct] = M::mma(accR[tt][ct], ub[ks][ct], op.aa[tt][ks]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) store4f(sO + (T0 + lr) * LO + 16 * ct + 4 * lq, scale * accR[tt][ct]);
        // This wave's output rows, 16 bytes per lane (wave-local staging).
        constexpr int V = 16 / sizeof(IO), PER = BV / V;
#pragma unroll
        for (int i = l; i < 16 * PER; i += 64) {
            const int tok = T0 + i / PER, c8 = (i % PER) * V;
            if (!TAIL || tok < n_valid)
                st16_stream(orow0 + tok * orow_stride + c8, *reinterpret_cast<const uint4 *>(sO + tok * LO + c8));
        }
    }
    if constexpr (RELOAD) op.load_b(*src, cn, w);
}

template <typename IO, int D, int NCT, int PF, bool CHAN>
__global__ __launch_bounds__(4 * D) void chunk_sweep(ChunkArgs a, int NVT, int G) {
    using Sh = SweepShape<IO, D, NCT>;
    constexpr int BV = Sh::BV, LS = Sh::LS, LU = Sh::LU, LO = Sh::LO, NWC = Sh::NWC;
    __shared__ __align__(16) IO sST[BV * LS];                 // S_c^T in the io dtype
    __shared__ __align__(16) IO sUT[BV * LU];                 // U^T in the io dtype
    __shared__ __align__(16) IO sUK[CHAN ? 1 : BV * LU];      // (Diag(exp(G_end - G)) U)^T (scalar decay)
    __shared__ __align__(16) IO sO[C * LO];                   // output rows (each output wave stages its own)

    // Work index: blocks that share an XCD (blockIdx % 8) take consecutive
    // work items, so the value tiles of one head read its chunk factors
    // through the same L2.
    const int x = blockIdx.x;
    const int wi = (x & 7) * (int)(gridDim.x >> 3) + (x >> 3);
    if (wi >= G) return;
    // Work item ((sequence, V head), segment, value tile); one segment unless the sweep is split.
    const int vt = wi % NVT, bs = wi / NVT, sg = bs % a.P, bh = bs / a.P, col0 = vt * BV;
    const int b = bh / a.Hv, h = bh - (bh / a.Hv) * a.Hv, hq = h / (a.Hv / a.Hqk);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
    const int cb = sg * a.L, NC = min(a.L, a.NC - cb);  // this segment's chunks [cb, cb + NC)
    // Entry state: S0 for the first segment, else the one the segment scan found.
    // Entry state: the one the segment scan found; for the first segment the
    // scan's copy of S0 when the sweep is split (the last segment's S_T may
    // overwrite S0 in place while the first segment has not read it yet),
    // else S0 itself.
    const float *Sin = sg > 0 ? a.ws_seg + ((size_t)(bh * (a.P - 1) + sg - 1) * 3 + 2) * D * D
                       : a.P > 1 ? a.ws_seg + ((size_t)bh * (a.P - 1) * 3 + 1) * D * D
                       : a.S0 ? a.S0 + (size_t)bh * D * D : nullptr;
    const bool last = sg == a.P - 1;

    SweepSrc<IO> src;
    src.ws = static_cast<const IO *>(a.ws_io);
    src.tab = a.ws_tab;
    src.u0 = (size_t)bh * a.NC + cb;
    src.kT = CHAN ? nullptr : static_cast<const IO *>(a.ws_kT) + ((size_t)(b * a.Hqk + hq) * a.NC + cb) * (2 * D * C);

    if (wv < NWC) {  // ---- chain wave ----
        const int w = wv;
        f32x4 S[2][NCT];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ch = 32 * w + 16 * rt + 4 * lq + r, col = col0 + 16 * ct + lr;
                    S[rt][ct][r] = Sin ? Sin[(size_t)ch * D + col] : 0.f;
                }
        if (NC > 0) {
            ChainOps<IO, D, NCT, CHAN> ring[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) ring[j].load(src, min(j, NC - 1), w, col0);
            int c = 0;
            for (; c + PF <= NC - 1; c += PF) {
#pragma unroll
                for (int j = 0; j < PF; ++j)
                    chain_chunk<IO, D, NCT, CHAN, true>(ring[j], S, sST, sUT, sUK, w, false, &src,
                                                        min(c + j + PF, NC - 1), col0);
            }
#pragma unroll
            for (int j = 0; j < PF; ++j)
                if (c + j < NC) chain_chunk<IO, D, NCT, CHAN>(ring[j], S, sST, sUT, sUK, w);
        }
        if (last)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int ch = 32 * w + 16 * rt + 4 * lq + r, col = col0 + 16 * ct + lr;
                        a.ST[((size_t)bh * D + ch) * D + col] = S[rt][ct][r];
                    }
    } else if (NC > 0) {  // ---- output wave: same chunk sequence, same barriers ----
        const int w = wv - NWC;
        const size_t orow_stride = (size_t)a.Hv * D;
        IO *obase = static_cast<IO *>(a.o) + (((size_t)b * a.T + (size_t)cb * C) * a.Hv + h) * D + col0;
        const auto nv = [&](int cj) { return min(C, a.T - (cb + cj) * C); };
        OutOps<IO, D, NCT, CHAN> ring[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) ring[j].load(src, min(j, NC - 1), w);
        int c = 0;
        for (; c + PF <= NC - 1; c += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j)
                out_chunk<IO, D, NCT, CHAN, false, true>(ring[j], sST, sUT, sO,
                                                         obase + (size_t)(c + j) * C * orow_stride, orow_stride, C,
                                                         a.scale, w, &src, min(c + j + PF, NC - 1));
        }
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int cj = c + j;
            if (cj < NC)
                out_chunk<IO, D, NCT, CHAN, true>(ring[j], sST, sUT, sO, obase + (size_t)cj * C * orow_stride,
                                                  orow_stride, nv(cj), a.scale, w);
        }
    }
}

// Segmented sweep, first pass: for every segment but the last, run the state
// chain from a zero entry state to get the segment's end state N, and on d_k
// more columns from the identity with U_z = 0 to get its transition M (the
// state after the segment is M S_in + N). Chain waves only. Fetching one chunk
// ahead, the pass is held to at least three waves per SIMD, so that three of
// its workgroups share a compute unit and hide each other's loads.
template <typename IO, int D, int NCT, int PF, bool CHAN>
__global__ __launch_bounds__(2 * D, (PF == 1 ? 3 : 1)) void chunk_seg_state(ChunkArgs a, int NVT, int G) {
    using Sh = SweepShape<IO, D, NCT>;
    constexpr int BV = Sh::BV, LS = Sh::LS, LU = Sh::LU;
    __shared__ __align__(16) IO sST[BV * LS];
    __shared__ __align__(16) IO sUT[BV * LU];
    __shared__ __align__(16) IO sUK[CHAN ? 1 : BV * LU];
    const int x = blockIdx.x;
    const int wi = (x & 7) * (int)(gridDim.x >> 3) + (x >> 3);
    if (wi >= G) return;
    const int NT2 = 2 * NVT;  // value tiles of N, then of M (d_k = d_v)
    const int t = wi % NT2, bs = wi / NT2, sg = bs % (a.P - 1), bh = bs / (a.P - 1);
    const bool mpart = t >= NVT;
    const int col0 = (mpart ? t - NVT : t) * BV;
    const int b = bh / a.Hv, h = bh - (bh / a.Hv) * a.Hv, hq = h / (a.Hv / a.Hqk);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
    const int cb = sg * a.L, NC = a.L;  // a full segment: only the last one can be shorter

    SweepSrc<IO> src;
    src.ws = static_cast<const IO *>(a.ws_io);
    src.tab = a.ws_tab;
    src.u0 = (size_t)bh * a.NC + cb;
    src.kT = CHAN ? nullptr : static_cast<const IO *>(a.ws_kT) + ((size_t)(b * a.Hqk + hq) * a.NC + cb) * (2 * D * C);

    f32x4 S[2][NCT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = 32 * w + 16 * rt + 4 * lq + r, col = col0 + 16 * ct + lr;
                S[rt][ct][r] = mpart && ch == col ? 1.f : 0.f;
            }
    ChainOps<IO, D, NCT, CHAN> ring[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) ring[j].load(src, min(j, NC - 1), w, col0);
    int c = 0;
    for (; c + PF <= NC - 1; c += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j)  // the refill goes out in two parts, each once its operands are used
            chain_chunk<IO, D, NCT, CHAN, true>(ring[j], S, sST, sUT, sUK, w, mpart, &src, min(c + j + PF, NC - 1),
                                                col0);
    }
#pragma unroll
    for (int j = 0; j < PF; ++j)
        if (c + j < NC) chain_chunk<IO, D, NCT, CHAN>(ring[j], S, sST, sUT, sUK, w, mpart);

    float *dst = a.ws_seg + ((size_t)(bh * (a.P - 1) + sg) * 3 + (mpart ? 0 : 1)) * D * D;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = 32 * w + 16 * rt + 4 * lq + r, col = col0 + 16 * ct + lr;
                dst[(size_t)ch * D + col] = S[rt][ct][r];
            }
}

// Segmented sweep, scan over segments: S_in(s + 1) = M_s S_in(s) + N_s in fp32
// on the matrix cores (v_mfma_f32_16x16x4_f32), one workgroup per (sequence,
// V head, 16 state columns); S_in(s) stays in shared memory. Each lane reads
// 4 consecutive entries of an M row at once and feeds them to 4 successive
// products (the k index of product (j, i) at lane group g is 16 j + 4 g + i,
// the same for the S_in operand), and the next segment's M and N are
// fetched while the current one is multiplied.
template <int D>
__global__ __launch_bounds__(256) void chunk_seg_combine(ChunkArgs a) {
    constexpr int NTC = 16, NKG = D / 16;
    constexpr int RPW = (D / 16 + 3) / 4;  // row tiles per wave
    __shared__ __align__(16) float sIn[D * NTC];
    const int bh = blockIdx.x / (D / NTC), c0 = (blockIdx.x % (D / NTC)) * NTC;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lr = l & 15, lg = l >> 4;
    for (int i = tid; i < D * NTC; i += 256)
        sIn[i] = a.S0 ? a.S0[((size_t)bh * D + i / NTC) * D + c0 + i % NTC] : 0.f;
    const auto seg = [&](int s) { return a.ws_seg + ((size_t)(bh * (a.P - 1) + s) * 3) * D * D; };
    f32x4 mr[2][RPW][NKG], nv[2][RPW];
    const auto fetch = [&](int s, auto bc) {
        constexpr int buf = decltype(bc)::value;
        const float *M = seg(s), *N = M + D * D;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rt = w + 4 * i;
            if (rt < D / 16) {
#pragma unroll
                for (int j = 0; j < NKG; ++j) mr[buf][i][j] = load4f(M + (size_t)(16 * rt + lr) * D + 16 * j + 4 * lg);
#pragma unroll
                for (int r = 0; r < 4; ++r) nv[buf][i][r] = N[(size_t)(16 * rt + 4 * lg + r) * D + c0 + lr];
            }
        }
    };
    // Steps alternate between the two operand buffers (compile-time indices,
    // so the buffers stay in registers).
    const auto step = [&](int s, auto cc) {
        constexpr int cur = decltype(cc)::value;
        if (s + 1 < a.P - 1) fetch(s + 1, std::integral_constant<int, cur ^ 1>{});
        float *N = seg(s) + D * D, *Sn = seg(s) + 2 * D * D;
        __syncthreads();  // S_in(s) complete
        f32x4 acc[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rt = w + 4 * i;
            if (rt < D / 16) {
                acc[i] = nv[cur][i];
                // Once read, N_0 keeps a copy of S0 for the sweep's first
                // segment (S_T may alias S0).
                if (s == 0)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * rt + 4 * lg + r;
                        N[(size_t)row * D + c0 + lr] = sIn[row * NTC + lr];
                    }
#pragma unroll
                for (int j = 0; j < NKG; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(mr[cur][i][j][q],
                                                                      sIn[(16 * j + 4 * lg + q) * NTC + lr], acc[i], 0, 0, 0);
            }
        }
        __syncthreads();  // everyone has read S_in(s)
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int rt = w + 4 * i;
            if (rt < D / 16)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * rt + 4 * lg + r;
                    sIn[row * NTC + lr] = acc[i][r];
                    Sn[(size_t)row * D + c0 + lr] = acc[i][r];
                }
        }
    };
    fetch(0, std::integral_constant<int, 0>{});
    for (int s = 0; s < a.P - 1; s += 2) {
        step(s, std::integral_constant<int, 0>{});
        if (s + 1 < a.P - 1) step(s + 1, std::integral_constant<int, 1>{});
    }
}

template <typename IO, int D, int NCT>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t s) {
    using Cfg = PrepCfg<IO, D>;
    // Shared memory per prep variant (CHAN, BW): the per-channel-decay and
    // decoupled-gate variants keep more tiles.
    // Once per process (thread-safe): allow each variant its shared memory.
    // Float32 io at d = 128 has only the tied-gate, scalar-decay prep: the
    // variants with an erase-key tile would need more than a CU's 160 KiB of
    // shared memory, and the input-stage and per-channel variants reduce over
    // a token row's lanes in 16-lane groups (a row spans 32 lanes there).
    constexpr bool ALL = !(sizeof(IO) == 4 && D == 128);
    static const hipError_t attr_err = [] {
        if constexpr (!ALL) {
            return hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_prep<IO, D, false, false, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::bytes(false, false));
        } else {
            // (With a per-channel decay and the input stage, the convolution
            // runs as a pass of its own, stage.hip, and the prep applies only
            // the gate and decay activations.)
            const void *fns[8] = {reinterpret_cast<const void *>(&chunk_prep<IO, D, false, false, false>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, false, true, false>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, true, false, false>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, true, true, false>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, false, false, true>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, false, true, true>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, true, false, true>),
                                  reinterpret_cast<const void *>(&chunk_prep<IO, D, true, true, true>)};
            const size_t lds[4] = {Cfg::bytes(false, false), Cfg::bytes(true, false), Cfg::bytes(true, true),
                                   Cfg::bytes(true, true)};
            for (int i = 0; i < 8; ++i) {
                hipError_t e = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds[i % 4]);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }();
    if (attr_err != hipSuccess) return attr_err;
    const long long units = (long long)a.B * a.Hv * a.NC;
    if (units > 0) {
        // Persistent: as many workgroups as fit on the device at once.
        const bool chan = a.decay == DECAY_CHANNEL, bw = a.beta == nullptr;
        const int occ = !chan && !bw && 2 * Cfg::bytes(false, false) <= (size_t)160 * 1024
                            ? prep_occupancy<IO, D, false, false>() : 1;
        const long long slots = (long long)occ * device_cus();
        // V heads per work item: a divisor of the group size, the one with
        // the shortest schedule counted in units (rounds of work items times
        // heads per item), the largest of those that tie.
        // (Grouped variant only; 1 otherwise.)
        const int grpsz = a.conv_w && !chan && !bw ? a.Hv / a.Hqk : 1;
        int pg = 1;
        long long best = -1;
        for (int d = 1; d <= grpsz; ++d) {
            if (grpsz % d) continue;
            const long long span = (units / d + slots - 1) / slots * d;
            if (best < 0 || span <= best) { best = span; pg = d; }
        }
        ChunkArgs ap = a;
        ap.prep_grp = pg;
        const long long items = units / pg;
        const long long grid = items < slots ? items : slots;
        const dim3 g((unsigned)grid), b(Cfg::NT);
        if constexpr (!ALL) {
            if (a.conv_w || chan || bw) return hipErrorInvalidValue;
            hipLaunchKernelGGL((chunk_prep<IO, D, false, false, false>), g, b, Cfg::bytes(false, false), s, ap);
        } else if (chan && a.raw_gates) {  // q, k, v from the stage pass; gate and decay activations here
            if (a.conv_w) return hipErrorInvalidValue;
            if (bw) hipLaunchKernelGGL((chunk_prep<IO, D, true, true, true>), g, b, Cfg::bytes(true, true), s, ap);
            else hipLaunchKernelGGL((chunk_prep<IO, D, true, false, true>), g, b, Cfg::bytes(true, true), s, ap);
        } else if (a.conv_w) {
            if (chan) return hipErrorInvalidValue;  // the convolution runs first as a pass of its own
            if (bw) hipLaunchKernelGGL((chunk_prep<IO, D, false, true, true>), g, b, Cfg::bytes(true, false), s, ap);
            else hipLaunchKernelGGL((chunk_prep<IO, D, false, false, true>), g, b, Cfg::bytes(false, false), s, ap);
        } else {
            if (chan && bw) hipLaunchKernelGGL((chunk_prep<IO, D, true, true, false>), g, b, Cfg::bytes(true, true), s, ap);
            else if (chan) hipLaunchKernelGGL((chunk_prep<IO, D, true, false, false>), g, b, Cfg::bytes(true, true), s, ap);
            else if (bw) hipLaunchKernelGGL((chunk_prep<IO, D, false, true, false>), g, b, Cfg::bytes(true, false), s, ap);
            else hipLaunchKernelGGL((chunk_prep<IO, D, false, false, false>), g, b, Cfg::bytes(false, false), s, ap);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NVT = D / (16 * NCT);
    constexpr int PF = sizeof(IO) == 2 ? SWEEP_PF : 1;  // prefetch depth (fp32 fragments are 2x larger)
    // A split sweep with bf16 io at d = 128 runs 64-column work items (the
    // segment policy counts on it), fetching 2 chunks ahead; the segment
    // pass keeps 32-column items.
    constexpr int NCTS = sizeof(IO) == 2 && D == 128 ? 4 : NCT, NVTS = D / (16 * NCTS);
    constexpr int PFS = NCTS != NCT ? 2 : PF;
    if (a.P > 1) {  // segmented: transitions and end states, then the scan over segments
        // With per-channel decay the segment pass fetches one chunk ahead and
        // runs three workgroups per CU instead of prefetching deeper.
        constexpr int NCT1 = NCT, NVT1 = NVT;
        const int G1 = a.B * a.Hv * (a.P - 1) * 2 * NVT1;
        const int grid1 = (G1 + 7) / 8 * 8;
        if (a.decay == DECAY_CHANNEL)
            hipLaunchKernelGGL((chunk_seg_state<IO, D, NCT1, 1, true>), dim3(grid1), dim3(2 * D), 0, s, a, NVT1, G1);
        else
            hipLaunchKernelGGL((chunk_seg_state<IO, D, NCT1, PF, false>), dim3(grid1), dim3(2 * D), 0, s, a, NVT1, G1);
        hipLaunchKernelGGL((chunk_seg_combine<D>), dim3(a.B * a.Hv * (D / 16)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (NCTS != NCT) {
        if (a.P > 1) {
            const int G = a.B * a.Hv * a.P * NVTS;
            const int grid = (G + 7) / 8 * 8;
            if (a.decay == DECAY_CHANNEL)
                hipLaunchKernelGGL((chunk_sweep<IO, D, NCTS, PFS, true>), dim3(grid), dim3(4 * D), 0, s, a, NVTS, G);
            else
                hipLaunchKernelGGL((chunk_sweep<IO, D, NCTS, PFS, false>), dim3(grid), dim3(4 * D), 0, s, a, NVTS, G);
            return hipGetLastError();
        }
    }
    const int G = a.B * a.Hv * a.P * NVT;
    const int grid = (G + 7) / 8 * 8;
    if (a.decay == DECAY_CHANNEL)
        hipLaunchKernelGGL((chunk_sweep<IO, D, NCT, PF, true>), dim3(grid), dim3(4 * D), 0, s, a, NVT, G);
    else
        hipLaunchKernelGGL((chunk_sweep<IO, D, NCT, PF, false>), dim3(grid), dim3(4 * D), 0, s, a, NVT, G);
    return hipGetLastError();
}

bool chunk_supported(int io, int D) { return D == 32 || D == 64 || D == 128; }

hipError_t launch_chunk(int io, int D, const ChunkArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_chunk_t<bf16_t, 32, 1>(a, s);
        if (D == 64) return launch_chunk_t<bf16_t, 64, 2>(a, s);
        if (D == 128) return launch_chunk_t<bf16_t, 128, SWEEP_NCT128>(a, s);
    } else {
        if (D == 32) return launch_chunk_t<float, 32, 1>(a, s);
        if (D == 64) return launch_chunk_t<float, 64, 2>(a, s);
        if (D == 128) return launch_chunk_t<float, 128, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
