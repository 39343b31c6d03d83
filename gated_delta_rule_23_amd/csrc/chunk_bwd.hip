// chunk_bwd.hip -- gradients of the gated delta-rule recurrence, chunked form.
//
// The page "Resumo Técnico: Gated DeltaNet-2", section "Treinamento Paralelo
// Eficiente por Blocos", names a backward pass that is parallel over blocks
// of tokens and in which the gates enter the gradient accumulation; it prints
// no formula. What is computed here is the exact gradient of the chunked
// (WY/UT) forward of the page "Uma análise das variantes de atenção linear
// da família DeltaNet", section "Chunkwise KDA" and its subsections, with the
// decoupled gates of that same "Treinamento Paralelo" section; the chunked
// form equals the token recurrence. Per (sequence, V head) and
// chunk of C = 64 tokens, with S the state entering the chunk, G the in-chunk
// inclusive sums of the log-decay g, e = beta k or b . k, z = beta v or w . v:
//
//   E~ = e . exp(G),  Q~ = q . exp(G),  Kend = k . exp(G_end - G),
//   Gamma = exp(G_end);  T (strictly lower), A (lower with the diagonal):
//   T_tj = sum_d e_t k_j exp(G_t - G_j),   A_tj = sum_d q_t k_j exp(G_t - G_j)
//   L = (I + T)^-1,  Y = L E~,  U_z = L Z,  U = U_z - Y S,
//   O = s (Q~ S + A U),  S_next = Diag(Gamma) S + Kend^T U.
//
// Given dO and dS_next, reverse-mode differentiation of these lines gives
//
//   dU = s A^T dO + Kend dS_next            dR = L^T dU  (dZ = dR)
//   dS = Diag(Gamma) dS_next + s Q~^T dO - Y^T dU
//   dT = -dR U^T (strictly lower),          dA = s dO U^T (lower)
//   dE~ = -dR S^T (+ the T part),           dQ~ = s dO S^T (+ the A part)
//   dKend = U dS_next^T,                    dGamma = rowsum(dS_next . S)
//
// then through T and A to e, k, q and through the exponentials to G: a
// factor exp(x) with x linear in G passes x' times its own value times its
// gradient. dg_m is the sum of dG_t over t >= m in the chunk plus dG_end.
//
// With a scalar decay the exponentials of T and A are kept per entry,
// exp(G_t - G_j) <= 1. With a per-channel decay the products over channels
// are referenced per 16-token block, as in the forward: with Gb the in-block
// prefix of g, B_b the block's sum and R_b the sum of the blocks before it,
//   E^ = e . exp(Gb),  Q^ = q . exp(Gb),  K^ = k . exp(B_b - Gb)  (<= |x|),
// and for t in block bi, j in block bj < bi,
//   exp(G_t - G_j) = exp(Gb_t) . exp(R_bi - R_{bj+1}) . exp(B_bj - Gb_j),
// every factor <= 1; on a diagonal block the middle factor is exp(-B_bi),
// at most exp(kBwdDiagRange), and a block that decays further on some
// channel has its diagonal entries formed one by one, sum_c e_tc k_jc
// exp(Gb_tc - Gb_jc). The same split serves the products through T and A in
// the gradient pass, so no factor overflows or vanishes at any decay. The
// chunk-referenced operands follow by factors <= 1: E~ = E^ . exp(R_b),
// Q~ = Q^ . exp(R_b), Kend = K^ . exp(G_end - R_{b+1}). The workspace keeps
// Gb (not G) per channel, from which every one of these is formed exactly.
//
// Shared-memory tiles keep 16-byte aligned rows (stride a multiple of 4
// floats); global arrays are staged through registers with 16-byte (8-byte
// for bf16) loads. All arithmetic is fp32: the dense products (T and A, the
// triangular solves, the sweeps' steps and the gradient products) on the
// matrix cores (v_mfma_f32_16x16x4_f32), the rest on the vector units.
//
// Four launches (five or six: grouped heads; a sweep whose chain bounds the call):
//  1. cb_prep (per chunk unit): G, the factors above, T and A, and the
//     triangular solve (I + T)[Y | U_z] = [E~ | Z] by 16 x 16 blocks.
//  1b. cb_rhs (per unit, when both sweeps fit on the GPU at once): the
//     products of the backward sweep's step that do not depend on dS_next.
//  2. cb_sweeps, per (sequence, V head, 32 value columns) twice over: the
//     states S entering every chunk and U, walking the chunks forward; and
//     dS_next of every chunk and dU, walking them backward (dS_0 at the end).
//  3. cb_grad_s (per unit): dR by back substitution, dT, dA and the products
//     with S and dS_next.
//  4. cb_grad_out (per unit): the products through T and A, the exponential
//     factors, the gates, and the reverse sums over the chunk giving dg; then
//     (grouped heads) cb_group_sum adds the V heads' dq and dk per QK head.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {
namespace {

constexpr int C = kChunk;
constexpr int NT = 512;     // threads per workgroup of the per-chunk kernels (two waves per SIMD)
constexpr int BV = 32;      // value columns per sweep workgroup
constexpr int LB = BV + 4;  // row stride of 32-column tiles
constexpr int LC = C + 4;   // row stride of 64-column tiles
constexpr int LT = C + 16;  // row stride of 64-column tiles that the matrix cores read down their columns
// Per-channel decay: a diagonal block whose decay exceeds kBwdDiagRange on
// some channel is formed entry by entry (its factor exp(-B) is not used).
constexpr float kBwdDiagRange = 40.f;
// Rows of the per-channel factor table of cb_prep (each D floats):
//   0-3 exp(R_b); 4-6 exp(B_1), exp(B_2), exp(B_1 + B_2) (tiles (2,0), (3,1),
//   (3,0)); 7-10 exp(-B_b), capped at exp(kBwdDiagRange); 11-14
//   exp(G_end - R_{b+1}). cb_grad_out keeps rows 4-10 only, as its rows 0-6.
constexpr int kBwdDecRows = 15;
__host__ __device__ constexpr int bwd_row_far(int bi, int bj) {  // row of tile (bi, bj), bi - bj >= 2
    return bi == 2 ? 4 : bj == 1 ? 5 : 6;
}

constexpr int NS = 512;  // threads per sweep workgroup (two waves per SIMD)
template <int D>
struct SwCfg {
    static constexpr int NL = C * D / (4 * NS);  // 4-element groups per thread of a C x D array
    // State rows: threads per row and columns each (at least 4 columns; with
    // d = 32 only the first D * TPR threads hold state rows).
    static constexpr int NTL = D / BV, TPR = NS / D < BV / 4 ? NS / D : BV / 4, CPT = BV / TPR;
};
// Element e (a multiple of 4) of a row-major array with W columns, group l of this sweep thread.
template <int W>
__device__ __forceinline__ void rcs(int l, int &e, int &t, int &d) {
    e = 4 * (l * NS + (int)threadIdx.x);
    t = e / W;
    d = e - t * W;
}

template <int D>
struct Cfg {
    static constexpr int LD = D + 4;              // row stride of D-column tiles
    static constexpr int NL = C * D / (4 * NT);   // 4-element groups per thread of a C x D array
    static constexpr int NCG = D / 4, NRG = NT / NCG, RT = C / NRG;  // cb_grad_out: column groups, row groups, rows each
};

__device__ __forceinline__ f32x4 lds4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void sts4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }
__device__ __forceinline__ f32x4 splat(float x) { return f32x4{x, x, x, x}; }
// Workspace stores between the passes, non-temporal: the fp32 factors,
// states and partial gradients of one call (0.5-3 GB a pass at these
// shapes) outgrow the memory-side cache, so caching them only churns it.
__device__ __forceinline__ void stg4(float *p, f32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p)); }
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b, float acc) {
    return fmaf(a[3], b[3], fmaf(a[2], b[2], fmaf(a[1], b[1], fmaf(a[0], b[0], acc))));
}
template <typename IO>
__device__ __forceinline__ f32x4 ld4io(const void *p, size_t i) {  // 4 consecutive io elements, widened
    return Raw4<IO>::widen(Raw4<IO>::load(static_cast<const IO *>(p) + i));
}
template <typename IO>
__device__ __forceinline__ float ld1io(const void *p, size_t i) {  // one io element, widened
    if constexpr (sizeof(IO) == 2) return bf2f(static_cast<const IO *>(p)[i]);
    else return static_cast<const IO *>(p)[i];
}
__device__ __forceinline__ f32x4 exp4(f32x4 x) { return f32x4{expf(x[0]), expf(x[1]), expf(x[2]), expf(x[3])}; }

struct Unit {
    int b, h, hq, c, t0, n;
    size_t rowq, rowv;  // token t0's row index in the [B, T, H] layouts of q, k and of v (and per-head scalars)
};
__device__ __forceinline__ Unit decode(const ChunkBwdArgs &a, int u) {
    Unit x;
    x.c = u % a.NC;
    const int bh = u / a.NC;
    x.b = bh / a.Hv;
    x.h = bh - x.b * a.Hv;
    x.hq = x.h / (a.Hv / a.Hqk);
    x.t0 = x.c * C;
    x.n = min(C, a.T - x.t0);
    x.rowq = ((size_t)x.b * a.T + x.t0) * a.Hqk + x.hq;
    x.rowv = ((size_t)x.b * a.T + x.t0) * a.Hv + x.h;
    return x;
}
// Element e (a multiple of 4) of a row-major C x D array: token row and column.
template <int D>
__device__ __forceinline__ void rc(int l, int &e, int &t, int &d, int tid) {
    e = 4 * (l * NT + tid);
    t = e / D;
    d = e - t * D;
}
template <int D>
__device__ __forceinline__ void rc(int l, int &e, int &t, int &d) {
    rc<D>(l, e, t, d, (int)threadIdx.x);
}

// Workgroup barrier ordering shared-memory accesses only: it does not wait
// for global loads in flight (the prefetch of the next chunk or unit) or for
// global stores, which no other thread of the same launch reads back.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Blocked solves on the matrix cores. The 64 x 64 unit triangular system
// splits into 16 x 16 blocks: the diagonal blocks are inverted first (one
// wave), then each wave carries 16-column tiles of the right-hand side
// through block substitution, X_b = L_b (R_b - sum_c M_bc X_c), with the
// products on v_mfma_f32_16x16x4_f32. A tile lives in registers in the
// accumulator layout (lane l: rows 4 (l / 16) + r of column l % 16 of each
// 16-row block), and each product takes its k index in the order 4 (l / 16)
// + i at step i, so a lane's accumulator rows are exactly the B operand it
// supplies and its A operand is one 16-byte read.
constexpr int LTT = C + 4;  // row stride of the negated 64 x 64 triangle in shared memory
constexpr int LL = 16 + 4;  // row stride of the inverted 16 x 16 diagonal blocks
constexpr int kSolveFloats = C * LTT + C * LL;

// Wave-wide: lane (b, j) = (l / 16, l % 16) forms column j of
// (I + T_bb)^-1 by forward substitution, with nt(i, k) = -T_ik for rows and
// columns of the 64 x 64 matrix, and writes it to L[(16 b + i) LL + j]
// (row-major blocks) or, TRANS, to L[(16 b + j) LL + i] (the transposes).
template <bool TRANS, typename F>
__device__ __forceinline__ void invert_diag16(F nt, float *L) {
    const int l = threadIdx.x & 63, b = l >> 4, j = l & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float acc = i == j ? 1.f : 0.f;
#pragma unroll
        for (int k = 0; k < i; ++k) acc = fmaf(nt(16 * b + i, 16 * b + k), x[k], acc);
        x[i] = acc;
        if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bounds the entries held in registers
    }
    if (TRANS) {
#pragma unroll
        for (int i = 0; i < 16; i += 4) *reinterpret_cast<f32x4 *>(L + (16 * b + j) * LL + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) L[(16 * b + i) * LL + j] = x[i];
    }
}

// One 64 x 16 tile x (registers, accumulator layout, the right-hand side on
// entry) through the block substitution: UP = false solves (I + T) X = R
// from the first block (M = -T, L = the inverted diagonal blocks, both
// row-major); UP = true solves (I + T)^T X = R from the last block (M = -T^T,
// L = the transposed inverted blocks).
template <bool UP>
__device__ __forceinline__ void block_solve(f32x4 (&x)[4], const float *M, const float *L) {
    const int l = threadIdx.x & 63, row = l & 15, g = l >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int b = UP ? 3 - s : s;
        f32x4 w = x[b];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (UP ? c <= b : c >= b) continue;
            const f32x4 t = *reinterpret_cast<const f32x4 *>(M + (16 * b + row) * LTT + 16 * c + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) w = __builtin_amdgcn_mfma_f32_16x16x4f32(t[i], x[c][i], w, 0, 0, 0);
        }
        const f32x4 li = *reinterpret_cast<const f32x4 *>(L + (16 * b + row) * LL + 4 * g);
        f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) y = __builtin_amdgcn_mfma_f32_16x16x4f32(li[i], w[i], y, 0, 0, 0);
        x[b] = y;
        __builtin_amdgcn_sched_barrier(0);  // one block at a time: bounds the operands held in registers
    }
}

template <int D>
constexpr size_t prep_smem() {
    constexpr size_t LD = D + 4, R0 = C * LD > (size_t)kSolveFloats ? C * LD : kSolveFloats;
    return (R0 + 3 * C * LD + C + kBwdDecRows * D + 4) * 4;
}
template <int D>
constexpr size_t fsweep_smem() {
    return ((size_t)D * LB + (size_t)C * LB + (size_t)D * LT + (size_t)D * LC + D) * 4;
}
template <int D>
constexpr size_t bsweep_full_smem() {
    return ((size_t)D * LB + 2 * (size_t)C * LB + (size_t)C * LT + 3 * (size_t)D * LC + D) * 4;
}
template <int D>
constexpr size_t bsweep_rhs_smem() {
    return ((size_t)D * LB + (size_t)C * LB + 2 * (size_t)D * LC + D) * 4;
}
template <int D>
constexpr size_t rhs_smem() {
    return (2 * (size_t)D * LC + (size_t)C * LC + (size_t)C * (D + 16)) * 4;
}
template <int D>
constexpr size_t grad_s_smem() {
    constexpr size_t LD = D + 4, R0 = kSolveFloats > 32 * LD ? kSolveFloats : 32 * LD;
    return (R0 + 3 * C * LD + 32 * LD) * 4;
}
template <int D>
constexpr size_t grad_out_smem() {
    return (3 * (size_t)C * (D + 4) + 2 * (size_t)C * LC + 2 * C + 2 * 32 * C + 2048 + D) * 4;
}

// ---------------------------------------------------------------------------
// 1. Per chunk unit: G, E~, Q~, Kend, Gamma, T, A, then [Y | U_z].
template <typename IO, int D, bool CHAN, bool BW>
__global__ __launch_bounds__(NT) void cb_prep(ChunkBwdArgs a) {
    constexpr int LD = Cfg<D>::LD, NL = Cfg<D>::NL, R0 = C * LD > kSolveFloats ? C * LD : kSolveFloats;
    extern __shared__ __align__(16) float smem[];
    float *sQ = smem;           // q (Q~ with a per-channel decay); then -T (row stride LTT) and the inverted blocks
    float *sK = sQ + R0;        // k (K~)
    float *sE = sK + C * LD;    // e, then E~, then Y
    float *sZ = sE + C * LD;    // per-channel decay: g, then Gb; then z, then U_z
    float *sGs = sZ + C * LD;   // scalar decay: G per token
    float *sF = sGs + C;        // per-channel decay: the factor table (kBwdDecRows rows of D)
    int *sSlow = reinterpret_cast<int *>(sF + kBwdDecRows * D);  // bit b: block b formed entry by entry
    const int tid0 = threadIdx.x, units = a.B * a.Hv * a.NC;
    // The workgroups are persistent: each takes units blockIdx.x, + gridDim.x,
    // ..., and fetches the next one's inputs into registers once the current
    // ones are staged in shared memory (before the solve), so that the input
    // loads overlap the solve instead of stalling every workgroup at its start.
    // The fetched values stay in the io type until they are staged.
    using R4 = typename Raw4<IO>::type;
    R4 rq[NL], rk[NL], rb[BW ? NL : 1], rw[BW ? NL : 1], rv[NL];
    f32x4 rg[CHAN ? NL : 1];
    float rbeta[BW ? 1 : NL];
    const auto fetch = [&](int u, int tid) {
        const Unit x = decode(a, u);
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d, tid);
            rq[l] = rk[l] = rv[l] = R4{};
            if (BW) rb[l] = rw[l] = R4{};
            else rbeta[l] = 0.f;
            if (CHAN) rg[l] = zero4();
            if (t < x.n) {
                const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + d, iv = (x.rowv + (size_t)t * a.Hv) * D + d;
                rq[l] = Raw4<IO>::load(static_cast<const IO *>(a.q) + iq);
                rk[l] = Raw4<IO>::load(static_cast<const IO *>(a.k) + iq);
                rv[l] = Raw4<IO>::load(static_cast<const IO *>(a.v) + iv);
                if (BW) {
                    rb[l] = Raw4<IO>::load(static_cast<const IO *>(a.bg) + iv);
                    rw[l] = Raw4<IO>::load(static_cast<const IO *>(a.wg) + iv);
                } else {
                    rbeta[l] = a.beta[x.rowv + (size_t)t * a.Hv];
                }
                if (CHAN) rg[l] = lds4(a.g + iv);
            }
        }
    };
    // (With fp32 io the fetched values would not fit in registers beside the
    // solve's; each unit then fetches its own inputs at its start.)
    constexpr bool PREF = sizeof(IO) == 2;
    if (PREF && (int)blockIdx.x < units) fetch(blockIdx.x, tid0);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        // The thread index passes through an empty asm statement each
        // iteration, so that the many index computations derived from it are
        // redone per unit rather than held in registers across the loop.
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int un = u + (int)gridDim.x;  // the unit fetched during this one
        const Unit x = decode(a, u);
        const size_t ucd = (size_t)u * C * D;
        if (CHAN && tid == 0) *sSlow = 0;
        if (!PREF) fetch(u, tid);
        {
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                int e, t, d;
                rc<D>(l, e, t, d, tid);
                const f32x4 k4 = Raw4<IO>::widen(rk[l]);
                sts4(sQ + t * LD + d, Raw4<IO>::widen(rq[l]));
                sts4(sK + t * LD + d, k4);
                sts4(sE + t * LD + d, (BW ? Raw4<IO>::widen(rb[BW ? l : 0]) : splat(rbeta[BW ? 0 : l])) * k4);
                if (CHAN) sts4(sZ + t * LD + d, rg[CHAN ? l : 0]);
            }
        }
        if (!CHAN && tid < C) sGs[tid] = a.g && tid < x.n ? a.g[x.rowv + (size_t)tid * a.Hv] : 0.f;
        lds_barrier();
        if (CHAN) {
            if (tid < D) {  // per channel: the column into registers, summed per block, written back
                float gc[C];
#pragma unroll
                for (int t = 0; t < C; ++t) gc[t] = sZ[t * LD + tid];
#pragma unroll
                for (int t = 1; t < C; ++t)
                    if (t % 16) gc[t] += gc[t - 1];
#pragma unroll
                for (int t = 0; t < C; ++t) sZ[t * LD + tid] = gc[t];
                const float B0 = gc[15], B1 = gc[31], B2 = gc[47], B3 = gc[63], Bs[4] = {B0, B1, B2, B3};
                const float R[5] = {0.f, B0, B0 + B1, B0 + B1 + B2, B0 + B1 + B2 + B3};
                float *f = sF + tid;
                int bits = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f[b * D] = expf(R[b]);
                    f[(7 + b) * D] = expf(fminf(-Bs[b], kBwdDiagRange));
                    f[(11 + b) * D] = expf(R[4] - R[b + 1]);
                    bits |= Bs[b] < -kBwdDiagRange ? 1 << b : 0;
                }
                f[4 * D] = expf(B1);
                f[5 * D] = expf(B2);
                f[6 * D] = expf(B1 + B2);
                a.wGam[(size_t)u * D + tid] = expf(R[4]);
                if (bits) atomicOr(sSlow, bits);
            }
        } else if (tid < 64) {
            float G = sGs[tid];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(G, off);
                if (tid >= off) G += y;
            }
            sGs[tid] = G;
        }
        lds_barrier();

        float *wG = a.wG + ucd;  // [C][D] per-channel decay (Gb), [C] scalar (G)
        if (CHAN)  // Q^, K^, E^ in place of q, k, e
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                int e, t, d;
                rc<D>(l, e, t, d, tid);
                const f32x4 Gb = lds4(sZ + t * LD + d), Bb = lds4(sZ + (t | 15) * LD + d), eg = exp4(Gb);
                sts4(wG + e, Gb);
                sts4(sQ + t * LD + d, lds4(sQ + t * LD + d) * eg);
                sts4(sK + t * LD + d, lds4(sK + t * LD + d) * exp4(Bb - Gb));
                sts4(sE + t * LD + d, lds4(sE + t * LD + d) * eg);
            }
        if (!CHAN && tid < C) wG[tid] = sGs[tid];
        if (!CHAN && tid < D) a.wGam[(size_t)u * D + tid] = expf(sGs[C - 1]);
        lds_barrier();
        // Q~^T and Kend^T (row = channel), which the sweeps over chunks read.
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, dd, t;
            rc<C>(l, e, dd, t, tid);
            f32x4 qv, kv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                qv[r] = sQ[(t + r) * LD + dd];
                kv[r] = sK[(t + r) * LD + dd];
            }
            if (CHAN) {  // Q~ = Q^ exp(R_b), Kend = K^ exp(G_end - R_{b+1}); the 4 tokens share block b
                qv *= sF[(t >> 4) * D + dd];
                kv *= sF[(11 + (t >> 4)) * D + dd];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    qv[r] *= expf(sGs[t + r]);
                    kv[r] *= expf(sGs[C - 1] - sGs[t + r]);
                }
            }
            stg4(a.wQt + ucd + e, qv);
            stg4(a.wKet + ucd + e, kv);
        }

        // T and A on the matrix cores: the ten 16 x 16 tiles (bi, bj) on and
        // below the block diagonal, T = E^ diag(f) K^T and A = Q^ diag(f) K^T
        // with the tile's per-channel factor f (none with a scalar decay,
        // whose factor exp(G_t - G_j) is applied per entry, or next to the
        // diagonal). Wave w takes tile w and, for w < 2, tile w + 8. Each
        // product takes its k index in the order 4 (l / 16) + i at step i,
        // so that a lane's operands are 16-byte reads.
        {
            const int w = tid >> 6, l = tid & 63, lr = l & 15, g = l >> 4;
            const int slow = CHAN ? *sSlow : 0;  // diagonal blocks formed entry by entry below
            f32x4 tT[2];                         // this lane's T entries of its tiles, for -T after the barrier
            int tb[2];                           // the tiles' (bi, bj) as 4 bi + bj, or -1
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tile = w + 8 * q;
                const int bi = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3, bj = tile - bi * (bi + 1) / 2;
                tb[q] = tile < 10 && !(bi == bj && ((slow >> bi) & 1)) ? 4 * bi + bj : -1;
                if (tb[q] < 0) continue;
                const float *fk = !CHAN || bi - bj == 1 ? nullptr
                                  : sF + (bi == bj ? 7 + bi : bwd_row_far(bi, bj)) * D + 4 * g;
                const float *pe = sE + (16 * bi + lr) * LD + 4 * g, *pq = sQ + (16 * bi + lr) * LD + 4 * g;
                const float *pk = sK + (16 * bj + lr) * LD + 4 * g;
                f32x4 at = zero4(), aa = zero4();
#pragma unroll 4
                for (int kb = 0; kb < D; kb += 16) {
                    const f32x4 e4 = lds4(pe + kb), q4 = lds4(pq + kb);
                    const f32x4 k4 = fk ? lds4(pk + kb) * lds4(fk + kb) : lds4(pk + kb);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        at = __builtin_amdgcn_mfma_f32_16x16x4f32(e4[i], k4[i], at, 0, 0, 0);
                        aa = __builtin_amdgcn_mfma_f32_16x16x4f32(q4[i], k4[i], aa, 0, 0, 0);
                    }
                }
                const int j = 16 * bj + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * bi + 4 * g + r;
                    const float f = !CHAN && j <= t ? expf(sGs[t] - sGs[j]) : 1.f;
                    tT[q][r] = j < t ? at[r] * f : 0.f;
                    const size_t o = (size_t)u * C * C + (size_t)t * C + j;
                    a.wT[o] = tT[q][r];
                    a.wA[o] = j <= t ? aa[r] * f : 0.f;
                }
            }
            // The six tiles above the block diagonal are zero: rows 0-15 from
            // column 16 on (12 groups of 4 per row), rows 16-31 from column 32
            // (8), rows 32-47 from column 48 (4); 384 groups per matrix.
            for (int i = tid; i < 2 * 384; i += NT) {
                const int k = i % 384;
                const int t = k < 192 ? k / 12 : k < 320 ? 16 + (k - 192) / 8 : 32 + (k - 320) / 4;
                const int j = 4 * (k < 192 ? 4 + k % 12 : k < 320 ? 8 + (k - 192) % 8 : 12 + (k - 320) % 4);
                sts4((i < 384 ? a.wT : a.wA) + (size_t)u * C * C + (size_t)t * C + j, zero4());
            }
            // A strongly decaying diagonal block, entry by entry from the
            // inputs: sum_c e_tc k_jc exp(Gb_tc - Gb_jc) (the same for q).
            // Thread = 2 x 4 block of rows r0.., columns c0.. of the block.
            float sT8[2][4];
            bool sOwn = false;
            const int r0 = (tid >> 4) * 2, c0 = (tid & 15) * 4;
            if (CHAN && slow) {
                const int bi = r0 >> 4, bj = c0 >> 4;
                if (bi == bj && ((slow >> bi) & 1)) {
                    sOwn = true;
                    float aT[2][4], aA[2][4];
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) aT[i][j] = aA[i][j] = 0.f;
                    if (c0 <= r0 + 1)
                        for (int d = 0; d < D; d += 4) {
                            f32x4 e4[2], q4[2], k4[4], g4[2], h4[4];
#pragma unroll
                            for (int i = 0; i < 2; ++i) {
                                const int t = r0 + i;
                                const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + d, iv = (x.rowv + (size_t)t * a.Hv) * D + d;
                                q4[i] = t < x.n ? ld4io<IO>(a.q, iq) : zero4();
                                e4[i] = t < x.n ? ld4io<IO>(a.k, iq) *
                                                      (BW ? ld4io<IO>(a.bg, iv) : splat(a.beta[x.rowv + (size_t)t * a.Hv]))
                                                : zero4();
                                g4[i] = lds4(sZ + t * LD + d);
                            }
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int t = c0 + j;
                                k4[j] = t < x.n ? ld4io<IO>(a.k, (x.rowq + (size_t)t * a.Hqk) * D + d) : zero4();
                                h4[j] = lds4(sZ + t * LD + d);
                            }
#pragma unroll
                            for (int i = 0; i < 2; ++i)
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    f32x4 kf;
#pragma unroll
                                    for (int r = 0; r < 4; ++r) kf[r] = k4[j][r] * expf(fminf(g4[i][r] - h4[j][r], 0.f));
                                    aT[i][j] = dot4(e4[i], kf, aT[i][j]);
                                    aA[i][j] = dot4(q4[i], kf, aA[i][j]);
                                }
                        }
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int t = r0 + i;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            sT8[i][j] = c0 + j < t ? aT[i][j] : 0.f;
                            aA[i][j] = c0 + j <= t ? aA[i][j] : 0.f;
                        }
                        const size_t o = (size_t)u * C * C + (size_t)t * C + c0;
                        stg4(a.wT + o, f32x4{sT8[i][0], sT8[i][1], sT8[i][2], sT8[i][3]});
                        stg4(a.wA + o, f32x4{aA[i][0], aA[i][1], aA[i][2], aA[i][3]});
                    }
                }
            }
            lds_barrier();  // q, k and e tiles read: -T goes where q was
#pragma unroll
            for (int q = 0; q < 2; ++q)
                if (tb[q] >= 0) {
                    const int bi = tb[q] >> 2, bj = tb[q] & 3;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sQ[(16 * bi + 4 * g + r) * LTT + 16 * bj + lr] = -tT[q][r];
                }
            if (sOwn)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    sts4(sQ + (r0 + i) * LTT + c0, -f32x4{sT8[i][0], sT8[i][1], sT8[i][2], sT8[i][3]});
        }
        // Right-hand sides: E~ (scalar decay: the raw e scaled by exp(G_t); per
        // channel: E^ scaled by exp(R_b)) and z.
        {
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                int e, t, d;
                rc<D>(l, e, t, d, tid);
                sts4(sZ + t * LD + d, (BW ? Raw4<IO>::widen(rw[BW ? l : 0]) : splat(rbeta[BW ? 0 : l])) * Raw4<IO>::widen(rv[l]));
                if (!CHAN) sts4(sE + t * LD + d, lds4(sE + t * LD + d) * expf(sGs[t]));
                else sts4(sE + t * LD + d, lds4(sE + t * LD + d) * lds4(sF + (t >> 4) * D + d));
            }
            if (PREF && un < units) fetch(un, tid);
        }
        lds_barrier();
        // (I + T) X = [E~ | Z] by blocks: the inverted diagonal blocks (wave
        // 0), then 16-column tiles of E~ and Z, each carried by one wave.
        float *sL = sQ + C * LTT;
        if (tid < 64) invert_diag16<false>([&](int i, int k) { return sQ[i * LTT + k]; }, sL);
        lds_barrier();
        {
            constexpr int NTI = D / 8, NQ = (NTI + 7) / 8;  // tiles of [E~ | Z]; per wave
            const int w = tid >> 6, l = tid & 63;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int tl = w + 8 * q;
                if (tl < NTI) {
                    float *X = (tl < D / 16 ? sE + 16 * tl : sZ + 16 * (tl - D / 16)) + (l & 15) + 4 * (l >> 4) * LD;
                    f32x4 xt[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) xt[b][r] = X[(16 * b + r) * LD];
                    block_solve<false>(xt, sQ, sL);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int r = 0; r < 4; ++r) X[(16 * b + r) * LD] = xt[b][r];
                }
            }
        }
        lds_barrier();
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d, tid);
            stg4(a.wUz + ucd + e, lds4(sZ + t * LD + d));
        }
#pragma unroll
        for (int l = 0; l < NL; ++l) {  // Y^T
            int e, dd, t;
            rc<C>(l, e, dd, t, tid);
            stg4(a.wYt + ucd + e, f32x4{sE[t * LD + dd], sE[(t + 1) * LD + dd], sE[(t + 2) * LD + dd], sE[(t + 3) * LD + dd]});
        }
        lds_barrier();  // shared memory read; the next unit overwrites it
    }
}

// ---------------------------------------------------------------------------
// Sweeps over chunks. A workgroup owns (sequence, V head, 32 value columns);
// each chunk's operands are fetched into registers one chunk ahead (the
// whole workgroup together) and moved to shared memory at the start of the
// chunk, so that the loop reads its operands from shared memory.

// Products in the sweeps run on the matrix cores (fp32 in, fp32
// accumulate), one 16 x 16 output tile per wave at a time: a lane holds rows
// 4 (l / 16) + r, r < 4, of column l % 16 of the tile. mfma_kloop adds
// A[16 x K] B[K x 16] with A row-major (row stride lda) and B row-major
// (row stride ldb); K a multiple of 4.
// Two accumulators over alternate K steps keep two independent chains in
// flight; they are added at the end.
template <int K>
__device__ __forceinline__ f32x4 mfma_kloop(f32x4 acc, const float *A, int lda, const float *B, int ldb) {
    const int l = threadIdx.x & 63;
    const float *pa = A + (l & 15) * lda + (l >> 4), *pb = B + (l >> 4) * ldb + (l & 15);
    f32x4 acc2 = zero4();
#pragma unroll 8
    for (int k = 0; k < K; k += 8) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k], pb[k * ldb], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k + 4], pb[(k + 4) * ldb], acc2, 0, 0, 0);
    }
    return acc + acc2;
}

// The same with A given transposed: A[row][k] at At[k * ldat + row].
template <int K>
__device__ __forceinline__ f32x4 mfma_kloop_at(f32x4 acc, const float *At, int ldat, const float *B, int ldb) {
    const int l = threadIdx.x & 63;
    const float *pa = At + (l >> 4) * ldat + (l & 15), *pb = B + (l >> 4) * ldb + (l & 15);
    f32x4 acc2 = zero4();
#pragma unroll 8
    for (int k = 0; k < K; k += 8) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k * ldat], pb[k * ldb], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[(k + 4) * ldat], pb[(k + 4) * ldb], acc2, 0, 0, 0);
    }
    return acc + acc2;
}

// The same as accumulation over k in [K0, K1) into two chains (acc over k =
// K0, K0 + 8, ...; acc2 over k = K0 + 4, ...), so that a product can be split
// into pieces with other work between them; the pieces of mfma_kloop's
// range in order give its sums exactly.
template <int K0, int K1>
__device__ __forceinline__ void mfma_krange(f32x4 &acc, f32x4 &acc2, const float *A, int lda, const float *B,
                                            int ldb) {
    const int l = threadIdx.x & 63;
    const float *pa = A + (l & 15) * lda + (l >> 4), *pb = B + (l >> 4) * ldb + (l & 15);
#pragma unroll
    for (int k = K0; k < K1; k += 8) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k], pb[k * ldb], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k + 4], pb[(k + 4) * ldb], acc2, 0, 0, 0);
    }
}
template <int K0, int K1>
__device__ __forceinline__ void mfma_krange_at(f32x4 &acc, f32x4 &acc2, const float *At, int ldat, const float *B,
                                               int ldb) {
    const int l = threadIdx.x & 63;
    const float *pa = At + (l >> 4) * ldat + (l & 15), *pb = B + (l >> 4) * ldb + (l & 15);
#pragma unroll
    for (int k = K0; k < K1; k += 8) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k * ldat], pb[k * ldb], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[(k + 4) * ldat], pb[(k + 4) * ldb], acc2, 0, 0, 0);
    }
}

// f(integral_constant<I>) for I = I0 .. I1 - 1, in order.
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I0 < I1) {
        f(std::integral_constant<int, I0>{});
        static_for<I0 + 1, I1>(f);
    }
}

// 1b. Per chunk unit, the parts of the backward sweep's step that do not
//     depend on dL/dS: p = s A^T dO and b = s P^T dO with P = Q~ - A Y. Then
//     dU = p + Kend dS_next and dS = Diag(Gamma) dS_next + b - Y^T Kend dS_next,
//     since s Q~^T dO - Y^T (s A^T dO) = s (Q~ - A Y)^T dO. The products run
//     on the matrix cores in 16 x 16 tiles, wave w taking tiles w, w + 8, ...
//     p goes to wP ([units][C][D]) and b to wB ([units][D][D]).
template <typename IO, int D>
__global__ __launch_bounds__(NT) void cb_rhs(ChunkBwdArgs a) {
    constexpr int NL = Cfg<D>::NL, NTT = C * C / (4 * NT), LO = D + 16, NQT = (D / 4 + 7) / 8;
    extern __shared__ __align__(16) float smem[];
    float *sYn = smem;          // -Y^T [D][LC]
    float *sAt = sYn + D * LC;  // A^T [C][LC]
    float *sPt = sAt + C * LC;  // P^T [D][LC]
    float *sO = sPt + D * LC;   // dO [C][LO]
    const int tid = threadIdx.x, u = blockIdx.x, w = tid >> 6, l = tid & 63;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C, udd = (size_t)u * D * D;
    f32x4 qacc[NQT];  // this lane's Q~^T entries of its P^T tiles, loaded with the other operands
    {
        f32x4 rY[NL], rO[NL], rA[NTT];
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            int e, t, d;
            rc<D>(l2, e, t, d);
            rY[l2] = lds4(a.wYt + ucd + e);
            rO[l2] = t < x.n ? ld4io<IO>(a.dO, (x.rowv + (size_t)t * a.Hv) * D + d) : zero4();
        }
#pragma unroll
        for (int l2 = 0; l2 < NTT; ++l2) rA[l2] = lds4(a.wA + ucc + 4 * (l2 * NT + tid));
#pragma unroll
        for (int q = 0; q < NQT; ++q) {
            const int tile = w + 8 * q, rt = tile >> 2, ct = tile & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                qacc[q][r] = tile < D / 4 ? a.wQt[ucd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * C + ct * 16 + (l & 15)] : 0.f;
        }
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            int e, dd, t;
            rc<C>(l2, e, dd, t);
            sts4(sYn + dd * LC + t, -rY[l2]);
            rc<D>(l2, e, t, dd);
            sts4(sO + t * LO + dd, rO[l2]);
        }
#pragma unroll
        for (int l2 = 0; l2 < NTT; ++l2) {  // A^T
            const int e = 4 * (l2 * NT + tid), t = e / C, j = e - t * C;
#pragma unroll
            for (int r = 0; r < 4; ++r) sAt[(j + r) * LC + t] = rA[l2][r];
        }
    }
    lds_barrier();
    // The products in 16 x 16 tiles, wave w taking tiles w, w + 8, ...
    // P^T = Q~^T - Y^T A^T: (D / 16) x 4 tiles; Q~^T enters as the accumulator.
#pragma unroll
    for (int q = 0; q < NQT; ++q) {
        const int tile = w + 8 * q, rt = tile >> 2, ct = tile & 3;
        if (tile < D / 4) {
            const f32x4 acc = mfma_kloop<C>(qacc[q], sYn + rt * 16 * LC, LC, sAt + ct * 16, LC);
#pragma unroll
            for (int r = 0; r < 4; ++r) sPt[(rt * 16 + 4 * (l >> 4) + r) * LC + ct * 16 + (l & 15)] = acc[r];
        }
    }
    // p = s A^T dO: 4 x (D / 16) tiles.
    for (int tile = w; tile < D / 4; tile += 8) {
        const int rt = tile / (D / 16), ct = tile % (D / 16);
        const f32x4 acc = mfma_kloop<C>(zero4(), sAt + rt * 16 * LC, LC, sO + ct * 16, LO);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            a.wP[ucd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * D + ct * 16 + (l & 15)] = a.scale * acc[r];
    }
    lds_barrier();
    // b = s P^T dO: (D / 16) x (D / 16) tiles.
    for (int tile = w; tile < D * D / 256; tile += 8) {
        const int rt = tile / (D / 16), ct = tile % (D / 16);
        const f32x4 acc = mfma_kloop<C>(zero4(), sPt + rt * 16 * LC, LC, sO + ct * 16, LO);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            a.wB[udd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * D + ct * 16 + (l & 15)] = a.scale * acc[r];
    }
}

// 2a. Forward over chunks: the state entering each chunk, and U = U_z - Y S.
//    Wave w: U tile (rows 16 (w / 2), columns 16 (w % 2)); state tiles w and
//    w + 8 of the (D / 16) x 2 tiles of the state.
template <int D>
__device__ __forceinline__ void fsweep(const ChunkBwdArgs &a, float *smem, int item) {
    using K = SwCfg<D>;
    constexpr int NTL = K::NTL, NL = K::NL, NST = D / 16 * 2;
    float *sS = smem, *sU = sS + D * LB, *sYt = sU + C * LB, *sKt = sYt + D * LT;  // Y^T [D][LT], Kend^T [D][LC]
    float *sGam = sKt + D * LC;
    const int tid = threadIdx.x, tile = item % NTL, bh = item / NTL, col0 = tile * BV;
    const int w = tid >> 6, l = tid & 63, rt = w >> 1, ct = w & 1;
    const size_t sb = (size_t)bh * D * D;
    for (int i = tid; i < D * BV / 4; i += NS) {
        const int d = 4 * i / BV, j = 4 * i - d * BV;
        sts4(sS + d * LB + j, a.S0 ? lds4(a.S0 + sb + (size_t)d * D + col0 + j) : zero4());
    }
    // The next chunk's operands, numbered -- Y^T (NL per thread), this
    // thread's 4 entries of U_z, Gamma (1), Kend^T (NL) -- and spread over
    // the current chunk's products as in the backward sweep.
    f32x4 pY[NL], pK[NL];
    float pZ[4], pg;
    constexpr int NLD = 2 * NL + 4 + 1;
    const auto load = [&](auto ic, int c) {
        constexpr int i = decltype(ic)::value;
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        if constexpr (i < NL) {
            pY[i] = lds4(a.wYt + ucd + 4 * (i * NS + tid));  // [D][C]
        } else if constexpr (i < NL + 4) {
            constexpr int r = i - NL;
            pZ[r] = a.wUz[ucd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * D + col0 + ct * 16 + (l & 15)];
        } else if constexpr (i == NL + 4) {
            pg = tid < D ? a.wGam[u * D + tid] : 0.f;
        } else {
            pK[i - (NL + 5)] = lds4(a.wKet + ucd + 4 * ((i - (NL + 5)) * NS + tid));  // [D][C]
        }
    };
    constexpr int NXT = NST > 8 ? 2 : 1;  // state tiles per wave
    constexpr int NG = D / 32 + C / 16;
    const auto spread = [&](auto gc, int c) {
        constexpr int g = decltype(gc)::value;
        __builtin_amdgcn_sched_barrier(0);
        static_for<g * NLD / NG, (g + 1) * NLD / NG>([&](auto ic) { load(ic, c); });
        __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, NLD>([&](auto ic) { load(ic, 0); });
    for (int c = 0; c < a.NC; ++c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        const int cn = c + 1 < a.NC ? c + 1 : c;  // the chunk fetched during this one (the last one's loads go unused)
        lds_barrier();  // the previous chunk is done with the operand tiles; S written
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            int e, d, t;
            rcs<C>(l2, e, d, t);
            sts4(sYt + d * LT + t, pY[l2]);
            sts4(sKt + d * LC + t, pK[l2]);
        }
        if (tid < D) sGam[tid] = pg;
        float uz[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) uz[r] = pZ[r];
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            stg4(a.wS + u * D * D + (size_t)d * D + col0 + j, lds4(sS + d * LB + j));
        }
        lds_barrier();
        {  // U = U_z - Y S
            f32x4 p0 = zero4(), p1 = zero4();
            static_for<0, D / 32>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                mfma_krange_at<32 * j, 32 * j + 32>(p0, p1, sYt + rt * 16, LT, sS + ct * 16, LB);
                spread(jc, cn);
            });
            const f32x4 p = p0 + p1;
            const int col = ct * 16 + (l & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * (l >> 4) + r;
                const float uv = uz[r] - p[r];
                sU[row * LB + col] = uv;
                a.wU[ucd + (size_t)row * D + col0 + col] = uv;
            }
        }
        lds_barrier();
        // S = Gamma . S + Kend^T U; a wave's tiles share their columns, so
        // each k step reads the U operand once for both.
        f32x4 sn[NXT];
        {
            const int sc = w & 1;
            const float *pb = sU + sc * 16 + (l >> 4) * LB + (l & 15);
            const float *pa[NXT];
            bool on[NXT];
            f32x4 acc[NXT][2];
#pragma unroll
            for (int q = 0; q < NXT; ++q) {
                on[q] = NST >= 8 * (q + 1) || w + 8 * q < NST;
                pa[q] = sKt + (((w + 8 * q) >> 1) * 16 + (l & 15)) * LC + (l >> 4);
                acc[q][0] = acc[q][1] = zero4();
            }
            static_for<0, C / 16>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
#pragma unroll
                for (int k = 16 * j; k < 16 * j + 16; k += 8) {
                    const float b0 = pb[k * LB], b1 = pb[(k + 4) * LB];
#pragma unroll
                    for (int q = 0; q < NXT; ++q)
                        if (on[q]) {
                            acc[q][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[q][k], b0, acc[q][0], 0, 0, 0);
                            acc[q][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[q][k + 4], b1, acc[q][1], 0, 0, 0);
                        }
                }
                spread(std::integral_constant<int, D / 32 + j>{}, cn);
            });
#pragma unroll
            for (int q = 0; q < NXT; ++q)
                if (on[q]) {
                    const int dt = (w + 8 * q) >> 1;
                    const f32x4 p = acc[q][0] + acc[q][1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = dt * 16 + 4 * (l >> 4) + r;
                        sn[q][r] = sGam[row] * sS[row * LB + sc * 16 + (l & 15)] + p[r];
                    }
                }
        }
        // No barrier: each wave rewrites only the state entries it has just
        // read, and every other read of S in this chunk was before the last one.
#pragma unroll
        for (int q = 0; q < NXT; ++q) {
            const int st = w + 8 * q, dt = st >> 1, sc = st & 1;
            if (NST >= 8 * (q + 1) || st < NST)
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[(dt * 16 + 4 * (l >> 4) + r) * LB + sc * 16 + (l & 15)] = sn[q][r];
        }
    }
}

// 2b. Backward over chunks for the same work items: X = dL/d(state leaving
//    the chunk), dU, and X for the chunk before. Tiles per wave as above.
//    Two forms: bsweep_full forms every product of the step itself (four
//    per chunk); bsweep_rhs takes the two that do not depend on X from
//    cb_rhs (two per chunk on the chain). The second pays when the sweep's
//    serial chain bounds the call (few sequences and heads, most compute
//    units idle); with enough work items to fill the GPU, cb_rhs's extra
//    pass over the units costs more than the sweep saves.
template <typename IO, int D>
__device__ __forceinline__ void bsweep_full(const ChunkBwdArgs &a, float *smem, int item) {
    using K = SwCfg<D>;
    constexpr int NTL = K::NTL, NL = K::NL, NST = D / 16 * 2;
    constexpr int NA = C * C / (4 * NS), NO = C * BV / (4 * NS);  // 4-element groups per thread: A, dO tile
    float *sX = smem, *sO = sX + D * LB, *sdU = sO + C * LB;
    float *sA = sdU + C * LB;    // A [C][LT]
    float *sKt = sA + C * LT;    // Kend^T [D][LC]
    float *sQt = sKt + D * LC;   // Q~^T [D][LC]
    float *sYt = sQt + D * LC;   // Y^T [D][LC]
    float *sGam = sYt + D * LC;  // [D]
    const int tid = threadIdx.x, tile = item % NTL, bh = item / NTL, col0 = tile * BV;
    const int w = tid >> 6, l = tid & 63, rt = w >> 1, ct = w & 1;
    const int b = bh / a.Hv, h = bh - b * a.Hv;
    const size_t sb = (size_t)bh * D * D;
    for (int i = tid; i < D * BV / 4; i += NS) {
        const int d = 4 * i / BV, j = 4 * i - d * BV;
        sts4(sX + d * LB + j, a.dST ? lds4(a.dST + sb + (size_t)d * D + col0 + j) : zero4());
    }
    // A chunk's operands, fetched by the whole workgroup one chunk ahead. The
    // loads are numbered -- Kend^T (NL per thread), A (NA), the dO tile (NO),
    // Gamma (1), Y^T (NL), Q~^T (NL) -- and spread over the pieces of the
    // current chunk's products, so that their latency overlaps the matrix
    // cores' work rather than stalling every wave at once.
    f32x4 pY[NL], pK[NL], pQ[NL], pA[NA], pO[NO];
    float pg;
    constexpr int NLD = 3 * NL + NA + NO + 1;
    const auto load = [&](auto ic, int c) {
        constexpr int i = decltype(ic)::value;
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        if constexpr (i < NL) {
            pK[i] = lds4(a.wKet + ucd + 4 * (i * NS + tid));  // [D][C]
        } else if constexpr (i < NL + NA) {
            pA[i - NL] = lds4(a.wA + u * C * C + 4 * ((i - NL) * NS + tid));
        } else if constexpr (i < NL + NA + NO) {
            const int t0 = c * C, n = min(C, a.T - t0);
            int e, t, j;
            rcs<BV>(i - NL - NA, e, t, j);
            pO[i - NL - NA] = t < n ? ld4io<IO>(a.dO, (((size_t)b * a.T + t0 + t) * a.Hv + h) * D + col0 + j) : zero4();
        } else if constexpr (i == NL + NA + NO) {
            pg = tid < D ? a.wGam[u * D + tid] : 0.f;
        } else if constexpr (i < 2 * NL + NA + NO + 1) {
            pY[i - (NL + NA + NO + 1)] = lds4(a.wYt + ucd + 4 * ((i - (NL + NA + NO + 1)) * NS + tid));  // [D][C]
        } else {
            pQ[i - (2 * NL + NA + NO + 1)] = lds4(a.wQt + ucd + 4 * ((i - (2 * NL + NA + NO + 1)) * NS + tid));  // [D][C]
        }
    };
    // The chunk's products run in NG pieces of 8 matrix instructions; after
    // piece g come loads [g NLD / NG, (g + 1) NLD / NG), fenced so that the
    // compiler keeps them there.
    constexpr int NXT = NST > 8 ? 2 : 1;  // X tiles per wave
    constexpr int NG = C / 32 + D / 32 + C / 16;
    const auto spread = [&](auto gc, int c) {
        constexpr int g = decltype(gc)::value;
        __builtin_amdgcn_sched_barrier(0);
        static_for<g * NLD / NG, (g + 1) * NLD / NG>([&](auto ic) { load(ic, c); });
        __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, NLD>([&](auto ic) { load(ic, a.NC - 1); });
    for (int c = a.NC - 1; c >= 0; --c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        const int cn = c > 0 ? c - 1 : 0;  // the chunk fetched during this one (at c = 0 the loads go unused)
        lds_barrier();  // X written; the previous chunk is done with the operand tiles
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            int e, d, t;
            rcs<C>(l2, e, d, t);
            sts4(sKt + d * LC + t, pK[l2]);
            sts4(sYt + d * LC + t, pY[l2]);
            sts4(sQt + d * LC + t, pQ[l2]);
        }
#pragma unroll
        for (int l2 = 0; l2 < NA; ++l2) {
            int e, t, j;
            rcs<C>(l2, e, t, j);
            sts4(sA + t * LT + j, pA[l2]);
        }
#pragma unroll
        for (int l2 = 0; l2 < NO; ++l2) {
            int e, t, j;
            rcs<BV>(l2, e, t, j);
            sts4(sO + t * LB + j, pO[l2]);
        }
        if (tid < D) sGam[tid] = pg;
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            stg4(a.wdS + u * D * D + (size_t)d * D + col0 + j, lds4(sX + d * LB + j));
        }
        lds_barrier();
        {  // dU = s A^T dO + Kend X
            f32x4 p0 = zero4(), p1 = zero4(), k0 = zero4(), k1 = zero4();
            static_for<0, C / 32>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                mfma_krange_at<32 * j, 32 * j + 32>(p0, p1, sA + rt * 16, LT, sO + ct * 16, LB);
                spread(std::integral_constant<int, j>{}, cn);
            });
            static_for<0, D / 32>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                mfma_krange_at<32 * j, 32 * j + 32>(k0, k1, sKt + rt * 16, LC, sX + ct * 16, LB);
                spread(std::integral_constant<int, C / 32 + j>{}, cn);
            });
            const f32x4 p = p0 + p1, k = k0 + k1;
            const int col = ct * 16 + (l & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * (l >> 4) + r;
                const float du = fmaf(a.scale, p[r], k[r]);
                sdU[row * LB + col] = du;
                a.wdU[ucd + (size_t)row * D + col0 + col] = du;
            }
        }
        lds_barrier();
        // X = Gamma . X + s Q~^T dO - Y^T dU. A wave's tiles share their
        // columns, so each k step reads the dO and dU operands once for both.
        f32x4 xn[NXT];
        {
            const int sc = w & 1;
            const float *pbq = sO + sc * 16 + (l >> 4) * LB + (l & 15), *pby = sdU + sc * 16 + (l >> 4) * LB + (l & 15);
            const float *paq[NXT], *pay[NXT];
            bool on[NXT];
            f32x4 aq[NXT][2], ay[NXT][2];
#pragma unroll
            for (int q = 0; q < NXT; ++q) {
                const int dt = (w + 8 * q) >> 1;
                on[q] = NST >= 8 * (q + 1) || w + 8 * q < NST;
                paq[q] = sQt + (dt * 16 + (l & 15)) * LC + (l >> 4);
                pay[q] = sYt + (dt * 16 + (l & 15)) * LC + (l >> 4);
                aq[q][0] = aq[q][1] = ay[q][0] = ay[q][1] = zero4();
            }
            static_for<0, C / 16>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
#pragma unroll
                for (int k = 16 * j; k < 16 * j + 16; k += 8) {
                    const float bq0 = pbq[k * LB], bq1 = pbq[(k + 4) * LB], by0 = pby[k * LB], by1 = pby[(k + 4) * LB];
#pragma unroll
                    for (int q = 0; q < NXT; ++q)
                        if (on[q]) {
                            aq[q][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(paq[q][k], bq0, aq[q][0], 0, 0, 0);
                            aq[q][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(paq[q][k + 4], bq1, aq[q][1], 0, 0, 0);
                            ay[q][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(pay[q][k], by0, ay[q][0], 0, 0, 0);
                            ay[q][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(pay[q][k + 4], by1, ay[q][1], 0, 0, 0);
                        }
                }
                spread(std::integral_constant<int, C / 32 + D / 32 + j>{}, cn);
            });
#pragma unroll
            for (int q = 0; q < NXT; ++q)
                if (on[q]) {
                    const int dt = (w + 8 * q) >> 1;
                    const f32x4 pq = aq[q][0] + aq[q][1], py = ay[q][0] + ay[q][1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = dt * 16 + 4 * (l >> 4) + r;
                        xn[q][r] = sGam[row] * sX[row * LB + sc * 16 + (l & 15)] + a.scale * pq[r] - py[r];
                    }
                }
        }
        // No barrier: each wave rewrites only the entries of X it has just
        // read, and every other read of X in this chunk was before the last one.
#pragma unroll
        for (int q = 0; q < NXT; ++q) {
            const int st = w + 8 * q, dt = st >> 1, sc = st & 1;
            if (NST >= 8 * (q + 1) || st < NST)
#pragma unroll
                for (int r = 0; r < 4; ++r) sX[(dt * 16 + 4 * (l >> 4) + r) * LB + sc * 16 + (l & 15)] = xn[q][r];
        }
    }
    lds_barrier();
    if (a.dS0)
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            sts4(a.dS0 + sb + (size_t)d * D + col0 + j, lds4(sX + d * LB + j));
        }
}

// With p = s A^T dO and b = s P^T dO from cb_rhs, V = Kend X gives dU = p +
// V and the X of the chunk before, Gamma . X + b - Y^T V.
template <typename IO, int D>
__device__ __forceinline__ void bsweep_rhs(const ChunkBwdArgs &a, float *smem, int item) {
    using K = SwCfg<D>;
    constexpr int NTL = K::NTL, NL = K::NL, NST = D / 16 * 2;
    constexpr int NXT = NST > 8 ? 2 : 1;  // X tiles per wave
    float *sX = smem, *sV = sX + D * LB;  // X [D][LB]; V = Kend X [C][LB]
    float *sKt = sV + C * LB;             // Kend^T [D][LC]
    float *sYt = sKt + D * LC;            // Y^T [D][LC]
    float *sGam = sYt + D * LC;           // [D]
    const int tid = threadIdx.x, tile = item % NTL, bh = item / NTL, col0 = tile * BV;
    const int w = tid >> 6, l = tid & 63, rt = w >> 1, ct = w & 1, sc = w & 1;
    const size_t sb = (size_t)bh * D * D;
    bool on[NXT];
#pragma unroll
    for (int q = 0; q < NXT; ++q) on[q] = NST >= 8 * (q + 1) || w + 8 * q < NST;
    for (int i = tid; i < D * BV / 4; i += NS) {
        const int d = 4 * i / BV, j = 4 * i - d * BV;
        sts4(sX + d * LB + j, a.dST ? lds4(a.dST + sb + (size_t)d * D + col0 + j) : zero4());
    }
    // A chunk's operands, fetched by the whole workgroup one chunk ahead. The
    // loads are numbered -- Kend^T (NL per thread), this lane's 4 entries of
    // p, its 4 entries of b per X tile, Gamma (1), Y^T (NL) -- and spread
    // over the pieces of the current chunk's products, so that their latency
    // overlaps the matrix cores' work rather than stalling every wave at once.
    f32x4 pY[NL], pK[NL], pP, pB[NXT];
    float pg;
    constexpr int NLD = 2 * NL + 4 + 4 * NXT + 1;
    const auto load = [&](auto ic, int c) {
        constexpr int i = decltype(ic)::value;
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        if constexpr (i < NL) {
            pK[i] = lds4(a.wKet + ucd + 4 * (i * NS + tid));  // [D][C]
        } else if constexpr (i < NL + 4) {
            constexpr int r = i - NL;
            pP[r] = a.wP[ucd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * D + col0 + ct * 16 + (l & 15)];
        } else if constexpr (i < NL + 4 + 4 * NXT) {
            constexpr int q = (i - NL - 4) / 4, r = (i - NL - 4) % 4;
            const int row = ((w + 8 * q) >> 1) * 16 + 4 * (l >> 4) + r;
            pB[q][r] = on[q] ? a.wB[u * D * D + (size_t)row * D + col0 + sc * 16 + (l & 15)] : 0.f;
        } else if constexpr (i == NL + 4 + 4 * NXT) {
            pg = tid < D ? a.wGam[u * D + tid] : 0.f;
        } else {
            pY[i - (NL + 5 + 4 * NXT)] = lds4(a.wYt + ucd + 4 * ((i - (NL + 5 + 4 * NXT)) * NS + tid));  // [D][C]
        }
    };
    // The chunk's products run in NG pieces of 8 matrix instructions per
    // tile; after piece g come loads [g NLD / NG, (g + 1) NLD / NG), fenced so
    // that the compiler keeps them there.
    constexpr int NG = D / 32 + C / 16;
    const auto spread = [&](auto gc, int c) {
        constexpr int g = decltype(gc)::value;
        __builtin_amdgcn_sched_barrier(0);
        static_for<g * NLD / NG, (g + 1) * NLD / NG>([&](auto ic) { load(ic, c); });
        __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, NLD>([&](auto ic) { load(ic, a.NC - 1); });
    for (int c = a.NC - 1; c >= 0; --c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        const int cn = c > 0 ? c - 1 : 0;  // the chunk fetched during this one (at c = 0 the loads go unused)
        lds_barrier();  // X written; the previous chunk is done with the operand tiles
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            int e, d, t;
            rcs<C>(l2, e, d, t);
            sts4(sKt + d * LC + t, pK[l2]);
            sts4(sYt + d * LC + t, pY[l2]);
        }
        if (tid < D) sGam[tid] = pg;
        const f32x4 pv = pP;
        f32x4 bv[NXT];
#pragma unroll
        for (int q = 0; q < NXT; ++q) bv[q] = pB[q];
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            stg4(a.wdS + u * D * D + (size_t)d * D + col0 + j, lds4(sX + d * LB + j));
        }
        lds_barrier();
        {  // V = Kend X; dU = p + V
            f32x4 k0 = zero4(), k1 = zero4();
            static_for<0, D / 32>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                mfma_krange_at<32 * j, 32 * j + 32>(k0, k1, sKt + rt * 16, LC, sX + ct * 16, LB);
                spread(jc, cn);
            });
            const f32x4 k = k0 + k1;
            const int col = ct * 16 + (l & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * (l >> 4) + r;
                sV[row * LB + col] = k[r];
                a.wdU[ucd + (size_t)row * D + col0 + col] = pv[r] + k[r];
            }
        }
        lds_barrier();
        // X = Gamma . X + b - Y^T V. A wave's tiles share their columns, so
        // each k step reads the V operand once for both.
        f32x4 xn[NXT];
        {
            const float *pbv = sV + sc * 16 + (l >> 4) * LB + (l & 15);
            const float *pay[NXT];
            f32x4 ay[NXT][2];
#pragma unroll
            for (int q = 0; q < NXT; ++q) {
                pay[q] = sYt + (((w + 8 * q) >> 1) * 16 + (l & 15)) * LC + (l >> 4);
                ay[q][0] = ay[q][1] = zero4();
            }
            static_for<0, C / 16>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
#pragma unroll
                for (int k = 16 * j; k < 16 * j + 16; k += 8) {
                    const float b0 = pbv[k * LB], b1 = pbv[(k + 4) * LB];
#pragma unroll
                    for (int q = 0; q < NXT; ++q)
                        if (on[q]) {
                            ay[q][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(pay[q][k], b0, ay[q][0], 0, 0, 0);
                            ay[q][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(pay[q][k + 4], b1, ay[q][1], 0, 0, 0);
                        }
                }
                spread(std::integral_constant<int, D / 32 + j>{}, cn);
            });
#pragma unroll
            for (int q = 0; q < NXT; ++q)
                if (on[q]) {
                    const int dt = (w + 8 * q) >> 1;
                    const f32x4 py = ay[q][0] + ay[q][1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = dt * 16 + 4 * (l >> 4) + r;
                        xn[q][r] = sGam[row] * sX[row * LB + sc * 16 + (l & 15)] + bv[q][r] - py[r];
                    }
                }
        }
        // No barrier: each wave rewrites only the entries of X it has just
        // read, and every other read of X in this chunk was before the last one.
#pragma unroll
        for (int q = 0; q < NXT; ++q) {
            const int dt = (w + 8 * q) >> 1;
            if (on[q])
#pragma unroll
                for (int r = 0; r < 4; ++r) sX[(dt * 16 + 4 * (l >> 4) + r) * LB + sc * 16 + (l & 15)] = xn[q][r];
        }
    }
    lds_barrier();
    if (a.dS0)
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            sts4(a.dS0 + sb + (size_t)d * D + col0 + j, lds4(sX + d * LB + j));
        }
}

// The two sweeps do not depend on each other (the chain of dL/dS does not
// use the forward states), so one launch runs both: the backward sweep's
// workgroups first, then the forward sweep's, which fill the CUs the first
// set leaves free and then follow as workgroups finish. Each set has P
// workgroups (items rounded up to a multiple of 8); workgroups that share an
// XCD (block index mod 8) take consecutive work items, so that the value
// tiles of one head read its chunk factors through the same L2.
template <typename IO, int D, bool RHS>
__global__ __launch_bounds__(NS) void cb_sweeps(ChunkBwdArgs a, int items, int P) {
    extern __shared__ __align__(16) float smem[];
    const int x = (int)blockIdx.x, back = x < P, xl = back ? x : x - P;
    const int wi = (xl & 7) * (P >> 3) + (xl >> 3);
    if (wi >= items) return;
    if (!back) fsweep<D>(a, smem, wi);
    else if constexpr (RHS) bsweep_rhs<IO, D>(a, smem, wi);
    else bsweep_full<IO, D>(a, smem, wi);
}

// ---------------------------------------------------------------------------
// 3. Per unit: dR = L^T dU (solve (I + T)^T dR = dU), dT, dA, and the
//    products with S and dS_next.
template <typename IO, int D>
__global__ __launch_bounds__(NT) void cb_grad_s(ChunkBwdArgs a) {
    constexpr int LD = Cfg<D>::LD, NL = Cfg<D>::NL, R0 = kSolveFloats > 32 * LD ? kSolveFloats : 32 * LD;
    constexpr int NG = 32 * D / 4, NB = (NG + NT - 1) / NT, NTT = C * C / (4 * NT);  // 4-element groups: S block, T
    extern __shared__ __align__(16) float smem[];
    float *sT = smem;  // -T^T (row stride LTT) and the inverted blocks; later 32 rows of S
    float *sX = sT + R0, *sU = sX + C * LD, *sO = sU + C * LD, *sB = sO + C * LD;
    const int tid0 = threadIdx.x, units = a.B * a.Hv * a.NC;
    // Persistent, as cb_prep: each workgroup takes units blockIdx.x, +
    // gridDim.x, ..., and fetches the next unit's dU, U, dO and T into
    // registers (dO in the io type) while it works on the current one; the
    // barriers order shared memory only and do not wait for them. Each
    // unit's S and dS_next rows come in blocks of 32, the next block fetched
    // while the current one is used (the first block of the next unit during
    // the current unit's last).
    using R4 = typename Raw4<IO>::type;
    f32x4 rX[NL], rU[NL], rT[NTT];
    R4 rO[NL];
    const auto fetch_unit = [&](int u, int tid) {
        const Unit x = decode(a, u);
        const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d, tid);
            rX[l] = lds4(a.wdU + ucd + e);
            rU[l] = lds4(a.wU + ucd + e);
            rO[l] = t < x.n ? Raw4<IO>::load(static_cast<const IO *>(a.dO) + (x.rowv + (size_t)t * a.Hv) * D + d) : R4{};
        }
#pragma unroll
        for (int l = 0; l < NTT; ++l) rT[l] = lds4(a.wT + ucc + 4 * (l * NT + tid));
    };
    f32x4 rb[NB], rs[NB];
    const auto fetch = [&](int u, int blk, int tid) {
        const size_t udd = (size_t)u * D * D;
#pragma unroll
        for (int l = 0; l < NB; ++l) {
            const int g = l * NT + tid;
            if (g < NG) {
                rs[l] = lds4(a.wS + udd + (size_t)blk * 32 * D + 4 * g);
                rb[l] = lds4(a.wdS + udd + (size_t)blk * 32 * D + 4 * g);
            }
        }
    };
    if ((int)blockIdx.x < units) {
        fetch_unit(blockIdx.x, tid0);
        fetch(blockIdx.x, 0, tid0);
    }
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        int tid = tid0;  // redone per unit (see cb_prep)
        asm volatile("" : "+v"(tid));
        const int un = u + (int)gridDim.x;
        const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d, tid);
            sts4(sX + t * LD + d, rX[l]);
            sts4(sU + t * LD + d, rU[l]);
            sts4(sO + t * LD + d, Raw4<IO>::widen(rO[l]));
        }
#pragma unroll
        for (int l = 0; l < NTT; ++l) {  // -T^T
            const int e = 4 * (l * NT + tid), t = e / C, j = e - t * C;
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(j + r) * LTT + t] = -rT[l][r];
        }
        if (un < units) fetch_unit(un, tid);
        lds_barrier();
        // (I + T)^T dR = dU by blocks: the inverted diagonal blocks (wave 0), then
        // one 16-column tile of dU per wave.
        float *sL = sT + C * LTT;
        if (tid < 64) invert_diag16<true>([&](int i, int k) { return sT[k * LTT + i]; }, sL);
        lds_barrier();
        if ((tid >> 6) < D / 16) {
            const int l = tid & 63;
            float *X = sX + 16 * (tid >> 6) + (l & 15) + 4 * (l >> 4) * LD;
            f32x4 xt[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) xt[b][r] = X[(16 * b + r) * LD];
            block_solve<true>(xt, sT, sL);
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) X[(16 * b + r) * LD] = xt[b][r];
        }
        lds_barrier();
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d, tid);
            stg4(a.wdU + ucd + e, lds4(sX + t * LD + d));  // dR replaces dU
        }
        {
            // dT = -dR U^T (strictly lower) and dA = s dO U^T (lower) on the matrix
            // cores: the 16 x 16 tiles of the two 64 x 64 results, 2 per wave; a
            // tile above the diagonal is written as zeros.
            const int w = tid >> 6, l = tid & 63;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int tile = w + 8 * p, rt = tile >> 2, ct = tile & 3;
                f32x4 at = zero4(), aa = zero4();
                if (ct <= rt) {
                    const int ao = (rt * 16 + (l & 15)) * LD + (l >> 4), bo = (ct * 16 + (l & 15)) * LD + (l >> 4);
#pragma unroll 4
                    for (int v = 0; v < D; v += 4) {
                        const float bu = sU[bo + v];
                        at = __builtin_amdgcn_mfma_f32_16x16x4f32(sX[ao + v], bu, at, 0, 0, 0);
                        aa = __builtin_amdgcn_mfma_f32_16x16x4f32(sO[ao + v], bu, aa, 0, 0, 0);
                    }
                }
                const int j = ct * 16 + (l & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = rt * 16 + 4 * (l >> 4) + r;
                    a.wdT[ucc + (size_t)t * C + j] = j < t ? -at[r] : 0.f;
                    a.wdA[ucc + (size_t)t * C + j] = j <= t ? a.scale * aa[r] : 0.f;
                }
            }
        }
        // Products with S and with dS_next, 32 state rows at a time; the next
        // block's rows are fetched into registers while the current one is used.
        float *sB2 = sT;  // S rows of the block (T is no longer needed)
        for (int blk = 0; blk < D / 32; ++blk) {
            lds_barrier();  // the previous block's rows (and T) are read
#pragma unroll
            for (int l = 0; l < NB; ++l) {
                const int g = l * NT + tid, e = 4 * g, r = e / D, v = e - r * D;
                if (g < NG) {
                    sts4(sB2 + r * LD + v, rs[l]);
                    sts4(sB + r * LD + v, rb[l]);
                }
            }
            if (blk + 1 < D / 32) fetch(u, blk + 1, tid);
            else if (un < units) fetch(un, 0, tid);
            lds_barrier();
            {
                // The block's 64 x 32 outputs of each product on the matrix cores
                // (fp32 in, fp32 accumulate): wave w takes the 16 x 16 tile
                // (rows 16 (w / 2), columns 16 (w % 2)). A lane holds rows
                // 4 (l / 16) + r of column l % 16 of its tile.
                const int w = tid >> 6, l = tid & 63, rt = w >> 1, ct = w & 1;
                const int ao = (rt * 16 + (l & 15)) * LD + (l >> 4), bo = (ct * 16 + (l & 15)) * LD + (l >> 4);
                f32x4 ae = zero4(), aq = zero4(), ak = zero4();
#pragma unroll 4
                for (int v = 0; v < D; v += 4) {
                    const float bs = sB2[bo + v], bdv = sB[bo + v];
                    ae = __builtin_amdgcn_mfma_f32_16x16x4f32(sX[ao + v], bs, ae, 0, 0, 0);
                    aq = __builtin_amdgcn_mfma_f32_16x16x4f32(sO[ao + v], bs, aq, 0, 0, 0);
                    ak = __builtin_amdgcn_mfma_f32_16x16x4f32(sU[ao + v], bdv, ak, 0, 0, 0);
                }
                const int col = blk * 32 + ct * 16 + (l & 15);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const size_t o = ucd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * D + col;
                    a.wdE[o] = -ae[r];
                    a.wdQ[o] = a.scale * aq[r];
                    a.wdK[o] = ak[r];
                }
            }
            {  // dGamma of the block's 32 rows: TG consecutive threads per row, D / TG columns each
                constexpr int TG = D / 4 < 16 ? D / 4 : 16;
                const int r = tid / TG, c0 = (tid % TG) * (D / TG);
                float acc = 0.f;
                if (r < 32)
#pragma unroll
                    for (int v = 0; v < D / TG; v += 4)
                        acc = dot4(lds4(sB + r * LD + c0 + v), lds4(sB2 + r * LD + c0 + v), acc);
#pragma unroll
                for (int off = 1; off < TG; off <<= 1) acc += __shfl_xor(acc, off);
                if (r < 32 && tid % TG == 0) a.wdGam[(size_t)u * D + blk * 32 + r] = acc;
            }
        }
        lds_barrier();  // shared memory read; the next unit overwrites it
    }
}

// ---------------------------------------------------------------------------
// 4. Per unit: the parts through T and A, the exponential factors, the
//    gates, and dg.
template <typename IO, int D, bool CHAN, bool BW>
__global__ __launch_bounds__(NT) void cb_grad_out(ChunkBwdArgs a) {
    using K = Cfg<D>;
    constexpr int LD = K::LD, NL = K::NL, NCG = K::NCG, RT = K::RT, NRG = K::NRG, NTT = C * C / (4 * NT);
    extern __shared__ __align__(16) float smem[];
    float *sP1 = smem;            // e (E~): left factor of T; then X_e
    float *sP2 = sP1 + C * LD;    // k (K~): right factor of T and A; then X_q
    float *sP3 = sP2 + C * LD;    // q (Q~): left factor of A; then X_k
    float *sdT = sP3 + C * LD;    // dT, for a scalar decay times exp(G_t - G_j); then dG [C][LD]
    float *sdA = sdT + C * LC;
    // Reductions go through per-thread parts summed in a fixed order, so that
    // the result does not depend on the order threads arrive in.
    float *sRow = sdA + C * LC;    // [C] row sums of dT . T + dA . A (scalar decay)
    float *sColP = sRow + C;       // [32][C] their column sums by row group; later sTokG
    float *sTokG = sColP;          // [C][32] per-token dG parts of the column groups (scalar decay)
    float *sCol = sColP + 32 * C;  // [C]
    float *sTokB = sCol + C;       // [C][32] per-token dbeta parts (tied gates)
    float *sGeP = sTokB + 32 * C;  // [NRG][D] dG_end parts
    float *sGe = sGeP + 2048;      // [D] dG_end (scalar decay: element 0)
    float *sGt = sdT;
    // Per-channel decay, until the final pass: the tiles' factors (rows 0-2
    // exp(B_1), exp(B_2), exp(B_1 + B_2); rows 3-6 exp(-B_b), capped) and
    // each channel's bits of the blocks formed entry by entry, where the
    // column sums of a scalar decay go.
    float *sF = sColP;
    int *sBits = reinterpret_cast<int *>(sColP + 7 * D);
    static_assert(C * LD <= 2 * C * LC && NRG * D <= 2048 && NCG <= 32 && NT / 16 == 32 && 8 * D <= 32 * C,
                  "shared-memory layout");
    const int tid = threadIdx.x, u = blockIdx.x;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C;
    const float *wG = a.wG + ucd;
    const bool tied = !BW, grouped = a.Hv > a.Hqk;
    {
        f32x4 rq[NL], rk[NL], re[NL];
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            rq[l] = rk[l] = re[l] = zero4();
            if (t < x.n) {
                const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + d, iv = (x.rowv + (size_t)t * a.Hv) * D + d;
                rq[l] = ld4io<IO>(a.q, iq);
                rk[l] = ld4io<IO>(a.k, iq);
                re[l] = BW ? ld4io<IO>(a.bg, iv) : splat(a.beta[x.rowv + (size_t)t * a.Hv]);
            }
        }
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            f32x4 ev = re[l] * rk[l], kv = rk[l], qv = rq[l];
            if (CHAN) {  // E^, K^, Q^
                const f32x4 Gb = lds4(wG + e), Bb = lds4(wG + (t | 15) * D + d), eg = exp4(Gb);
                qv *= eg;
                ev *= eg;
                kv *= exp4(Bb - Gb);
            }
            sts4(sP1 + t * LD + d, ev);
            sts4(sP2 + t * LD + d, kv);
            sts4(sP3 + t * LD + d, qv);
        }
    }
    {
        // Thread: 4 consecutive columns j of rows t = 32 l + tid / 16; the 16
        // threads of a row are 16 consecutive lanes.
        f32x4 colw = zero4();
#pragma unroll
        for (int l = 0; l < NTT; ++l) {
            const int e = 4 * (l * NT + tid), t = e / C, j = e - t * C;
            f32x4 dt = lds4(a.wdT + ucc + e), da = lds4(a.wdA + ucc + e);
            if (!CHAN) {
                const f32x4 tt = lds4(a.wT + ucc + e), aa = lds4(a.wA + ucc + e);
                float wrow = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float wv = 0.f;
                    if (j + r <= t) {
                        wv = dt[r] * tt[r] + da[r] * aa[r];
                        const float f = expf(wG[t] - wG[j + r]);
                        dt[r] *= f;
                        da[r] *= f;
                    }
                    colw[r] += wv;
                    wrow += wv;
                }
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) wrow += __shfl_xor(wrow, off);
                if ((tid & 15) == 0) sRow[t] = wrow;
            }
            sts4(sdT + t * LC + j, dt);
            sts4(sdA + t * LC + j, da);
        }
        if (!CHAN) sts4(sColP + (tid >> 4) * C + 4 * (tid & 15), colw);
    }
    if (CHAN && tid < D) {
        float Bs[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) Bs[b] = wG[(16 * b + 15) * D + tid];
        int bits = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            sF[(3 + b) * D + tid] = expf(fminf(-Bs[b], kBwdDiagRange));
            bits |= Bs[b] < -kBwdDiagRange ? 1 << b : 0;
        }
        sF[tid] = expf(Bs[1]);
        sF[D + tid] = expf(Bs[2]);
        sF[2 * D + tid] = expf(Bs[1] + Bs[2]);
        sBits[tid] = bits;
    }
    __syncthreads();
    if (!CHAN && tid < C) {
        float cs = 0.f;
        for (int r = 0; r < 32; ++r) cs += sColP[r * C + tid];
        sCol[tid] = cs;
    }
    // X_e = dT' P2, X_q = dA' P2, X_k = dT'^T P1 + dA'^T P3 on the matrix
    // cores: 16 x 16 output tiles, wave w taking tiles w, w + 8, ...; then
    // through shared memory (where P1..P3 were) to the thread layout below.
    // Per-channel decay: with P1..P3 = E^, K^, Q^ the products split by
    // 16-token blocks, each block pair (bi, bj) taking its factor per channel
    // (1 for bj = bi - 1; exp(-B) on the diagonal, which a strongly decaying
    // block forms entry by entry further below); then exp(Gb_t) (X_e, X_q) and
    // exp(B - Gb_j) (X_k) per element make them the exact parts of de, dq, dk.
    int slow = 0;
    if (CHAN) {
        const int l = tid & 63;
        int m = 0;
        for (int c = l; c < D; c += 64) m |= sBits[c];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (__ballot((m >> b) & 1)) slow |= 1 << b;
    }
    {
        constexpr int NTC = D / 16, NTW = C / 16 * NTC / 8;
        const int w = tid >> 6, l = tid & 63;
        f32x4 te[NTW], tq[NTW], tk[NTW];
#pragma unroll
        for (int q = 0; q < NTW; ++q) {
            const int tile = w + 8 * q, rt = tile / NTC, ct = tile - rt * NTC;
            if constexpr (CHAN) {
                const int col = ct * 16 + (l & 15);
                const auto factor = [&](int bi, int bj) {
                    return bi == bj ? sF[(3 + bi) * D + col] : bi - bj == 1 ? 1.f : sF[(bwd_row_far(bi, bj) - 4) * D + col];
                };
                // The factor depends on the output column only, so it scales
                // the B operand, and each product accumulates over its block
                // pairs in one chain.
                te[q] = tq[q] = tk[q] = zero4();
                f32x4 tk2 = zero4();
                const int g = l >> 4, r16 = l & 15;
                for (int bj = 0; bj <= rt; ++bj) {  // rows t in block rt, columns j in block bj
                    if (bj == rt && ((slow >> rt) & 1)) continue;
                    const float f = factor(rt, bj);
                    const float *pt = sdT + (rt * 16 + r16) * LC + bj * 16 + g, *pa = sdA + (rt * 16 + r16) * LC + bj * 16 + g;
                    const float *pb = sP2 + (bj * 16 + g) * LD + col;
#pragma unroll
                    for (int k = 0; k < 16; k += 4) {
                        const float b = pb[k * LD] * f;
                        te[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(pt[k], b, te[q], 0, 0, 0);
                        tq[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k], b, tq[q], 0, 0, 0);
                    }
                }
                for (int bi = rt; bi < 4; ++bi) {  // rows j in block rt, tokens t in block bi
                    if (bi == rt && ((slow >> rt) & 1)) continue;
                    const float f = factor(bi, rt);
                    const float *pt = sdT + (bi * 16 + g) * LC + rt * 16 + r16, *pa = sdA + (bi * 16 + g) * LC + rt * 16 + r16;
                    const float *p1 = sP1 + (bi * 16 + g) * LD + col, *p3 = sP3 + (bi * 16 + g) * LD + col;
#pragma unroll
                    for (int k = 0; k < 16; k += 4) {
                        tk[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(pt[k * LC], p1[k * LD] * f, tk[q], 0, 0, 0);
                        tk2 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k * LC], p3[k * LD] * f, tk2, 0, 0, 0);
                    }
                }
                tk[q] += tk2;
            } else {
                te[q] = mfma_kloop<C>(zero4(), sdT + rt * 16 * LC, LC, sP2 + ct * 16, LD);
                tq[q] = mfma_kloop<C>(zero4(), sdA + rt * 16 * LC, LC, sP2 + ct * 16, LD);
                tk[q] = mfma_kloop_at<C>(zero4(), sdT + rt * 16, LC, sP1 + ct * 16, LD);
                tk[q] = mfma_kloop_at<C>(tk[q], sdA + rt * 16, LC, sP3 + ct * 16, LD);
            }
        }
        __syncthreads();  // dT, dA and the P tiles read
#pragma unroll
        for (int q = 0; q < NTW; ++q) {
            const int tile = w + 8 * q, rt = tile / NTC, ct = tile - rt * NTC, col = ct * 16 + (l & 15);
            const float Bb = CHAN ? wG[(rt * 16 + 15) * D + col] : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rt * 16 + 4 * (l >> 4) + r, o = row * LD + col;
                float fe = 1.f, fk = 1.f;
                if (CHAN) {
                    const float Gb = wG[row * D + col];
                    fe = expf(Gb);
                    fk = expf(Bb - Gb);
                }
                sP1[o] = te[q][r] * fe;
                sP2[o] = tq[q][r] * fe;
                sP3[o] = tk[q][r] * fk;
            }
        }
    }
    __syncthreads();  // X tiles written
    if (CHAN && slow) {
        // The diagonal blocks formed entry by entry: for token t and channel
        // d of such a block, the sums over the block's tokens m of
        // dT_tm k_m, dA_tm k_m (m before t) and dT_mt e_m + dA_mt q_m (m after
        // t), each times exp(Gb_t - Gb_m) or exp(Gb_m - Gb_t).
        for (int b = 0; b < 4; ++b) {
            if (!((slow >> b) & 1)) continue;
            for (int idx = tid; idx < 16 * D; idx += NT) {
                const int i = idx / D, d = idx - i * D, t = 16 * b + i;
                const float gt = wG[t * D + d];
                float xe = 0.f, xq = 0.f, xk = 0.f;
                for (int mm = 0; mm < 16; ++mm) {
                    const int m = 16 * b + mm;
                    if (m >= x.n) break;
                    const size_t iq = (x.rowq + (size_t)m * a.Hqk) * D + d, iv = (x.rowv + (size_t)m * a.Hv) * D + d;
                    const float km = ld1io<IO>(a.k, iq), gm = wG[m * D + d];
                    if (m <= t) {
                        const float f = expf(fminf(gt - gm, 0.f)) * km;
                        xq = fmaf(sdA[t * LC + m], f, xq);
                        if (m < t) xe = fmaf(sdT[t * LC + m], f, xe);
                    }
                    if (m >= t) {
                        const float f = expf(fminf(gm - gt, 0.f));
                        const float em = km * (BW ? ld1io<IO>(a.bg, iv) : a.beta[x.rowv + (size_t)m * a.Hv]);
                        xk = fmaf(sdA[m * LC + t], f * ld1io<IO>(a.q, iq), xk);
                        if (m > t) xk = fmaf(sdT[m * LC + t], f * em, xk);
                    }
                }
                sP1[t * LD + d] += xe;
                sP2[t * LD + d] += xq;
                sP3[t * LD + d] += xk;
            }
        }
        __syncthreads();
    }
    // dT's space holds dG from here.
    const int cg = tid % NCG, rg = tid / NCG, m0 = rg * RT, n0 = 4 * cg;

    f32x4 gend = zero4();
    // Per-channel decay: this thread's rows lie in one block b; G_t = R_b +
    // Gb_t and G_end - G_t = B_b - Gb_t + (the blocks after b).
    f32x4 Rb = zero4(), Aft = zero4(), Bb = zero4();
    if (CHAN) {
        const int b = m0 >> 4;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) {
            const f32x4 B2 = lds4(wG + (16 * b2 + 15) * D + n0);
            if (b2 < b) Rb += B2;
            if (b2 > b) Aft += B2;
            if (b2 == b) Bb = B2;
        }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = m0 + i;
        float dgs = 0.f, dbs = 0.f;
        if (t < x.n) {
            const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + n0, iv = (x.rowv + (size_t)t * a.Hv) * D + n0;
            const size_t o = ucd + (size_t)t * D + n0;
            const float bt = tied ? a.beta[x.rowv + (size_t)t * a.Hv] : 0.f;
            const f32x4 G = CHAN ? lds4(wG + t * D + n0) : splat(wG[t]);
            const f32x4 eg = CHAN ? exp4(Rb + G) : exp4(G);
            const f32x4 egend = CHAN ? exp4(Bb - G + Aft) : exp4(splat(wG[C - 1]) - G);
            const f32x4 qv = ld4io<IO>(a.q, iq), kv = ld4io<IO>(a.k, iq), vv = ld4io<IO>(a.v, iv);
            const f32x4 gb = BW ? ld4io<IO>(a.bg, iv) : splat(bt), gw = BW ? ld4io<IO>(a.wg, iv) : splat(bt);
            const f32x4 dEY = lds4(a.wdE + o), dQS = lds4(a.wdQ + o), dKE = lds4(a.wdK + o), dR = lds4(a.wdU + o);
            const f32x4 xe = lds4(sP1 + t * LD + n0), xq = lds4(sP2 + t * LD + n0), xk = lds4(sP3 + t * LD + n0);
            const f32x4 de = xe + dEY * eg;
            const f32x4 dq = xq + dQS * eg;
            const f32x4 ke = kv * egend;
            f32x4 dk = xk + dKE * egend;
            f32x4 dG = gb * kv * eg * dEY + qv * eg * dQS - ke * dKE;
            if (CHAN) dG += gb * kv * xe - kv * xk + qv * xq;  // the exponentials of T and A
            gend += ke * dKE;
            if (CHAN) sts4(sGt + t * LD + n0, dG);
            else dgs = dG[0] + dG[1] + dG[2] + dG[3];
            dk += gb * de;
            if (BW) {
                sts4(a.db + iv, de * kv);
                sts4(a.dw + iv, dR * vv);
            } else {
                const f32x4 pb = de * kv + dR * vv;
                dbs = pb[0] + pb[1] + pb[2] + pb[3];
            }
            sts4(a.dv + iv, gw * dR);
            if (grouped) {
                sts4(a.wdq + iv, dq);
                sts4(a.wdk + iv, dk);
            } else {
                sts4(a.dq + iq, dq);
                sts4(a.dk + iq, dk);
            }
        } else if (CHAN) {
            sts4(sGt + t * LD + n0, zero4());  // padded token
        }
        sTokG[t * 32 + cg] = dgs;
        sTokB[t * 32 + cg] = dbs;
    }
    sts4(sGeP + rg * D + n0, gend);
    __syncthreads();
    // dG_end = sum over the chunk of Kend . dKend, plus Gamma . dGamma.
    if (tid < D) {
        float g = a.wGam[(size_t)u * D + tid] * a.wdGam[(size_t)u * D + tid];
        for (int r = 0; r < NRG; ++r) g += sGeP[r * D + tid];
        sGe[tid] = g;
    }
    if (tid < C) {
        float g = 0.f, bsum = 0.f;
        for (int r = 0; r < NCG; ++r) {
            g += sTokG[tid * 32 + r];
            bsum += sTokB[tid * 32 + r];
        }
        sTokG[tid * 32] = g;
        sTokB[tid * 32] = bsum;
    }
    __syncthreads();
    if (!CHAN && tid == 0) {
        float g = 0.f;
        for (int d = 0; d < D; ++d) g += sGe[d];
        sGe[0] = g;
    }
    __syncthreads();
    if (a.dg) {
        if (CHAN) {
            if (tid < D) {
                float acc = sGe[tid];
                for (int t = C - 1; t >= 0; --t) {
                    acc += sGt[t * LD + tid];
                    if (t < x.n) a.dg[(x.rowv + (size_t)t * a.Hv) * D + tid] = acc;
                }
            }
        } else if (tid < 64) {
            // Suffix sums over the chunk's tokens; lane = token.
            float v = sTokG[tid * 32] + sRow[tid] - sCol[tid];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(v, off);
                if (tid + off < 64) v += y;
            }
            if (tid < x.n) a.dg[x.rowv + (size_t)tid * a.Hv] = v + sGe[0];
        }
    }
    if (tied && tid < x.n) a.dbeta[x.rowv + (size_t)tid * a.Hv] = sTokB[tid * 32];
}

// dq, dk of a QK head: the sum of its V heads' parts.
template <int D>
__global__ __launch_bounds__(NT) void cb_group_sum(ChunkBwdArgs a) {
    const int grp = a.Hv / a.Hqk;
    const size_t n4 = (size_t)a.B * a.T * a.Hqk * D / 4;
    for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * NT) {
        const size_t e = 4 * i, d = e % D, r = e / D, hq = r % a.Hqk, bt = r / a.Hqk;
        const size_t base = (bt * a.Hv + hq * grp) * D + d;
        f32x4 sq = zero4(), sk = zero4();
        for (int j = 0; j < grp; ++j) {
            sq += lds4(a.wdq + base + (size_t)j * D);
            sk += lds4(a.wdk + base + (size_t)j * D);
        }
        sts4(a.dq + e, sq);
        sts4(a.dk + e, sk);
    }
}

template <typename IO, int D, bool CHAN, bool BW>
hipError_t run(const ChunkBwdArgs &a, hipStream_t s) {
    constexpr size_t bmax = bsweep_full_smem<D>() > bsweep_rhs_smem<D>() ? bsweep_full_smem<D>() : bsweep_rhs_smem<D>();
    constexpr size_t sweep_smem = bmax > fsweep_smem<D>() ? bmax : fsweep_smem<D>();
    static_assert(sweep_smem <= 160 * 1024, "the sweeps' tiles exceed a workgroup's local data share");
    static const hipError_t attr = [] {
        const void *fn[6] = {reinterpret_cast<const void *>(&cb_prep<IO, D, CHAN, BW>),
                             reinterpret_cast<const void *>(&cb_rhs<IO, D>),
                             reinterpret_cast<const void *>(&cb_sweeps<IO, D, false>),
                             reinterpret_cast<const void *>(&cb_sweeps<IO, D, true>),
                             reinterpret_cast<const void *>(&cb_grad_s<IO, D>),
                             reinterpret_cast<const void *>(&cb_grad_out<IO, D, CHAN, BW>)};
        const size_t bytes[6] = {prep_smem<D>(), rhs_smem<D>(), sweep_smem, sweep_smem, grad_s_smem<D>(), grad_out_smem<D>()};
        for (int i = 0; i < 6; ++i) {
            const hipError_t e = hipFuncSetAttribute(fn[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes[i]);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    const unsigned units = (unsigned)((size_t)a.B * a.Hv * a.NC), items = (unsigned)((size_t)a.B * a.Hv * (D / BV));
    // One persistent prep workgroup per compute unit (its shared memory takes the unit's).
    const unsigned pgrid = units < (unsigned)device_cus() ? units : (unsigned)device_cus();
    hipLaunchKernelGGL((cb_prep<IO, D, CHAN, BW>), dim3(pgrid), dim3(NT), prep_smem<D>(), s, a);
    const unsigned P = (items + 7) / 8 * 8;
    // The X-independent products leave the backward sweep's chain when both
    // sweeps' workgroups fit on the compute units at once (the chain then
    // bounds the call).
    if (2 * P <= (unsigned)device_cus()) {
        hipLaunchKernelGGL((cb_rhs<IO, D>), dim3(units), dim3(NT), rhs_smem<D>(), s, a);
        hipLaunchKernelGGL((cb_sweeps<IO, D, true>), dim3(2 * P), dim3(NS), sweep_smem, s, a, (int)items, (int)P);
    } else {
        hipLaunchKernelGGL((cb_sweeps<IO, D, false>), dim3(2 * P), dim3(NS), sweep_smem, s, a, (int)items, (int)P);
    }
    hipLaunchKernelGGL((cb_grad_s<IO, D>), dim3(pgrid), dim3(NT), grad_s_smem<D>(), s, a);
    hipLaunchKernelGGL((cb_grad_out<IO, D, CHAN, BW>), dim3(units), dim3(NT), grad_out_smem<D>(), s, a);
    if (a.Hv > a.Hqk) {
        const size_t n4 = (size_t)a.B * a.T * a.Hqk * D / 4;
        const size_t blocks = (n4 + NT - 1) / NT;
        hipLaunchKernelGGL((cb_group_sum<D>), dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

template <typename IO, int D>
hipError_t run_modes(const ChunkBwdArgs &a, hipStream_t s) {
    const bool chan = a.decay == DECAY_CHANNEL, bw = a.beta == nullptr;
    if (chan) return bw ? run<IO, D, true, true>(a, s) : run<IO, D, true, false>(a, s);
    return bw ? run<IO, D, false, true>(a, s) : run<IO, D, false, false>(a, s);
}

template <typename IO>
hipError_t run_dims(int D, const ChunkBwdArgs &a, hipStream_t s) {
    switch (D) {
    case 32: return run_modes<IO, 32>(a, s);
    case 64: return run_modes<IO, 64>(a, s);
    case 128: return run_modes<IO, 128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_backward(int io, int D, const ChunkBwdArgs &a, hipStream_t s) {
    return io == IO_BF16 ? run_dims<bf16_t>(D, a, s) : run_dims<float>(D, a, s);
}

}  // namespace gdr
