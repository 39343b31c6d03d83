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
//   E~ = e . exp(G)     K~ = k . exp(-G)     Q~ = q . exp(G)
//   Kend = k . exp(G_end - G)                gamma = exp(G_end)
//   T = strict_lower(E~ K~^T)      A = lower_incl(Q~ K~^T)
//   L = (I + T)^-1                 (unit lower triangular; no dense solve)
//   Y = L E~        U_z = L Z      (erase side / write side of the WY form)
//   U = U_z - Y S_c                (the resolved errors)
//   O = s (Q~ S_c + A U) = (s (Q~ - A Y)) S_c + s A U_z
//   S_{c+1} = Diag(gamma) S_c + Kend^T U
//
// Two kernels. chunk_prep is parallel over every (sequence, V head, chunk):
// it does everything that does not depend on the state -- prefix sums, decay
// absorption, both Gram products, the triangular inverse, and the products
// Y, U_z, W_q = s (Q~ - A Y), O_z = s A U_z -- and stores them in a
// workspace. chunk_sweep is the single sequential pass over chunks: per
// (sequence, V head, value tile) it keeps the fp32 state in matrix-core
// accumulator registers and per chunk does U = U_z - Y S_c,
// O = W_q S_c + O_z and S_{c+1} = gamma . S_c + Kend^T U. Value columns of the
// state evolve independently, so the sweep is split over value tiles.
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

__host__ __device__ constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t a16(size_t x) { return (x + 15) & ~(size_t)15; }

// Copy a rows x cols block between row strides, 16 bytes per access.
template <typename T>
__device__ __forceinline__ void copy_block(T *dst, int dld, const T *src, int sld, int rows, int cols, int tid, int nt) {
    constexpr int V = 16 / sizeof(T);
    const int per_row = cols / V;
    for (int i = tid; i < rows * per_row; i += nt) {
        const int r = i / per_row, c = (i - r * per_row) * V;
        *reinterpret_cast<uint4 *>(dst + (size_t)r * dld + c) = *reinterpret_cast<const uint4 *>(src + (size_t)r * sld + c);
    }
}

// The 10 lower-triangular 16 x 16 tiles of a 64 x 64 matrix.
__device__ __forceinline__ void lower_tile(int idx, int &ti, int &tj) {
    ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    tj = idx - ti * (ti + 1) / 2;
}

// exp(x) = 2^(x log2 e) on the hardware exp2 (v_exp_f32, ~1 ulp).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// acc += A[16 x 16] * (Bt[16 x 16])^T. For bf16 this is one 16x16x32 step:
// columns 16..31 of A must be zero and those of Bt finite.
template <typename IO>
__device__ __forceinline__ f32x4 mma_k16(f32x4 acc, const IO *A, int lda, const IO *Bt, int ldb) {
    using M = Mma<IO>;
#pragma unroll
    for (int ks = 0; ks < (16 + M::KS - 1) / M::KS; ++ks) acc = M::step(acc, A + ks * M::KS, lda, Bt + ks * M::KS, ldb);
    return acc;
}

template <typename IO, int D>
struct PrepCfg {
    static constexpr int NW = D / 16 < 4 ? D / 16 : 4;  // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int CQ = D / 4;         // channel quads
    static constexpr int NGRP = NT / CQ;     // token groups (threads per channel quad)
    static constexpr int TPT = C / NGRP;     // tokens per thread in the elementwise phase
    static constexpr int NCTS = 2 * D / NW / 16;  // 16-wide right-hand-side column tiles per wave
    static constexpr int PD = D + 8;    // row stride of [C x D] row-major tiles
    static constexpr int PT = C + 8;    // row stride of token-contiguous tiles
    static constexpr int PDB = sizeof(IO) == 2 ? 40 : 20;   // D_b rows (bf16: K padded to 32 with zeros)
    static constexpr int PTMP = sizeof(IO) == 2 ? 32 : 20;  // per-wave solve temporary rows
    static constexpr size_t SLOT = a16(cmax((size_t)C * PD, (size_t)D * PT) * sizeof(IO));
    static constexpr size_t XT = a16((size_t)2 * D * PT * sizeof(IO));
    static constexpr size_t TA = a16((size_t)2 * C * PT * sizeof(IO));
    static constexpr size_t TD = a16((size_t)4 * 16 * 17 * 4);
    static constexpr size_t DB = a16((size_t)4 * 16 * PDB * sizeof(IO));
    static constexpr size_t PART = a16((size_t)NGRP * D * 4);
    static constexpr size_t OFF_K = SLOT, OFF_Q = 2 * SLOT, OFF_XT = 3 * SLOT, OFF_TA = OFF_XT + XT,
                            OFF_TD = OFF_TA + TA, OFF_DB = OFF_TD + TD, OFF_PART = OFF_DB + DB,
                            BYTES = OFF_PART + PART;
    static_assert(TA >= (size_t)D * PT * sizeof(IO), "Kend^T staging");
    static_assert((size_t)NW * 16 * NCTS * PTMP * sizeof(IO) <= SLOT, "solve temporaries");
    static_assert(NGRP * TPT == C && TPT % 4 == 0, "elementwise mapping");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// One thread's raw inputs for a chunk: 4 tokens x 4 channels of q, k, v (and
// b, w, per-channel g) plus the 4 tokens' beta; lane l of every wave also
// holds token l's scalar g for the in-wave prefix scan. Kept raw so that the
// loads for the next chunk are issued early and waited for only when used.
template <typename IO, int D, bool CHAN, bool BW>
struct PrepIn {
    using R4 = Raw4<IO>;
    static constexpr int TPT = PrepCfg<IO, D>::TPT;
    typename R4::type q[TPT], k[TPT], v[TPT], bg[BW ? TPT : 1], wg[BW ? TPT : 1];
    f32x4 g[CHAN ? TPT : 1];
    float betal, gs;  // lane l of every wave: token l's beta and scalar g

    __device__ __forceinline__ void load(const ChunkArgs &a, int u, int cq, int grp) {
        const int NC = a.NC, c = u % NC, bh = u / NC, b = bh / a.Hv, h = bh - b * a.Hv;
        const int hq = h / (a.Hv / a.Hqk), t0 = c * C, n = min(C, a.T - t0);
        const int l = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const size_t tok = (size_t)b * a.T + t0 + min(TPT * grp + j, n - 1);  // clamped: padded tokens are zeroed at use
            q[j] = R4::load(static_cast<const IO *>(a.q) + (tok * a.Hqk + hq) * D + 4 * cq);
            k[j] = R4::load(static_cast<const IO *>(a.k) + (tok * a.Hqk + hq) * D + 4 * cq);
            v[j] = R4::load(static_cast<const IO *>(a.v) + (tok * a.Hv + h) * D + 4 * cq);
            if constexpr (BW) {
                bg[j] = R4::load(static_cast<const IO *>(a.bg) + (tok * a.Hv + h) * D + 4 * cq);
                wg[j] = R4::load(static_cast<const IO *>(a.wg) + (tok * a.Hv + h) * D + 4 * cq);
            }
            if constexpr (CHAN) g[j] = *reinterpret_cast<const f32x4 *>(a.g + (tok * a.Hv + h) * D + 4 * cq);
        }
        const size_t tl = ((size_t)b * a.T + t0 + min(l, n - 1)) * a.Hv + h;
        if constexpr (!BW) betal = a.beta[tl];
        if constexpr (!CHAN) gs = a.decay == DECAY_SCALAR ? a.g[tl] : 0.f;
    }
};

// Everything in a chunk that does not depend on the state, for every
// (sequence, V head, chunk) unit; persistent over units, with the next unit's
// inputs prefetched while the current one is processed. Per unit:
//  A. decay prefix sums and decay absorption; E~ (row-major, and token-
//     contiguous as the right-hand side), K~, Q~, Z; Kend^T; gamma.
//  B. Gram products T = E~ K~^T and A = Q~ K~^T on the matrix cores (lower tiles).
//     Scalar decay (and none) uses the raw Gram with exp(G_i - G_j) applied per
//     entry, so no factor can overflow; per-channel decay uses the factored form.
//  C. (I + T) X = [E~ | Z] by blocked forward substitution over four 16-token
//     blocks: the 16 x 16 diagonal blocks are inverted in fp32, the rest are
//     matrix-core products; each wave solves its own 32 right-hand-side columns.
//  D. W_q = s (Q~ - A Y), O_z = s A U_z, and the workspace stores.
template <typename IO, int D, bool CHAN, bool BW>
__global__ __launch_bounds__(D >= 64 ? 256 : 128) void chunk_prep(ChunkArgs a) {  // = PrepCfg<IO, D>::NT
    using E = Elem<IO>;
    using M = Mma<IO>;
    using R4 = Raw4<IO>;
    using Cfg = PrepCfg<IO, D>;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, CQ = Cfg::CQ, PD = Cfg::PD, PT = Cfg::PT;
    constexpr int NGRP = Cfg::NGRP, TPT = Cfg::TPT, NCTS = Cfg::NCTS, WC = 16 * NCTS;  // WC: columns per wave
    static_assert(NT == (D >= 64 ? 256 : 128), "launch bounds");
    constexpr int PDB = Cfg::PDB, PTMP = Cfg::PTMP, KS = M::KS;
    constexpr int NG = (20 + NW - 1) / NW;  // Gram tile products per wave

    extern __shared__ __align__(16) unsigned char smem[];
    IO *sE = reinterpret_cast<IO *>(smem);                    // E~ (or raw e) [C][PD]; then solve temporaries
    IO *sK = reinterpret_cast<IO *>(smem + Cfg::OFF_K);       // K~ (or raw k) [C][PD]; then W_q staging [C][PD]
    IO *sQ = reinterpret_cast<IO *>(smem + Cfg::OFF_Q);       // Q~ (or raw q) [C][PD]
    IO *sXT = reinterpret_cast<IO *>(smem + Cfg::OFF_XT);     // [E~ | Z]^T [2D][PT] -> [Y | U_z]^T in place
    IO *sTo = reinterpret_cast<IO *>(smem + Cfg::OFF_TA);     // -T without its diagonal blocks [C][PT]
    IO *sA = sTo + C * PT;                                     // A [C][PT]
    IO *sKT = sTo;                                             // Kend^T staging [D][PT] (phase A only)
    float *sTd = reinterpret_cast<float *>(smem + Cfg::OFF_TD);  // T diagonal blocks [4][16][17] fp32
    IO *sDb = reinterpret_cast<IO *>(smem + Cfg::OFF_DB);        // their inverses [4][16][PDB]
    float *sPart = reinterpret_cast<float *>(smem + Cfg::OFF_PART);  // [16][D] per-group channel sums
    IO *sWs = sK;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;
    const int cq = tid % CQ, grp = tid / CQ;
    const int units = a.B * a.Hv * a.NC;
    constexpr bool chan = CHAN;

    // D_b's padding columns (bf16 K = 32 steps) stay zero for the whole kernel.
    for (int i = tid; i < 4 * 16 * PDB; i += NT) sDb[i] = E::to(0.f);

    PrepIn<IO, D, CHAN, BW> in;
    if ((int)blockIdx.x < units) in.load(a, blockIdx.x, cq, grp);

    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int NC = a.NC, c = u % NC, bh = u / NC;
        const int n = min(C, a.T - c * C);
        IO *ws = static_cast<IO *>(a.ws_io) + (size_t)u * chunk_ws_io_elems(D);
        IO *wY = ws, *wWq = ws + C * D, *wKT = ws + 2 * C * D, *wUzT = ws + 3 * C * D, *wOzT = ws + 4 * C * D;
        __syncthreads();  // the previous unit's readers of shared memory are done

        // ---- A. prefix sums and decay absorption ----
        // Scalar decay: each wave scans the 64 token values itself (lane = token).
        float Gl = 0.f;
        if (!CHAN) {
            Gl = l < n ? in.gs : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(Gl, off);
                if (l >= off) Gl += y;
            }
        }
        const float Gend_s = __shfl(Gl, 63);
        float G[TPT][4];
        if constexpr (CHAN) {
            // Running sums over this thread's tokens, then add the totals of the
            // earlier token groups.
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch)
                    G[j][ch] = (TPT * grp + j < n ? in.g[CHAN ? j : 0][ch] : 0.f) + (j > 0 ? G[j - 1][ch] : 0.f);
            store4f(sPart + grp * D + 4 * cq, f32x4{G[TPT - 1][0], G[TPT - 1][1], G[TPT - 1][2], G[TPT - 1][3]});
        }
        __syncthreads();
        float Gend[4];
        if constexpr (CHAN) {
            f32x4 off = zero4(), tot = zero4();
#pragma unroll
            for (int g2 = 0; g2 < NGRP; ++g2) {
                const f32x4 p = load4f(sPart + g2 * D + 4 * cq);
                if (g2 < grp) off += p;
                tot += p;
            }
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) G[j][ch] += off[ch];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) Gend[ch] = tot[ch];
        } else {
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const float Gt = __shfl(Gl, TPT * grp + j);
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) G[j][ch] = Gt;
            }
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) Gend[ch] = Gend_s;
        }
        // Per token: operands for the Gram (row-major), and the token-contiguous
        // right-hand side E~, Z and Kend^T (4 tokens per 8/16-byte store).
        float xE[4][4], xZ[4][4], xKe[4][4];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const int tk = TPT * grp + j;
            const bool valid = tk < n;
            const f32x4 kk = R4::widen(in.k[j]), qq = R4::widen(in.q[j]), vv = R4::widen(in.v[j]);
            f32x4 eb, wz;
            if constexpr (BW) {
                eb = R4::widen(in.bg[j]);
                wz = R4::widen(in.wg[j]);
            } else {
                const float bt = __shfl(in.betal, tk);
                eb = f32x4{bt, bt, bt, bt};
                wz = eb;
            }
            float gE[4], gK[4], gQ[4];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const float kv = valid ? kk[ch] : 0.f, qv = valid ? qq[ch] : 0.f;
                const float ev = eb[ch] * kv;
                const float eg = fast_exp(G[j][ch]);
                xE[j & 3][ch] = ev * eg;
                xZ[j & 3][ch] = valid ? wz[ch] * vv[ch] : 0.f;
                xKe[j & 3][ch] = kv * fast_exp(Gend[ch] - G[j][ch]);
                if (chan) {  // factored form for the Gram
                    gE[ch] = ev * eg;
                    gK[ch] = kv * __builtin_amdgcn_rcpf(eg);
                    gQ[ch] = qv * eg;
                } else {     // raw operands; the decay is applied to the Gram entries
                    gE[ch] = ev;
                    gK[ch] = kv;
                    gQ[ch] = qv;
                }
            }
            store4f(sE + tk * PD + 4 * cq, f32x4{gE[0], gE[1], gE[2], gE[3]});
            store4f(sK + tk * PD + 4 * cq, f32x4{gK[0], gK[1], gK[2], gK[3]});
            store4f(sQ + tk * PD + 4 * cq, f32x4{gQ[0], gQ[1], gQ[2], gQ[3]});
            if ((j & 3) == 3) {
                const int t4 = tk - 3;
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const int cc = 4 * cq + ch;
                    store4f(sXT + cc * PT + t4, f32x4{xE[0][ch], xE[1][ch], xE[2][ch], xE[3][ch]});
                    store4f(sXT + (D + cc) * PT + t4, f32x4{xZ[0][ch], xZ[1][ch], xZ[2][ch], xZ[3][ch]});
                    store4f(sKT + cc * PT + t4, f32x4{xKe[0][ch], xKe[1][ch], xKe[2][ch], xKe[3][ch]});
                }
            }
        }
        if (grp == NGRP - 1)
            store4f(a.ws_gamma + (size_t)u * D + 4 * cq,
                    f32x4{fast_exp(Gend[0]), fast_exp(Gend[1]), fast_exp(Gend[2]), fast_exp(Gend[3])});
        // The raw inputs are consumed: fetch the next unit's now.
        if (u + (int)gridDim.x < units) in.load(a, u + gridDim.x, cq, grp);
        __syncthreads();
        copy_block(wKT, C, sKT, PT, D, C, tid, NT);

        // ---- B. Gram products (20 lower 16x16 tiles: 10 of T, 10 of A) ----
        f32x4 gacc[NG];
#pragma unroll
        for (int s = 0; s < NG; ++s) {
            const int p = w + NW * s;
            gacc[s] = zero4();
            if (p < 20) {
                const int kind = p / 10;
                int ti, tj;
                lower_tile(p - kind * 10, ti, tj);
                const IO *X = kind == 0 ? sE : sQ;
#pragma unroll
                for (int ks = 0; ks < D / KS; ++ks)
                    gacc[s] = M::step(gacc[s], X + ti * 16 * PD + ks * KS, PD, sK + tj * 16 * PD + ks * KS, PD);
            }
        }
        __syncthreads();  // Kend^T staging copied out (its space becomes -T and A)
#pragma unroll
        for (int s = 0; s < NG; ++s) {
            const int p = w + NW * s;
            if (p < 20) {
                const int kind = p / 10;
                int ti, tj;
                lower_tile(p - kind * 10, ti, tj);
                const int col = tj * 16 + lr;
                const float Gc = __shfl(Gl, col);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = ti * 16 + 4 * lq + r;
                    float x = gacc[s][r];
                    if (!chan) x *= fast_exp(fminf(__shfl(Gl, row) - Gc, 0.f));
                    if (kind == 0) {
                        if (ti == tj) sTd[(ti * 16 + 4 * lq + r) * 17 + lr] = col < row ? x : 0.f;
                        else sTo[row * PT + col] = E::to(-x);
                    } else {
                        sA[row * PT + col] = E::to(col <= row ? x : 0.f);
                    }
                }
            }
        }
        // Zero tiles: -T on and above the diagonal blocks, A above them.
        for (int i = tid; i < C * C; i += NT) {
            const int row = i / C, col = i - (i / C) * C;
            if ((col >> 4) >= (row >> 4)) sTo[row * PT + col] = E::to(0.f);
            if ((col >> 4) > (row >> 4)) sA[row * PT + col] = E::to(0.f);
        }
        __syncthreads();

        // ---- C. diagonal block inverses (fp32 forward substitution) ----
        for (int blk = w; blk < 4; blk += NW) {
            if (lr == l) {  // lanes 0..15: one column each
                const float *Tb = sTd + blk * 16 * 17;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s = i == lr ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < i; ++m) s -= Tb[i * 17 + m] * x[m];
                    x[i] = s;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) sDb[(blk * 16 + i) * PDB + lr] = E::to(x[i]);
            }
        }
        __syncthreads();

        // ---- C. blocked forward substitution; wave w owns columns WC*w..WC*w+WC-1 of [E~ | Z] ----
        IO *tmp = sE + w * WC * PTMP;
        if (PTMP > 16)  // bf16: the 32-deep K step reads temporary columns 16..31; keep them zero
            for (int i = l; i < WC * (PTMP - 16); i += 64)
                tmp[(i / (PTMP - 16)) * PTMP + 16 + i % (PTMP - 16)] = E::to(0.f);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4 acc[NCTS];
#pragma unroll
            for (int ct = 0; ct < NCTS; ++ct)
                acc[ct] = R4::widen(R4::load(sXT + (WC * w + 16 * ct + lr) * PT + 16 * blk + 4 * lq));
#pragma unroll
            for (int ks = 0; ks < (16 * blk + KS - 1) / KS; ++ks)
#pragma unroll
                for (int ct = 0; ct < NCTS; ++ct)
                    acc[ct] = M::step(acc[ct], sTo + 16 * blk * PT + ks * KS, PT,
                                      sXT + (WC * w + 16 * ct) * PT + ks * KS, PT);
#pragma unroll
            for (int ct = 0; ct < NCTS; ++ct) store4f(tmp + (16 * ct + lr) * PTMP + 4 * lq, acc[ct]);
#pragma unroll
            for (int ct = 0; ct < NCTS; ++ct) {
                const f32x4 x = mma_k16<IO>(zero4(), sDb + blk * 16 * PDB, PDB, tmp + 16 * ct * PTMP, PTMP);
                store4f(sXT + (WC * w + 16 * ct + lr) * PT + 16 * blk + 4 * lq, x);
            }
        }

        // ---- D. P = A [Y | U_z] on this wave's columns; W_q = s (Q~ - P), O_z = s P ----
        const float sc = a.scale;
        const bool yside = WC * w < D;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc[NCTS];
#pragma unroll
            for (int ct = 0; ct < NCTS; ++ct) acc[ct] = zero4();
#pragma unroll
            for (int ks = 0; ks < (16 * (rt + 1) + KS - 1) / KS; ++ks)
#pragma unroll
                for (int ct = 0; ct < NCTS; ++ct)
                    acc[ct] = M::step(acc[ct], sA + 16 * rt * PT + ks * KS, PT, sXT + (WC * w + 16 * ct) * PT + ks * KS,
                                      PT);
#pragma unroll
            for (int ct = 0; ct < NCTS; ++ct) {
                const int col = WC * w + 16 * ct + lr, tok = 16 * rt + 4 * lq;
                if (yside) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float qd = E::from(sQ[(tok + r) * PD + col]);
                        if (!chan) qd *= fast_exp(__shfl(Gl, tok + r));
                        sWs[(tok + r) * PD + col] = E::to(sc * (qd - acc[ct][r]));
                    }
                } else {
                    store4f(wOzT + (size_t)(col - D) * C + tok, sc * acc[ct]);
                }
            }
        }
        __syncthreads();

        // Workspace stores: Y row-major (transposed read of Y^T), U_z^T, W_q.
        {
            constexpr int V = 16 / sizeof(IO), PER = D / V;
            for (int i = tid; i < C * PER; i += NT) {
                const int tok = i / PER, c0 = (i - tok * PER) * V;
                IO vals[V];
#pragma unroll
                for (int j = 0; j < V; ++j) vals[j] = sXT[(c0 + j) * PT + tok];
                *reinterpret_cast<uint4 *>(wY + tok * D + c0) = *reinterpret_cast<const uint4 *>(vals);
            }
        }
        copy_block(wUzT, C, sXT + D * PT, PT, D, C, tid, NT);
        copy_block(wWq, D, sWs, PD, C, D, tid, NT);
    }
}

// Sequential sweep over chunks for one (sequence, V head, value tile of BV =
// 16*NCT columns). NW = D/32 waves; wave w keeps state rows 32w..32w+31 in
// accumulator layout and computes token tiles [w*TPW, (w+1)*TPW) of P, R.
// Each wave reads only its own slice of a chunk's factors (its token rows of
// Y and W_q, its channel rows of Kend^T), so those slices are prefetched into
// registers PF chunks ahead and the global-memory latency leaves the chain.
template <typename IO, int D, int NCT>
struct SweepOps {
    using M = Mma<IO>;
    using F = typename M::Frag;
    static constexpr int NW = D / 32, TPW = 4 / NW, KD = D / M::KS, KC = C / M::KS;
    using R4 = Raw4<IO>;
    F ya[TPW][KD], wa[TPW][KD], ka[2][KC];
    typename R4::type uz[TPW][NCT], oz[TPW][NCT];
    f32x4 g4[2];

    __device__ __forceinline__ void load(const IO *wsb, const float *wsg, size_t u, int w, int col0) {
        const int l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
        const IO *Y = wsb + u * chunk_ws_io_elems(D), *Wq = Y + C * D, *KT = Wq + C * D, *UzT = KT + D * C,
                 *OzT = UzT + D * C;
        const float *gam = wsg + u * D;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int T0 = (w * TPW + tt) * 16;
#pragma unroll
            for (int ks = 0; ks < KD; ++ks) {
                ya[tt][ks] = M::load(Y + T0 * D + ks * M::KS, D);
                wa[tt][ks] = M::load(Wq + T0 * D + ks * M::KS, D);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const size_t off = (size_t)(col0 + 16 * ct + lr) * C + T0 + 4 * lq;
                uz[tt][ct] = R4::load(UzT + off);
                oz[tt][ct] = R4::load(OzT + off);
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int ch0 = 32 * w + 16 * rt;
#pragma unroll
            for (int ks = 0; ks < KC; ++ks) ka[rt][ks] = M::load(KT + ch0 * C + ks * M::KS, C);
            g4[rt] = load4f(gam + ch0 + 4 * lq);
        }
    }
};

// One chunk of the sweep. TAIL = the chunk may hold fewer than C tokens
// (only the last one), so output rows are stored under a predicate; every
// other chunk stores unconditionally, which keeps the number of memory
// operations in flight static and lets the prefetches stay in flight.
template <typename IO, int D, int NCT, bool TAIL>
__device__ __forceinline__ void sweep_chunk(const SweepOps<IO, D, NCT> &op, f32x4 (&S)[2][NCT], IO *sST, IO *sUT,
                                            IO *sO, IO *orow0, size_t orow_stride, int n_valid) {
    using M = Mma<IO>;
    using F = typename M::Frag;
    using Ops = SweepOps<IO, D, NCT>;
    constexpr int BV = 16 * NCT, TPW = Ops::TPW, KS = M::KS, KD = Ops::KD, KC = Ops::KC;
    constexpr int LS = D + 8, LU = C + 8, LO = BV + 8;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;

#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            store4f(sST + (16 * ct + lr) * LS + 32 * w + 16 * rt + 4 * lq, S[rt][ct]);
    __syncthreads();

#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int T0 = (w * TPW + tt) * 16;
        f32x4 accP[NCT], accR[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) { accP[ct] = zero4(); accR[ct] = zero4(); }
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const F sb = M::load(sST + 16 * ct * LS + ks * KS, LS);
                accP[ct] = M::mma(accP[ct], op.ya[tt][ks], sb);
                accR[ct] = M::mma(accR[ct], op.wa[tt][ks], sb);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int col = 16 * ct + lr, tok = T0 + 4 * lq;
            const f32x4 U = Ops::R4::widen(op.uz[tt][ct]) - accP[ct];
            const f32x4 O = accR[ct] + Ops::R4::widen(op.oz[tt][ct]);
            store4f(sUT + col * LU + tok, U);
#pragma unroll
            for (int r = 0; r < 4; ++r) sO[(tok + r) * LO + col] = Elem<IO>::to(O[r]);
        }
    }
    __syncthreads();

    // Output rows: 16 bytes per thread, contiguous within each token row.
    {
        constexpr int V = 16 / sizeof(IO), PER = BV / V;
        for (int i = threadIdx.x; i < C * PER; i += blockDim.x) {
            const int tok = i / PER, c8 = (i - tok * PER) * V;
            if (!TAIL || tok < n_valid)
                *reinterpret_cast<uint4 *>(orow0 + tok * orow_stride + c8) =
                    *reinterpret_cast<const uint4 *>(sO + tok * LO + c8);
        }
    }

#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= op.g4[rt];
#pragma unroll
        for (int ks = 0; ks < KC; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                S[rt][ct] = M::mma(S[rt][ct], op.ka[rt][ks], M::load(sUT + 16 * ct * LU + ks * KS, LU));
    }
}

template <typename IO, int D, int NCT, int PF>
__global__ __launch_bounds__(2 * D) void chunk_sweep(ChunkArgs a, int NVT, int G) {
    using Ops = SweepOps<IO, D, NCT>;
    constexpr int BV = 16 * NCT;
    constexpr int LS = D + 8, LU = C + 8, LO = BV + 8;
    __shared__ __align__(16) IO sST[BV * LS];  // S_c^T in the io dtype
    __shared__ __align__(16) IO sUT[BV * LU];  // U^T in the io dtype
    __shared__ __align__(16) IO sO[C * LO];    // output tile, token rows

    // Work index: blocks that share an XCD (blockIdx % 8) take consecutive
    // work items, so the value tiles of one head read its chunk factors
    // through the same L2.
    const int x = blockIdx.x;
    const int wi = (x & 7) * (int)(gridDim.x >> 3) + (x >> 3);
    if (wi >= G) return;
    const int bh = wi / NVT, vt = wi - (wi / NVT) * NVT, col0 = vt * BV;
    const int b = bh / a.Hv, h = bh - (bh / a.Hv) * a.Hv;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;

    f32x4 S[2][NCT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = 32 * w + 16 * rt + 4 * lq + r, col = col0 + 16 * ct + lr;
                S[rt][ct][r] = a.S0 ? a.S0[((size_t)bh * D + ch) * D + col] : 0.f;
            }

    const IO *wsb = static_cast<const IO *>(a.ws_io);
    const size_t u0 = (size_t)bh * a.NC;
    const int NC = a.NC;
    const size_t orow_stride = (size_t)a.Hv * D;
    IO *obase = static_cast<IO *>(a.o) + ((size_t)b * a.T * a.Hv + h) * D + col0;

    if (NC > 0) {
        Ops ring[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) ring[j].load(wsb, a.ws_gamma, u0 + min(j, NC - 1), w, col0);

        // Pipelined part: every chunk but the last is full (C tokens).
        int c = 0;
        for (; c + PF <= NC - 1; c += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                sweep_chunk<IO, D, NCT, false>(ring[j], S, sST, sUT, sO, obase + (size_t)(c + j) * C * orow_stride,
                                               orow_stride, C);
                ring[j].load(wsb, a.ws_gamma, u0 + min(c + j + PF, NC - 1), w, col0);
            }
        }
        // Remainder: ring slot j holds chunk c + j (clamped); the last chunk may be partial.
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int cj = c + j;
            if (cj < NC)
                sweep_chunk<IO, D, NCT, true>(ring[j], S, sST, sUT, sO, obase + (size_t)cj * C * orow_stride,
                                              orow_stride, a.T - cj * C);
        }
    }

#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ch = 32 * w + 16 * rt + 4 * lq + r, col = col0 + 16 * ct + lr;
                a.ST[((size_t)bh * D + ch) * D + col] = S[rt][ct][r];
            }
}

static int device_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

template <typename IO, int D, int NCT>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t s) {
    using Cfg = PrepCfg<IO, D>;
    static bool attr_set = false;
    if (!attr_set) {
        const void *fns[4] = {reinterpret_cast<const void *>(&chunk_prep<IO, D, false, false>),
                              reinterpret_cast<const void *>(&chunk_prep<IO, D, false, true>),
                              reinterpret_cast<const void *>(&chunk_prep<IO, D, true, false>),
                              reinterpret_cast<const void *>(&chunk_prep<IO, D, true, true>)};
        for (const void *f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cfg::BYTES);
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    const long long units = (long long)a.B * a.Hv * a.NC;
    if (units > 0) {
        // Persistent: one workgroup per compute unit (the LDS footprint allows one).
        const long long grid = units < device_cus() ? units : device_cus();
        const bool chan = a.decay == DECAY_CHANNEL, bw = a.beta == nullptr;
        if (chan && bw) hipLaunchKernelGGL((chunk_prep<IO, D, true, true>), dim3((unsigned)grid), dim3(Cfg::NT), Cfg::BYTES, s, a);
        else if (chan) hipLaunchKernelGGL((chunk_prep<IO, D, true, false>), dim3((unsigned)grid), dim3(Cfg::NT), Cfg::BYTES, s, a);
        else if (bw) hipLaunchKernelGGL((chunk_prep<IO, D, false, true>), dim3((unsigned)grid), dim3(Cfg::NT), Cfg::BYTES, s, a);
        else hipLaunchKernelGGL((chunk_prep<IO, D, false, false>), dim3((unsigned)grid), dim3(Cfg::NT), Cfg::BYTES, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NVT = D / (16 * NCT);
    const int G = a.B * a.Hv * NVT;
    const int grid = (G + 7) / 8 * 8;
    constexpr int PF = sizeof(IO) == 2 ? 3 : 1;  // prefetch depth (fp32 fragments are 2x larger)
    hipLaunchKernelGGL((chunk_sweep<IO, D, NCT, PF>), dim3(grid), dim3(2 * D), 0, s, a, NVT, G);
    return hipGetLastError();
}

bool chunk_supported(int io, int D) {
    if (io == IO_BF16) return D == 32 || D == 64 || D == 128;
    return D == 32 || D == 64;
}

hipError_t launch_chunk(int io, int D, const ChunkArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_chunk_t<bf16_t, 32, 1>(a, s);
        if (D == 64) return launch_chunk_t<bf16_t, 64, 2>(a, s);
        if (D == 128) return launch_chunk_t<bf16_t, 128, 2>(a, s);
    } else {
        if (D == 32) return launch_chunk_t<float, 32, 1>(a, s);
        if (D == 64) return launch_chunk_t<float, 64, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
