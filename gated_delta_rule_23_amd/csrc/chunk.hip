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
//   O = s (Q~ S_c + A U)
//   S_{c+1} = Diag(gamma) S_c + Kend^T U
//
// Two kernels. chunk_prep is parallel over every (sequence, V head, chunk):
// it does everything that does not depend on the state -- prefix sums, decay
// absorption, both Gram products, the triangular solve for Y and U_z -- and
// stores Y, Q~, Kend^T, U_z^T, A and gamma in a workspace, each matrix in
// the order the sweep's matrix-core operand loads read it. chunk_sweep is the
// single sequential pass over chunks: per (sequence, V head, value tile) it
// keeps the fp32 state in matrix-core accumulator registers and per chunk
// does U = U_z - Y S_c, O = s (Q~ S_c + A U) and
// S_{c+1} = gamma . S_c + Kend^T U. Value columns of the state evolve
// independently, so the sweep is split over value tiles.
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

// Workspace matrices are stored in "fragment order": the data one wave's
// matrix-core operand load needs is contiguous. For a row-major R x K matrix
// read as A (or B^T) operand fragments, the fragment (row tile rt, K step ks)
// is one block of 64 lanes x FE elements (FE = KS / 4: 8 for bf16, 1 for
// fp32), lane l holding row 16 rt + l % 16, columns KS ks + FE (l / 16) ...
template <typename IO>
__device__ __forceinline__ size_t frag_off(int r, int c, int K) {
    constexpr int KS = Mma<IO>::KS, FE = KS / 4;
    const int lane = (r & 15) + 16 * ((c % KS) / FE);
    return ((size_t)((r >> 4) * (K / KS) + c / KS) * 64 + lane) * FE + c % FE;
}
template <typename IO>
__device__ __forceinline__ typename Mma<IO>::Frag load_frag(const IO *M, int rt, int ks, int K) {
    constexpr int KS = Mma<IO>::KS, FE = KS / 4;
    return *reinterpret_cast<const typename Mma<IO>::Frag *>(M + ((size_t)(rt * (K / KS) + ks) * 64 + (threadIdx.x & 63)) * FE);
}
// ... and a token-contiguous D x C matrix read in accumulator layout (lane
// l = col % 16 + 16 (tok % 16) / 4 holds 4 consecutive tokens of one column)
// is stored as one block of 64 lanes x 4 elements per (token tile, column tile).
template <int D>
__device__ __forceinline__ size_t cfrag_off(int col, int tok) {
    const int lane = (col & 15) + 16 * ((tok & 15) >> 2);
    return ((size_t)((tok >> 4) * (D / 16) + (col >> 4)) * 64 + lane) * 4 + (tok & 3);
}

// Store a row-major R x K matrix from shared memory in fragment order,
// optionally scaling row r by rowscale[r].
template <typename IO>
__device__ __forceinline__ void store_frag_rows(IO *dst, int R, int K, const IO *src, int sld, const float *rowscale,
                                                int tid, int nt) {
    constexpr int V = 16 / sizeof(IO);
    const int per = K / V;
    for (int i = tid; i < R * per; i += nt) {
        const int r = i / per, c0 = (i - r * per) * V;
        IO vals[V];
        *reinterpret_cast<uint4 *>(vals) = *reinterpret_cast<const uint4 *>(src + r * sld + c0);
        if (rowscale) {
            const float sc = rowscale[r];
#pragma unroll
            for (int j = 0; j < V; ++j) vals[j] = Elem<IO>::to(Elem<IO>::from(vals[j]) * sc);
        }
        if constexpr (sizeof(IO) == 2) {  // V == FE: one fragment slot
            *reinterpret_cast<uint4 *>(dst + frag_off<IO>(r, c0, K)) = *reinterpret_cast<const uint4 *>(vals);
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) dst[frag_off<IO>(r, c0 + j, K)] = vals[j];
        }
    }
}

// Store a token-contiguous D x C matrix (row stride sld) in accumulator fragment order.
template <typename IO, int D>
__device__ __forceinline__ void store_cfrag(IO *dst, const IO *src, int sld, int tid, int nt) {
    for (int i = tid; i < D * (C / 4); i += nt) {
        const int col = i / (C / 4), t4 = (i - col * (C / 4)) * 4;
        *reinterpret_cast<typename Raw4<IO>::type *>(dst + cfrag_off<D>(col, t4)) =
            *reinterpret_cast<const typename Raw4<IO>::type *>(src + col * sld + t4);
    }
}

// The 10 lower-triangular 16 x 16 tiles of a 64 x 64 matrix.
__device__ __forceinline__ void lower_tile(int idx, int &ti, int &tj) {
    ti = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
    tj = idx - ti * (ti + 1) / 2;
}

// exp(x) = 2^(x log2 e) on the hardware exp2 (v_exp_f32, ~1 ulp).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

template <typename IO, int D>
struct PrepCfg {
    static constexpr int NW = D / 16 < 4 ? D / 16 : 4;  // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int CQ = D / 4;              // channel quads
    static constexpr int NGRP = NT / CQ;          // token groups
    static constexpr int TPT = C / NGRP;          // tokens per thread in the elementwise phase
    static constexpr int NCTS = 2 * D / NW / 16;  // 16-wide right-hand-side column tiles per wave
    static constexpr int WC = 16 * NCTS;          // right-hand-side columns per wave
    static constexpr int PD = D + 8;              // row stride of [C x D] row-major tiles
    static constexpr int PT = C + 8;              // row stride of token-contiguous tiles
    static constexpr int PDB = sizeof(IO) == 2 ? 24 : 20;   // D_b rows (16 + pad)
    static constexpr int PTMP = sizeof(IO) == 2 ? 24 : 20;  // solve temporaries (16 tokens + pad)
    static constexpr size_t SLOT = a16(cmax((size_t)C * PD, (size_t)D * PT) * sizeof(IO));
    static constexpr size_t SLOT_E = a16(cmax(SLOT, (size_t)NW * WC * PTMP * sizeof(IO)));
    static constexpr size_t XT = a16((size_t)2 * D * PT * sizeof(IO));
    static constexpr size_t TA = a16((size_t)2 * C * PT * sizeof(IO));
    static constexpr size_t TD = a16((size_t)4 * 16 * 17 * 4);
    static constexpr size_t DB = a16((size_t)4 * 16 * PDB * sizeof(IO));
    static constexpr size_t PART = a16((size_t)NGRP * D * 4);
    static constexpr size_t GT = a16((size_t)4 * C * 4);  // per-token G, exp(G), exp(G_end - G), beta
    static constexpr size_t OFF_K = SLOT_E, OFF_Q = OFF_K + SLOT, OFF_XT = OFF_Q + SLOT, OFF_TA = OFF_XT + XT,
                            OFF_TD = OFF_TA + TA, OFF_DB = OFF_TD + TD, OFF_PART = OFF_DB + DB,
                            OFF_GT = OFF_PART + PART, BYTES = OFF_GT + GT;
    static_assert(TA >= (size_t)D * PT * sizeof(IO), "Kend^T staging");
    static_assert(NGRP * TPT == C && TPT % 4 == 0, "elementwise mapping");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// One thread's raw inputs for a chunk: TPT tokens x 4 channels of q, k, v
// (and b, w, per-channel g); lane l of every wave also holds token l's beta
// and scalar g. Kept raw so that the loads for the next chunk are issued
// early and waited for only when used.
template <typename IO, int D, bool CHAN, bool BW>
struct PrepIn {
    using R4 = Raw4<IO>;
    static constexpr int TPT = PrepCfg<IO, D>::TPT;
    typename R4::type q[TPT], k[TPT], v[TPT], bg[BW ? TPT : 1], wg[BW ? TPT : 1];
    f32x4 g[CHAN ? TPT : 1];
    float betal, gs;

    __device__ __forceinline__ void load(const ChunkArgs &a, int u, int cq, int grp) {
        const int NC = a.NC, c = u % NC, bh = u / NC, b = bh / a.Hv, h = bh - b * a.Hv;
        const int hq = h / (a.Hv / a.Hqk), t0 = c * C, n = min(C, a.T - t0);
        const int l = threadIdx.x & 63;
        const size_t row0 = (size_t)b * a.T + t0;  // first token row of the chunk
        const IO *qb = static_cast<const IO *>(a.q) + (row0 * a.Hqk + hq) * D + 4 * cq;
        const IO *kb = static_cast<const IO *>(a.k) + (row0 * a.Hqk + hq) * D + 4 * cq;
        const size_t vo = (row0 * a.Hv + h) * D + 4 * cq;
        const int sqk = a.Hqk * D, sv = a.Hv * D;  // token strides (elements)
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const int t = min(TPT * grp + j, n - 1);  // clamped: padded tokens are zeroed at use
            q[j] = R4::load(qb + t * sqk);
            k[j] = R4::load(kb + t * sqk);
            v[j] = R4::load(static_cast<const IO *>(a.v) + vo + t * sv);
            if constexpr (BW) {
                bg[j] = R4::load(static_cast<const IO *>(a.bg) + vo + t * sv);
                wg[j] = R4::load(static_cast<const IO *>(a.wg) + vo + t * sv);
            }
            if constexpr (CHAN) g[j] = *reinterpret_cast<const f32x4 *>(a.g + vo + t * sv);
        }
        if (threadIdx.x < 64) {  // wave 0: one token per lane
            const size_t tl = (row0 + min(l, n - 1)) * a.Hv + h;
            if constexpr (!BW) betal = a.beta[tl];
            if constexpr (!CHAN) gs = a.decay == DECAY_SCALAR ? a.g[tl] : 0.f;
        }
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
//     matrix-core products; each wave solves its own WC right-hand-side columns.
// Workspace per unit, in fragment order: Y, Q~ (C x D), Kend^T (D x C), A
// (C x C) as matrix-core operands, U_z^T in accumulator layout; gamma. Threads of the elementwise phase run token-fast
// (grp = tid % NGRP) so the token-contiguous stores of neighbouring lanes are
// adjacent in LDS.
template <typename IO, int D, bool CHAN, bool BW>
__global__ __launch_bounds__(D >= 64 ? 256 : 128) void chunk_prep(ChunkArgs a) {  // = PrepCfg<IO, D>::NT
    using E = Elem<IO>;
    using M = Mma<IO>;
    using R4 = Raw4<IO>;
    using Cfg = PrepCfg<IO, D>;
    constexpr int NW = Cfg::NW, NT = Cfg::NT, PD = Cfg::PD, PT = Cfg::PT;
    constexpr int NGRP = Cfg::NGRP, TPT = Cfg::TPT, NCTS = Cfg::NCTS, WC = Cfg::WC;
    constexpr int PDB = Cfg::PDB, PTMP = Cfg::PTMP, KS = M::KS;
    constexpr int NG = (20 + NW - 1) / NW;  // Gram tile products per wave
    static_assert(NT == (D >= 64 ? 256 : 128), "launch bounds");

    extern __shared__ __align__(16) unsigned char smem[];
    IO *sE = reinterpret_cast<IO *>(smem);                    // E~ (or raw e) [C][PD] -> solve temporaries
    IO *sK = reinterpret_cast<IO *>(smem + Cfg::OFF_K);       // K~ (or raw k) [C][PD] -> Y staging [C][PD]
    IO *sQ = reinterpret_cast<IO *>(smem + Cfg::OFF_Q);       // Q~ (or raw q) [C][PD]
    IO *sXT = reinterpret_cast<IO *>(smem + Cfg::OFF_XT);     // [E~ | Z]^T [2D][PT] -> [Y | U_z]^T in place
    IO *sTo = reinterpret_cast<IO *>(smem + Cfg::OFF_TA);     // -T without its diagonal blocks [C][PT]
    IO *sA = sTo + C * PT;                                     // A [C][PT]
    IO *sKT = sTo;                                             // Kend^T staging [D][PT] (phase A only)
    float *sTd = reinterpret_cast<float *>(smem + Cfg::OFF_TD);      // T diagonal blocks, column-major [4][16][17]
    IO *sDb = reinterpret_cast<IO *>(smem + Cfg::OFF_DB);            // their inverses [4][16][PDB]
    float *sPart = reinterpret_cast<float *>(smem + Cfg::OFF_PART);  // [NGRP][D] per-group channel sums
    float *sG = reinterpret_cast<float *>(smem + Cfg::OFF_GT);       // per token: G,
    float *sEG = sG + C;                                             //   exp(G),
    float *sER = sG + 2 * C;                                         //   exp(G_end - G),
    float *sBt = sG + 3 * C;                                         //   beta
    IO *sYs = sK;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;
    const int grp = tid % NGRP, cq = tid / NGRP;
    const int units = a.B * a.Hv * a.NC;
    IO *tmp = sE + w * WC * PTMP;

    PrepIn<IO, D, CHAN, BW> in;
    if ((int)blockIdx.x < units) in.load(a, blockIdx.x, cq, grp);

    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int NC = a.NC, c = u % NC;
        const int n = min(C, a.T - c * C);
        IO *ws = static_cast<IO *>(a.ws_io) + (size_t)u * chunk_ws_io_elems(D);
        IO *wY = ws, *wQ = ws + C * D, *wKT = ws + 2 * C * D, *wUzT = ws + 3 * C * D, *wA = ws + 4 * C * D;
        __syncthreads();  // the previous unit's readers of shared memory are done

        // ---- A. prefix sums and decay absorption ----
        float G[TPT][4];
        if constexpr (CHAN) {
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int ch = 0; ch < 4; ++ch)
                    G[j][ch] = (TPT * grp + j < n ? in.g[j][ch] : 0.f) + (j > 0 ? G[j - 1][ch] : 0.f);
            store4f(sPart + grp * D + 4 * cq, f32x4{G[TPT - 1][0], G[TPT - 1][1], G[TPT - 1][2], G[TPT - 1][3]});
        } else if (w == 0) {
            // Scalar decay: wave 0 scans the 64 token values (lane = token) into tables.
            float Gl = l < n ? in.gs : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(Gl, off);
                if (l >= off) Gl += y;
            }
            sG[l] = Gl;
            sEG[l] = fast_exp(Gl);
            sER[l] = fast_exp(__shfl(Gl, 63) - Gl);
        }
        if constexpr (!BW)
            if (w == 0) sBt[l] = in.betal;
        __syncthreads();
        float Gend[4], eGend[4];
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
            for (int ch = 0; ch < 4; ++ch) {
                Gend[ch] = tot[ch];
                eGend[ch] = fast_exp(tot[ch]);
            }
        } else {
            const float e = sEG[C - 1];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) eGend[ch] = e;
        }

#pragma unroll
        for (int h4 = 0; h4 < TPT / 4; ++h4) {  // 4 tokens at a time
            const int t4 = TPT * grp + 4 * h4;
            f32x4 egt4 = zero4(), ert4 = zero4(), bt4 = zero4();
            if constexpr (!CHAN) { egt4 = load4f(sEG + t4); ert4 = load4f(sER + t4); }
            if constexpr (!BW) bt4 = load4f(sBt + t4);
            float xE[4][4], xZ[4][4], xKe[4][4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = 4 * h4 + jj, tk = t4 + jj;
                const bool valid = tk < n;
                const f32x4 kk = R4::widen(in.k[j]), qq = R4::widen(in.q[j]), vv = R4::widen(in.v[j]);
                f32x4 eb, wz;
                if constexpr (BW) {
                    eb = R4::widen(in.bg[j]);
                    wz = R4::widen(in.wg[j]);
                } else {
                    eb = f32x4{bt4[jj], bt4[jj], bt4[jj], bt4[jj]};
                    wz = eb;
                }
                float gE[4], gK[4], gQ[4];
#pragma unroll
                for (int ch = 0; ch < 4; ++ch) {
                    const float kv = valid ? kk[ch] : 0.f, qv = valid ? qq[ch] : 0.f;
                    const float ev = eb[ch] * kv;
                    xZ[jj][ch] = valid ? wz[ch] * vv[ch] : 0.f;
                    if constexpr (CHAN) {  // factored form for the Gram
                        const float eg = fast_exp(G[j][ch]), emg = __builtin_amdgcn_rcpf(eg);
                        xE[jj][ch] = ev * eg;
                        xKe[jj][ch] = kv * (eGend[ch] * emg);
                        gE[ch] = xE[jj][ch];
                        gK[ch] = kv * emg;
                        gQ[ch] = qv * eg;
                    } else {  // raw operands; the decay is applied to the Gram entries
                        xE[jj][ch] = ev * egt4[jj];
                        xKe[jj][ch] = kv * ert4[jj];
                        gE[ch] = ev;
                        gK[ch] = kv;
                        gQ[ch] = qv;
                    }
                }
                store4f(sE + tk * PD + 4 * cq, f32x4{gE[0], gE[1], gE[2], gE[3]});
                store4f(sK + tk * PD + 4 * cq, f32x4{gK[0], gK[1], gK[2], gK[3]});
                store4f(sQ + tk * PD + 4 * cq, f32x4{gQ[0], gQ[1], gQ[2], gQ[3]});
            }
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const int cc = 4 * cq + ch;
                store4f(sXT + cc * PT + t4, f32x4{xE[0][ch], xE[1][ch], xE[2][ch], xE[3][ch]});
                store4f(sXT + (D + cc) * PT + t4, f32x4{xZ[0][ch], xZ[1][ch], xZ[2][ch], xZ[3][ch]});
                store4f(sKT + cc * PT + t4, f32x4{xKe[0][ch], xKe[1][ch], xKe[2][ch], xKe[3][ch]});
            }
        }
        if (grp == NGRP - 1)
            store4f(a.ws_gamma + (size_t)u * D + 4 * cq, f32x4{eGend[0], eGend[1], eGend[2], eGend[3]});
        // The raw inputs are consumed: fetch the next unit's now.
        if (u + (int)gridDim.x < units) in.load(a, u + gridDim.x, cq, grp);
        __syncthreads();
        store_frag_rows(wKT, D, C, sKT, PT, nullptr, tid, NT);
        // Q~ for the sweep (scalar decay: the stored raw q times exp(G) per token).
        store_frag_rows(wQ, C, D, sQ, PD, CHAN ? nullptr : sEG, tid, NT);

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
        __syncthreads();  // Kend^T staging copied out (its space becomes -T and A); E~, K~ are dead
#pragma unroll
        for (int s = 0; s < NG; ++s) {
            const int p = w + NW * s;
            if (p < 20) {
                const int kind = p / 10;
                int ti, tj;
                lower_tile(p - kind * 10, ti, tj);
                const int col = tj * 16 + lr, row0 = ti * 16 + 4 * lq;
                f32x4 x = gacc[s];
                if constexpr (!CHAN) {
                    const f32x4 Gr = load4f(sG + row0);
                    const float Gc = sG[col];
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] *= fast_exp(fminf(Gr[r] - Gc, 0.f));
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = row0 + r;
                    if (kind == 0) {
                        if (ti == tj) sTd[(ti * 16 + lr) * 17 + 4 * lq + r] = col < row ? x[r] : 0.f;  // column-major
                        else sTo[row * PT + col] = E::to(-x[r]);
                    } else {
                        sA[row * PT + col] = E::to(col <= row ? x[r] : 0.f);
                    }
                }
            }
        }
        // Zero tiles, 16 bytes at a time: -T on and above the diagonal blocks, A above them.
        {
            constexpr int V = 16 / sizeof(IO);
#pragma unroll
            for (int i = tid; i < C * C / V; i += NT) {
                const int row = i / (C / V), col = (i - row * (C / V)) * V;
                if ((col >> 4) >= (row >> 4)) *reinterpret_cast<uint4 *>(sTo + row * PT + col) = uint4{0, 0, 0, 0};
                if ((col >> 4) > (row >> 4)) *reinterpret_cast<uint4 *>(sA + row * PT + col) = uint4{0, 0, 0, 0};
            }
        }
        __syncthreads();
        store_frag_rows(wA, C, C, sA, PT, nullptr, tid, NT);

        // ---- C. diagonal block inverses: right-looking fp32 substitution, one column per lane ----
        for (int blk = w; blk < 4; blk += NW) {
            if (lr == l) {  // lanes 0..15
                const float *Tb = sTd + blk * 16 * 17;  // column m at Tb + 17 m
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = i == lr ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < 15; ++m) {
                    float col[16];
#pragma unroll
                    for (int i = m + 1; i < 16; ++i) col[i] = Tb[m * 17 + i];
#pragma unroll
                    for (int i = m + 1; i < 16; ++i) x[i] -= col[i] * x[m];
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) sDb[(blk * 16 + i) * PDB + lr] = E::to(x[i]);
            }
        }
        __syncthreads();

        // ---- C. blocked forward substitution; wave w owns columns WC*w..WC*w+WC-1 of [E~ | Z] ----
        const bool yside = WC * w < D;
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
                const f32x4 x = Mma16<IO>::step(zero4(), sDb + blk * 16 * PDB, PDB, tmp + 16 * ct * PTMP, PTMP);
                const int col = WC * w + 16 * ct + lr, tok = 16 * blk + 4 * lq;
                store4f(sXT + col * PT + tok, x);
                if (yside)  // Y also row-major, for the workspace
#pragma unroll
                    for (int r = 0; r < 4; ++r) sYs[(tok + r) * PD + col] = E::to(x[r]);
            }
        }
        __syncthreads();

        // Workspace stores: Y row-major; U_z^T.
        store_frag_rows(wY, C, D, sYs, PD, nullptr, tid, NT);
        store_cfrag<IO, D>(wUzT, sXT + D * PT, PT, tid, NT);
    }
}

// Sequential sweep over chunks for one (sequence, V head, value tile of BV =
// 16*NCT columns). NW = D/32 waves; wave w keeps state rows 32w..32w+31 in
// accumulator layout and computes token tiles [w*TPW, (w+1)*TPW) of the
// outputs. Per chunk:
//   P = Y S_c, R = Q~ S_c          (S_c^T shared through LDS)
//   U = U_z - P                    (U^T shared through LDS)
//   O = s (R + A U)
//   S_{c+1} = gamma . S_c + Kend^T U
// Each wave reads only its own slice of a chunk's factors (its token rows of
// Y, Q~ and A, its channel rows of Kend^T), so those slices are prefetched
// into registers PF chunks ahead and the global-memory latency leaves the chain.
template <typename IO, int D, int NCT>
struct SweepOps {
    using M = Mma<IO>;
    using F = typename M::Frag;
    using R4 = Raw4<IO>;
    static constexpr int NW = D / 32, TPW = 4 / NW, KD = D / M::KS, KC = C / M::KS;
    F ya[TPW][KD], qa[TPW][KD], aa[TPW][KC], ka[2][KC];
    typename R4::type uz[TPW][NCT];
    f32x4 g4[2];

    __device__ __forceinline__ void load(const IO *wsb, const float *wsg, size_t u, int w, int col0) {
        const int l = threadIdx.x & 63, lq = l >> 4;
        const IO *Y = wsb + u * chunk_ws_io_elems(D), *Qt = Y + C * D, *KT = Qt + C * D, *UzT = KT + D * C,
                 *A = UzT + D * C;
        const float *gam = wsg + u * D;
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int rt = w * TPW + tt;
#pragma unroll
            for (int ks = 0; ks < KD; ++ks) {
                ya[tt][ks] = load_frag(Y, rt, ks, D);
                qa[tt][ks] = load_frag(Qt, rt, ks, D);
            }
#pragma unroll
            for (int ks = 0; ks < KC; ++ks) aa[tt][ks] = load_frag(A, rt, ks, C);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                uz[tt][ct] = R4::load(UzT + ((size_t)(rt * (D / 16) + col0 / 16 + ct) * 64 + l) * 4);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int ch0 = 32 * w + 16 * rt;
#pragma unroll
            for (int ks = 0; ks < KC; ++ks) ka[rt][ks] = load_frag(KT, ch0 / 16, ks, C);
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
                                            IO *sO, IO *orow0, size_t orow_stride, int n_valid, float scale) {
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

    f32x4 accR[TPW][NCT];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int T0 = (w * TPW + tt) * 16;
        f32x4 accP[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) { accP[ct] = zero4(); accR[tt][ct] = zero4(); }
#pragma unroll
        for (int ks = 0; ks < KD; ++ks) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const F sb = M::load(sST + 16 * ct * LS + ks * KS, LS);
                accP[ct] = M::mma(accP[ct], op.ya[tt][ks], sb);
                accR[tt][ct] = M::mma(accR[tt][ct], op.qa[tt][ks], sb);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            store4f(sUT + (16 * ct + lr) * LU + T0 + 4 * lq, Ops::R4::widen(op.uz[tt][ct]) - accP[ct]);
    }
    __syncthreads();

    // O = s (R + A U); U fragments come from LDS and also feed the state update.
    F ub[KC][NCT];
#pragma unroll
    for (int ks = 0; ks < KC; ++ks)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) ub[ks][ct] = M::load(sUT + 16 * ct * LU + ks * KS, LU);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const int T0 = (w * TPW + tt) * 16;
        // All K steps (A is zero above its diagonal tiles): a trip count that
        // depends on the wave would put branches around the prefetch
        // bookkeeping and force a full drain of the loads in flight.
#pragma unroll
        for (int ks = 0; ks < KC; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) accR[tt][ct] = M::mma(accR[tt][ct], op.aa[tt][ks], ub[ks][ct]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sO[(T0 + 4 * lq + r) * LO + 16 * ct + lr] = Elem<IO>::to(scale * accR[tt][ct][r]);
        // This wave's output rows, 16 bytes per lane (wave-local staging).
        constexpr int V = 16 / sizeof(IO), PER = BV / V;
#pragma unroll
        for (int i = l; i < 16 * PER; i += 64) {
            const int tok = T0 + i / PER, c8 = (i % PER) * V;
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
            for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = M::mma(S[rt][ct], op.ka[rt][ks], ub[ks][ct]);
    }
}

template <typename IO, int D, int NCT, int PF>
__global__ __launch_bounds__(2 * D) void chunk_sweep(ChunkArgs a, int NVT, int G) {
    using Ops = SweepOps<IO, D, NCT>;
    constexpr int BV = 16 * NCT;
    constexpr int LS = D + 8, LU = C + 8, LO = BV + 8;
    __shared__ __align__(16) IO sST[BV * LS];  // S_c^T in the io dtype
    __shared__ __align__(16) IO sUT[BV * LU];  // U^T in the io dtype
    __shared__ __align__(16) IO sO[C * LO];    // output rows (each wave stages its own)

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
                                               orow_stride, C, a.scale);
                ring[j].load(wsb, a.ws_gamma, u0 + min(c + j + PF, NC - 1), w, col0);
            }
        }
        // Remainder: ring slot j holds chunk c + j (clamped); the last chunk may be partial.
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int cj = c + j;
            if (cj < NC)
                sweep_chunk<IO, D, NCT, true>(ring[j], S, sST, sUT, sO, obase + (size_t)cj * C * orow_stride,
                                              orow_stride, a.T - cj * C, a.scale);
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
    constexpr int PF = sizeof(IO) == 2 ? SWEEP_PF : 1;  // prefetch depth (fp32 fragments are 2x larger)
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
        if (D == 128) return launch_chunk_t<bf16_t, 128, SWEEP_NCT128>(a, s);
    } else {
        if (D == 32) return launch_chunk_t<float, 32, 1>(a, s);
        if (D == 64) return launch_chunk_t<float, 64, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
