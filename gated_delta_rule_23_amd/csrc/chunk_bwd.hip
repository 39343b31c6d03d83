// chunk_bwd.hip -- gradients of the gated delta-rule recurrence, chunked form.
//
// The page "Resumo Técnico: Gated DeltaNet-2", section "Treinamento Paralelo
// Eficiente por Blocos", names a backward pass that is parallel over blocks
// of tokens and in which the gates enter the gradient accumulation; it prints
// no formula. What is computed here is the exact gradient of the chunked
// forward of the page "Gated Delta Networks", sections on the chunked
// (WY/UT) form, which equals the token recurrence. Per (sequence, V head) and
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
// With a per-channel decay T and A are formed as E~ K~^T and Q~ K~^T with
// K~ = k . exp(-G) (as in the forward); with a scalar decay the exponentials
// are kept per entry, exp(G_t - G_j) <= 1, so strong decays stay finite.
//
// Five launches, all arithmetic in fp32:
//  1. cb_prep (per chunk unit): G, the factors above, T and A, and the
//     triangular solve (I + T)[Y | U_z] = [E~ | Z] by forward substitution.
//  2. cb_fsweep (per sequence, V head, 32 value columns): the states S
//     entering every chunk, and U, walking the chunks forward.
//  3. cb_bsweep (same work items): dS_next of every chunk and dU, walking the
//     chunks backward; dS_0 at the end.
//  4. cb_grad_s (per unit): dR by back substitution, dT, dA and the products
//     with S and dS_next.
//  5. cb_grad_out (per unit): the products through T and A, the exponential
//     factors, the gates, and the reverse sums over the chunk giving dg; then
//     (grouped heads) cb_group_sum adds the V heads' dq and dk per QK head.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {
namespace {

constexpr int C = kChunk;
constexpr int NT = 256;  // threads per workgroup
constexpr int BV = 32;   // value columns per sweep workgroup
constexpr int PB = BV + 1, PC = C + 1;

template <typename IO>
__device__ __forceinline__ float ldio(const void *p, size_t i) {
    return Elem<IO>::load(static_cast<const IO *>(p) + i);
}

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

template <int D>
constexpr size_t prep_smem() {
    return ((size_t)(C * (D + 1) > C * PC ? C * (D + 1) : C * PC) + 3 * (size_t)C * (D + 1) + C) * 4;
}
template <int D>
constexpr size_t grad_s_smem() {
    return ((size_t)C * PC + 3 * (size_t)C * (D + 1) + 32 * (size_t)(D + 1)) * 4;
}
template <int D>
constexpr size_t grad_out_smem() {
    return (3 * (size_t)C * (D + 1) + 2 * (size_t)C * PC + 2 * C + 4 * C + 2 * 16 * C + 16 * (size_t)D + D) * 4;
}

// ---------------------------------------------------------------------------
// 1. Per chunk unit: G, E~, Q~, Kend, Gamma, T, A, then [Y | U_z].
template <typename IO, int D, bool CHAN, bool BW>
__global__ __launch_bounds__(NT) void cb_prep(ChunkBwdArgs a) {
    constexpr int PD = D + 1, R0 = C * PD > C * PC ? C * PD : C * PC;
    extern __shared__ __align__(16) float smem[];
    float *sQ = smem;           // q (Q~ with a per-channel decay); then T
    float *sK = sQ + R0;        // k (K~)
    float *sE = sK + C * PD;    // e, then E~, then Y
    float *sZ = sE + C * PD;    // per-channel decay: g, then G; then z, then U_z
    float *sGs = sZ + C * PD;   // scalar decay: G per token
    const int tid = threadIdx.x, u = blockIdx.x;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D;

    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        float qv = 0.f, kv = 0.f, ev = 0.f, gv = 0.f;
        if (t < x.n) {
            const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + d, iv = (x.rowv + (size_t)t * a.Hv) * D + d;
            qv = ldio<IO>(a.q, iq);
            kv = ldio<IO>(a.k, iq);
            ev = (BW ? ldio<IO>(a.bg, iv) : a.beta[x.rowv + (size_t)t * a.Hv]) * kv;
            if (CHAN) gv = a.g[iv];
        }
        sQ[t * PD + d] = qv;
        sK[t * PD + d] = kv;
        sE[t * PD + d] = ev;
        if (CHAN) sZ[t * PD + d] = gv;
    }
    if (!CHAN && tid < C) sGs[tid] = a.g && tid < x.n ? a.g[x.rowv + (size_t)tid * a.Hv] : 0.f;
    __syncthreads();
    if (CHAN) {
        if (tid < D) {
            float acc = 0.f;
            for (int t = 0; t < C; ++t) {
                acc += sZ[t * PD + tid];
                sZ[t * PD + tid] = acc;
            }
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
    __syncthreads();

    float *wG = a.wG + ucd;  // [C][D] per-channel decay, [C] scalar
    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        const float G = CHAN ? sZ[t * PD + d] : sGs[t];
        const float Ge = CHAN ? sZ[(C - 1) * PD + d] : sGs[C - 1];
        const float eg = expf(G), qv = sQ[t * PD + d], kv = sK[t * PD + d];
        a.wQt[ucd + i] = qv * eg;
        a.wKe[ucd + i] = kv * expf(Ge - G);
        if (CHAN) {
            wG[i] = G;
            sQ[t * PD + d] = qv * eg;
            sK[t * PD + d] = kv * expf(-G);
            sE[t * PD + d] *= eg;
        }
    }
    if (!CHAN && tid < C) wG[tid] = sGs[tid];
    if (tid < D) a.wGam[(size_t)u * D + tid] = expf(CHAN ? sZ[(C - 1) * PD + tid] : sGs[C - 1]);
    __syncthreads();

    // T and A: thread = 4 x 4 block of rows r0.., columns c0..
    {
        const int r0 = (tid >> 4) * 4, c0 = (tid & 15) * 4;
        float aT[4][4], aA[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) aT[i][j] = aA[i][j] = 0.f;
        if (c0 <= r0 + 3)
            for (int d = 0; d < D; ++d) {
                float e4[4], q4[4], k4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e4[i] = sE[(r0 + i) * PD + d];
                    q4[i] = sQ[(r0 + i) * PD + d];
                    k4[i] = sK[(c0 + i) * PD + d];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        aT[i][j] = fmaf(e4[i], k4[j], aT[i][j]);
                        aA[i][j] = fmaf(q4[i], k4[j], aA[i][j]);
                    }
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = r0 + i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int jj = c0 + j;
                const float f = !CHAN && jj <= t ? expf(sGs[t] - sGs[jj]) : 1.f;
                aT[i][j] = jj < t ? aT[i][j] * f : 0.f;
                aA[i][j] = jj <= t ? aA[i][j] * f : 0.f;
            }
            const size_t o = (size_t)u * C * C + (size_t)t * C + c0;
            *reinterpret_cast<f32x4 *>(a.wT + o) = f32x4{aT[i][0], aT[i][1], aT[i][2], aT[i][3]};
            *reinterpret_cast<f32x4 *>(a.wA + o) = f32x4{aA[i][0], aA[i][1], aA[i][2], aA[i][3]};
        }
        __syncthreads();  // q, k and e tiles read: T goes where q was
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) sQ[(r0 + i) * PC + c0 + j] = aT[i][j];
    }
    // Right-hand sides: E~ (scalar decay: the raw e scaled by exp(G_t)) and z.
    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        if (!CHAN) sE[t * PD + d] *= expf(sGs[t]);
        float zv = 0.f;
        if (t < x.n) {
            const size_t iv = (x.rowv + (size_t)t * a.Hv) * D + d;
            zv = (BW ? ldio<IO>(a.wg, iv) : a.beta[x.rowv + (size_t)t * a.Hv]) * ldio<IO>(a.v, iv);
        }
        sZ[t * PD + d] = zv;
    }
    __syncthreads();
    // (I + T) X = [E~ | Z], column by column, rows in order: X_i = R_i - sum_{m<i} T_im X_m.
    if (tid < 2 * D) {
        const float *sT = sQ;
        float *X = tid < D ? sE + tid : sZ + (tid - D);
        for (int i = 1; i < C; ++i) {
            float p0 = X[i * PD], p1 = 0.f;
            int m = 0;
            for (; m + 1 < i; m += 2) {
                p0 = fmaf(-sT[i * PC + m], X[m * PD], p0);
                p1 = fmaf(-sT[i * PC + m + 1], X[(m + 1) * PD], p1);
            }
            if (m < i) p0 = fmaf(-sT[i * PC + m], X[m * PD], p0);
            X[i * PD] = p0 + p1;
        }
    }
    __syncthreads();
    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        a.wY[ucd + i] = sE[t * PD + d];
        a.wUz[ucd + i] = sZ[t * PD + d];
    }
}

// ---------------------------------------------------------------------------
// 2. Forward over chunks for one (sequence, V head, 32 value columns): the
//    state entering each chunk, and U = U_z - Y S.
template <int D>
__global__ __launch_bounds__(NT) void cb_fsweep(ChunkBwdArgs a) {
    constexpr int NTL = D / BV, TPR = NT / D, CPT = BV / TPR;
    __shared__ float sS[D * PB];
    __shared__ float sU[C * PB];
    const int tid = threadIdx.x, tile = blockIdx.x % NTL, bh = blockIdx.x / NTL, col0 = tile * BV;
    const size_t sb = (size_t)bh * D * D;
    for (int i = tid; i < D * BV; i += NT) {
        const int d = i / BV, j = i - d * BV;
        sS[d * PB + j] = a.S0 ? a.S0[sb + (size_t)d * D + col0 + j] : 0.f;
    }
    __syncthreads();
    const int ut = tid >> 2, uj = (tid & 3) * 8;       // U: row ut, columns uj..uj+7
    const int sd = tid / TPR, sj = (tid % TPR) * CPT;  // S: row sd, columns sj..
    for (int c = 0; c < a.NC; ++c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        for (int i = tid; i < D * BV; i += NT) {
            const int d = i / BV, j = i - d * BV;
            a.wS[u * D * D + (size_t)d * D + col0 + j] = sS[d * PB + j];
        }
        float acc[8];
        const float *Y = a.wY + ucd + (size_t)ut * D;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = a.wUz[ucd + (size_t)ut * D + col0 + uj + j];
        for (int d = 0; d < D; d += 4) {
            const f32x4 y = *reinterpret_cast<const f32x4 *>(Y + d);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = fmaf(-y[r], sS[(d + r) * PB + uj + j], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sU[ut * PB + uj + j] = acc[j];
            a.wU[ucd + (size_t)ut * D + col0 + uj + j] = acc[j];
        }
        __syncthreads();
        const float gam = a.wGam[u * D + sd];
        float s[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) s[j] = gam * sS[sd * PB + sj + j];
        const float *Ke = a.wKe + ucd + sd;
        for (int t = 0; t < C; ++t) {
            const float kv = Ke[(size_t)t * D];
#pragma unroll
            for (int j = 0; j < CPT; ++j) s[j] = fmaf(kv, sU[t * PB + sj + j], s[j]);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) sS[sd * PB + sj + j] = s[j];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// 3. Backward over chunks for the same work items: X = dL/d(state leaving
//    the chunk), dU, and X for the chunk before.
template <typename IO, int D>
__global__ __launch_bounds__(NT) void cb_bsweep(ChunkBwdArgs a) {
    constexpr int NTL = D / BV, TPR = NT / D, CPT = BV / TPR;
    __shared__ float sX[D * PB];
    __shared__ float sO[C * PB];
    __shared__ float sdU[C * PB];
    const int tid = threadIdx.x, tile = blockIdx.x % NTL, bh = blockIdx.x / NTL, col0 = tile * BV;
    const int b = bh / a.Hv, h = bh - b * a.Hv;
    const size_t sb = (size_t)bh * D * D;
    for (int i = tid; i < D * BV; i += NT) {
        const int d = i / BV, j = i - d * BV;
        sX[d * PB + j] = a.dST ? a.dST[sb + (size_t)d * D + col0 + j] : 0.f;
    }
    const int ut = tid >> 2, uj = (tid & 3) * 8;
    const int sd = tid / TPR, sj = (tid % TPR) * CPT;
    for (int c = a.NC - 1; c >= 0; --c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        const int t0 = c * C, n = min(C, a.T - t0);
        __syncthreads();  // X written; the previous chunk's reads of dO and dU done
        for (int i = tid; i < D * BV; i += NT) {
            const int d = i / BV, j = i - d * BV;
            a.wdS[u * D * D + (size_t)d * D + col0 + j] = sX[d * PB + j];
        }
        for (int i = tid; i < C * BV; i += NT) {
            const int t = i / BV, j = i - t * BV;
            sO[t * PB + j] = t < n ? ldio<IO>(a.dO, (((size_t)b * a.T + t0 + t) * a.Hv + h) * D + col0 + j) : 0.f;
        }
        __syncthreads();
        // dU (row ut) = s sum_{t >= ut} A_t,ut dO_t + Kend_ut X
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.f;
        const float *A = a.wA + u * C * C;
        for (int t = ut; t < C; ++t) {
            const float av = A[(size_t)t * C + ut];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = fmaf(av, sO[t * PB + uj + j], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= a.scale;
        const float *Ke = a.wKe + ucd + (size_t)ut * D;
        for (int d = 0; d < D; d += 4) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(Ke + d);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = fmaf(kv[r], sX[(d + r) * PB + uj + j], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sdU[ut * PB + uj + j] = acc[j];
            a.wdU[ucd + (size_t)ut * D + col0 + uj + j] = acc[j];
        }
        __syncthreads();
        // X (row sd) = Gamma_sd X + s Q~^T dO - Y^T dU
        const float gam = a.wGam[u * D + sd];
        float xa[CPT], qa[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            xa[j] = gam * sX[sd * PB + sj + j];
            qa[j] = 0.f;
        }
        const float *Qt = a.wQt + ucd + sd, *Y = a.wY + ucd + sd;
        for (int t = 0; t < C; ++t) {
            const float qv = Qt[(size_t)t * D], yv = Y[(size_t)t * D];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                qa[j] = fmaf(qv, sO[t * PB + sj + j], qa[j]);
                xa[j] = fmaf(-yv, sdU[t * PB + sj + j], xa[j]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) sX[sd * PB + sj + j] = fmaf(a.scale, qa[j], xa[j]);
    }
    __syncthreads();
    if (a.dS0)
        for (int i = tid; i < D * BV; i += NT) {
            const int d = i / BV, j = i - d * BV;
            a.dS0[sb + (size_t)d * D + col0 + j] = sX[d * PB + j];
        }
}

// ---------------------------------------------------------------------------
// 4. Per unit: dR = L^T dU (solve (I + T)^T dR = dU), dT, dA, and the
//    products with S and dS_next.
template <typename IO, int D>
__global__ __launch_bounds__(NT) void cb_grad_s(ChunkBwdArgs a) {
    constexpr int PD = D + 1;
    extern __shared__ __align__(16) float smem[];
    float *sT = smem, *sX = sT + C * PC, *sU = sX + C * PD, *sO = sU + C * PD, *sB = sO + C * PD;
    const int tid = threadIdx.x, u = blockIdx.x;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C, udd = (size_t)u * D * D;
    for (int i = tid; i < C * C; i += NT) {
        const int t = i / C, j = i - t * C;
        sT[t * PC + j] = a.wT[ucc + i];
    }
    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        sX[t * PD + d] = a.wdU[ucd + i];
        sU[t * PD + d] = a.wU[ucd + i];
        sO[t * PD + d] = t < x.n ? ldio<IO>(a.dO, (x.rowv + (size_t)t * a.Hv) * D + d) : 0.f;
    }
    __syncthreads();
    // Rows from the last: dR_i = dU_i - sum_{m > i} T_mi dR_m.
    if (tid < D) {
        float *X = sX + tid;
        for (int i = C - 2; i >= 0; --i) {
            float p0 = X[i * PD], p1 = 0.f;
            int m = i + 1;
            for (; m + 1 < C; m += 2) {
                p0 = fmaf(-sT[m * PC + i], X[m * PD], p0);
                p1 = fmaf(-sT[(m + 1) * PC + i], X[(m + 1) * PD], p1);
            }
            if (m < C) p0 = fmaf(-sT[m * PC + i], X[m * PD], p0);
            X[i * PD] = p0 + p1;
        }
    }
    __syncthreads();
    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        a.wdU[ucd + i] = sX[t * PD + d];  // dR replaces dU
    }
    {
        const int r0 = (tid >> 4) * 4, c0 = (tid & 15) * 4;
        float aT[4][4], aA[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) aT[i][j] = aA[i][j] = 0.f;
        if (c0 <= r0 + 3)
            for (int v = 0; v < D; ++v) {
                float x4[4], o4[4], u4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x4[i] = sX[(r0 + i) * PD + v];
                    o4[i] = sO[(r0 + i) * PD + v];
                    u4[i] = sU[(c0 + i) * PD + v];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        aT[i][j] = fmaf(x4[i], u4[j], aT[i][j]);
                        aA[i][j] = fmaf(o4[i], u4[j], aA[i][j]);
                    }
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = r0 + i;
            f32x4 dt, da;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dt[j] = c0 + j < t ? -aT[i][j] : 0.f;
                da[j] = c0 + j <= t ? a.scale * aA[i][j] : 0.f;
            }
            *reinterpret_cast<f32x4 *>(a.wdT + ucc + (size_t)t * C + c0) = dt;
            *reinterpret_cast<f32x4 *>(a.wdA + ucc + (size_t)t * C + c0) = da;
        }
    }
    // Products with S, then with dS_next, 32 state rows at a time.
    const int bt = tid >> 2, bd = (tid & 3) * 8;
    for (int pass = 0; pass < 2; ++pass)
        for (int blk = 0; blk < D / 32; ++blk) {
            __syncthreads();
            const float *src = (pass == 0 ? a.wS : a.wdS) + udd + (size_t)blk * 32 * D;
            for (int i = tid; i < 32 * D; i += NT) {
                const int r = i / D, v = i - r * D;
                sB[r * PD + v] = src[i];
            }
            __syncthreads();
            float p[8], q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = q[j] = 0.f;
            const float *L0 = (pass == 0 ? sX : sU) + bt * PD;
            for (int v = 0; v < D; ++v) {
                const float l0 = L0[v], o0 = sO[bt * PD + v];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float sv = sB[(bd + j) * PD + v];
                    p[j] = fmaf(l0, sv, p[j]);
                    if (pass == 0) q[j] = fmaf(o0, sv, q[j]);
                }
            }
            const size_t o = ucd + (size_t)bt * D + blk * 32 + bd;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (pass == 0) {
                    a.wdE[o + j] = -p[j];
                    a.wdQ[o + j] = a.scale * q[j];
                } else {
                    a.wdK[o + j] = p[j];
                }
            }
            if (pass == 1 && tid < 32) {
                const float *Sr = a.wS + udd + (size_t)(blk * 32 + tid) * D;
                float acc = 0.f;
                for (int v = 0; v < D; ++v) acc = fmaf(sB[tid * PD + v], Sr[v], acc);
                a.wdGam[(size_t)u * D + blk * 32 + tid] = acc;
            }
        }
}

// ---------------------------------------------------------------------------
// 5. Per unit: the parts through T and A, the exponential factors, the
//    gates, and dg.
template <typename IO, int D, bool CHAN, bool BW>
__global__ __launch_bounds__(NT) void cb_grad_out(ChunkBwdArgs a) {
    constexpr int PD = D + 1, CT = D / 16;
    extern __shared__ __align__(16) float smem[];
    float *sP1 = smem;            // e (E~): left factor of T
    float *sP2 = sP1 + C * PD;    // k (K~): right factor of T and A
    float *sP3 = sP2 + C * PD;    // q (Q~): left factor of A
    float *sdT = sP3 + C * PD;    // dT, scaled per entry by exp(G_t - G_j) for a scalar decay; then dG [C][PD]
    float *sdA = sdT + C * PC;
    // Reductions go through per-thread partials summed in a fixed order, so
    // that the result does not depend on the order threads arrive in.
    float *sRow = sdA + C * PC;    // [C] row sums of dT . T + dA . A (scalar decay)
    float *sColW = sRow + C;       // [4 waves][C] their column sums
    float *sCol = sColW + 4 * C;   // [C]
    float *sTokG = sCol + C;       // [C][16] per-token dG parts of the 16 column groups (scalar decay)
    float *sTokB = sTokG + 16 * C; // [C][16] per-token dbeta parts (tied gates)
    float *sGeP = sTokB + 16 * C;  // [16 row groups][D] dG_end parts
    float *sGe = sGeP + 16 * D;    // [D] dG_end (scalar decay: element 0)
    float *sGt = sdT;
    static_assert(C * PD <= 2 * C * PC, "dG tile fits where dT and dA were");
    const int tid = threadIdx.x, u = blockIdx.x;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C;
    const float *wG = a.wG + ucd;
    const bool tied = !BW, grouped = a.Hv > a.Hqk;

    for (int i = tid; i < C * D; i += NT) {
        const int t = i / D, d = i - t * D;
        float qv = 0.f, kv = 0.f, ev = 0.f;
        if (t < x.n) {
            const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + d, iv = (x.rowv + (size_t)t * a.Hv) * D + d;
            qv = ldio<IO>(a.q, iq);
            kv = ldio<IO>(a.k, iq);
            ev = (BW ? ldio<IO>(a.bg, iv) : a.beta[x.rowv + (size_t)t * a.Hv]) * kv;
        }
        if (CHAN) {
            const float G = wG[i], eg = expf(G);
            qv *= eg;
            ev *= eg;
            kv *= expf(-G);
        }
        sP1[t * PD + d] = ev;
        sP2[t * PD + d] = kv;
        sP3[t * PD + d] = qv;
    }
    // One wave per row of dT and dA (lane = column; wave w takes rows w, w + 4, ...).
    float colw = 0.f;
    for (int i = tid; i < C * C; i += NT) {
        const int t = i / C, j = i - t * C;
        float dt = a.wdT[ucc + i], da = a.wdA[ucc + i];
        if (!CHAN) {
            float wv = 0.f;
            if (j <= t) {
                wv = dt * a.wT[ucc + i] + da * a.wA[ucc + i];
                const float f = expf(wG[t] - wG[j]);
                dt *= f;
                da *= f;
            }
            colw += wv;
            wv = wave_sum(wv);
            if (j == 0) sRow[t] = wv;
        }
        sdT[t * PC + j] = dt;
        sdA[t * PC + j] = da;
    }
    if (!CHAN) sColW[(tid >> 6) * C + (tid & 63)] = colw;
    __syncthreads();
    if (!CHAN && tid < C) sCol[tid] = sColW[tid] + sColW[C + tid] + sColW[2 * C + tid] + sColW[3 * C + tid];
    // X_e = dT' P2, X_q = dA' P2, X_k = dT'^T P1 + dA'^T P3; thread = rows m0..m0+3, columns n0..n0+CT-1.
    const int m0 = (tid >> 4) * 4, n0 = (tid & 15) * CT;
    float xe[4][CT], xq[4][CT], xk[4][CT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < CT; ++c) xe[i][c] = xq[i][c] = xk[i][c] = 0.f;
    for (int j = 0; j < C; ++j) {
        float dt4[4], da4[4], tt4[4], ta4[4], p1[CT], p2[CT], p3[CT];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dt4[i] = sdT[(m0 + i) * PC + j];
            da4[i] = sdA[(m0 + i) * PC + j];
            tt4[i] = sdT[j * PC + m0 + i];
            ta4[i] = sdA[j * PC + m0 + i];
        }
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            p1[c] = sP1[j * PD + n0 + c];
            p2[c] = sP2[j * PD + n0 + c];
            p3[c] = sP3[j * PD + n0 + c];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                xe[i][c] = fmaf(dt4[i], p2[c], xe[i][c]);
                xq[i][c] = fmaf(da4[i], p2[c], xq[i][c]);
                xk[i][c] = fmaf(ta4[i], p3[c], fmaf(tt4[i], p1[c], xk[i][c]));
            }
    }
    __syncthreads();  // dT and dA read: their space holds dG from here

    float gend[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) gend[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = m0 + i;
        float dgs = 0.f, dbs = 0.f;
        if (t < x.n) {
            const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D, iv = (x.rowv + (size_t)t * a.Hv) * D;
            const float bt = tied ? a.beta[x.rowv + (size_t)t * a.Hv] : 0.f;
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const int d = n0 + c;
                const float G = CHAN ? wG[t * D + d] : wG[t], Ge = CHAN ? wG[(C - 1) * D + d] : wG[C - 1];
                const float eg = expf(G), egend = expf(Ge - G);
                const float qv = ldio<IO>(a.q, iq + d), kv = ldio<IO>(a.k, iq + d), vv = ldio<IO>(a.v, iv + d);
                const float gb = BW ? ldio<IO>(a.bg, iv + d) : bt, gw = BW ? ldio<IO>(a.wg, iv + d) : bt;
                const size_t o = ucd + (size_t)t * D + d;
                const float dEY = a.wdE[o], dQS = a.wdQ[o], dKE = a.wdK[o], dR = a.wdU[o];
                const float de = (CHAN ? xe[i][c] * eg : xe[i][c]) + dEY * eg;
                const float dq = (CHAN ? xq[i][c] * eg : xq[i][c]) + dQS * eg;
                float dk = (CHAN ? xk[i][c] * expf(-G) : xk[i][c]) + dKE * egend;
                const float ke = kv * egend;
                float dG = gb * kv * eg * dEY + qv * eg * dQS - ke * dKE;
                if (CHAN) dG += sP1[t * PD + d] * xe[i][c] - sP2[t * PD + d] * xk[i][c] + sP3[t * PD + d] * xq[i][c];
                gend[c] += ke * dKE;
                if (CHAN) sGt[t * PD + d] = dG;
                else dgs += dG;
                dk = fmaf(gb, de, dk);
                if (BW) {
                    a.db[iv + d] = de * kv;
                    a.dw[iv + d] = dR * vv;
                } else {
                    dbs += de * kv + dR * vv;
                }
                a.dv[iv + d] = gw * dR;
                if (grouped) {
                    a.wdq[iv + d] = dq;
                    a.wdk[iv + d] = dk;
                } else {
                    a.dq[iq + d] = dq;
                    a.dk[iq + d] = dk;
                }
            }
        }
        else if (CHAN)
#pragma unroll
            for (int c = 0; c < CT; ++c) sGt[t * PD + n0 + c] = 0.f;  // padded token
        sTokG[t * 16 + (tid & 15)] = dgs;
        sTokB[t * 16 + (tid & 15)] = dbs;
    }
#pragma unroll
    for (int c = 0; c < CT; ++c) sGeP[(tid >> 4) * D + n0 + c] = gend[c];
    __syncthreads();
    // dG_end = sum over the chunk of Kend . dKend, plus Gamma . dGamma.
    if (tid < D) {
        float g = a.wGam[(size_t)u * D + tid] * a.wdGam[(size_t)u * D + tid];
        for (int r = 0; r < 16; ++r) g += sGeP[r * D + tid];
        sGe[tid] = g;
    }
    if (tid < C) {
        float g = 0.f, bsum = 0.f;
        for (int r = 0; r < 16; ++r) {
            g += sTokG[tid * 16 + r];
            bsum += sTokB[tid * 16 + r];
        }
        sTokG[tid * 16] = g;
        sTokB[tid * 16] = bsum;
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
                    acc += sGt[t * PD + tid];
                    if (t < x.n) a.dg[(x.rowv + (size_t)t * a.Hv) * D + tid] = acc;
                }
            }
        } else if (tid < 64) {
            // Suffix sums over the chunk's tokens; lane = token.
            float v = sTokG[tid * 16] + sRow[tid] - sCol[tid];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_down(v, off);
                if (tid + off < 64) v += y;
            }
            if (tid < x.n) a.dg[x.rowv + (size_t)tid * a.Hv] = v + sGe[0];
        }
    }
    if (tied && tid < x.n) a.dbeta[x.rowv + (size_t)tid * a.Hv] = sTokB[tid * 16];
}

// dq, dk of a QK head: the sum of its V heads' parts.
template <int D>
__global__ __launch_bounds__(NT) void cb_group_sum(ChunkBwdArgs a) {
    const int grp = a.Hv / a.Hqk;
    const size_t n = (size_t)a.B * a.T * a.Hqk * D;
    for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n; i += (size_t)gridDim.x * NT) {
        const size_t d = i % D, r = i / D, hq = r % a.Hqk, bt = r / a.Hqk;
        const size_t base = (bt * a.Hv + hq * grp) * D + d;
        float sq = 0.f, sk = 0.f;
        for (int j = 0; j < grp; ++j) {
            sq += a.wdq[base + (size_t)j * D];
            sk += a.wdk[base + (size_t)j * D];
        }
        a.dq[i] = sq;
        a.dk[i] = sk;
    }
}

template <typename IO, int D, bool CHAN, bool BW>
hipError_t run(const ChunkBwdArgs &a, hipStream_t s) {
    static const hipError_t attr = [] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&cb_prep<IO, D, CHAN, BW>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)prep_smem<D>());
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&cb_grad_s<IO, D>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)grad_s_smem<D>());
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&cb_grad_out<IO, D, CHAN, BW>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)grad_out_smem<D>());
        return e;
    }();
    if (attr != hipSuccess) return attr;
    const unsigned units = (unsigned)((size_t)a.B * a.Hv * a.NC), items = (unsigned)((size_t)a.B * a.Hv * (D / BV));
    hipLaunchKernelGGL((cb_prep<IO, D, CHAN, BW>), dim3(units), dim3(NT), prep_smem<D>(), s, a);
    hipLaunchKernelGGL((cb_fsweep<D>), dim3(items), dim3(NT), 0, s, a);
    hipLaunchKernelGGL((cb_bsweep<IO, D>), dim3(items), dim3(NT), 0, s, a);
    hipLaunchKernelGGL((cb_grad_s<IO, D>), dim3(units), dim3(NT), grad_s_smem<D>(), s, a);
    hipLaunchKernelGGL((cb_grad_out<IO, D, CHAN, BW>), dim3(units), dim3(NT), grad_out_smem<D>(), s, a);
    if (a.Hv > a.Hqk) {
        const size_t n = (size_t)a.B * a.T * a.Hqk * D;
        const size_t blocks = (n + NT - 1) / NT;
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
