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
// Shared-memory tiles keep 16-byte aligned rows (stride a multiple of 4
// floats); global arrays are staged through registers with 16-byte (8-byte
// for bf16) loads. All arithmetic is fp32: the dense products of the sweeps,
// of cb_grad_s and of cb_grad_out on the matrix cores
// (v_mfma_f32_16x16x4_f32), the rest on the vector units.
//
// Four launches (five with grouped heads):
//  1. cb_prep (per chunk unit): G, the factors above, T and A, and the
//     triangular solve (I + T)[Y | U_z] = [E~ | Z] by forward substitution.
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
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b, float acc) {
    return fmaf(a[3], b[3], fmaf(a[2], b[2], fmaf(a[1], b[1], fmaf(a[0], b[0], acc))));
}
template <typename IO>
__device__ __forceinline__ f32x4 ld4io(const void *p, size_t i) {  // 4 consecutive io elements, widened
    return Raw4<IO>::widen(Raw4<IO>::load(static_cast<const IO *>(p) + i));
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
__device__ __forceinline__ void rc(int l, int &e, int &t, int &d) {
    e = 4 * (l * NT + (int)threadIdx.x);
    t = e / D;
    d = e - t * D;
}

// Workgroup barrier ordering shared-memory accesses only: it does not wait
// for global loads in flight (the sweeps' prefetch of the next chunk) or
// for global stores, which nothing in the same launch reads back.
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

// (I + T) x = r for one column x (in registers, r on entry), T strictly
// lower triangular. Right-looking: once x_m is final it is taken out of every
// later row at once, so the dependent chain is one multiply-add per row and
// the rest is independent work. sTt = T^T, row-major with row stride C
// (row m = column m of T, 16-byte aligned rows).
__device__ __forceinline__ void solve_lower(float (&x)[C], const float *sTt) {
#pragma unroll
    for (int m = 0; m < C - 1; ++m) {
#pragma unroll
        for (int i4 = (m + 1) & ~3; i4 < C; i4 += 4) {
            const f32x4 t = lds4(sTt + m * C + i4);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (i4 + r > m) x[i4 + r] = fmaf(-t[r], x[m], x[i4 + r]);
        }
    }
}
// (I + T)^T x = r, rows from the last: x_i = r_i - sum_{m > i} T_mi x_m,
// right-looking as above. sT = T, row-major with row stride C.
__device__ __forceinline__ void solve_upper(float (&x)[C], const float *sT) {
#pragma unroll
    for (int m = C - 1; m > 0; --m) {
#pragma unroll
        for (int i4 = 0; i4 < m; i4 += 4) {
            const f32x4 t = lds4(sT + m * C + i4);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (i4 + r < m) x[i4 + r] = fmaf(-t[r], x[m], x[i4 + r]);
        }
    }
}

template <int D>
constexpr size_t prep_smem() {
    constexpr size_t LD = D + 4, R0 = C * LD > C * C ? C * LD : C * C;
    return (R0 + 3 * C * LD + C) * 4;
}
template <int D>
constexpr size_t fsweep_smem() {
    return ((size_t)D * LB + (size_t)C * LB + (size_t)D * LT + (size_t)D * LC + D) * 4;
}
template <int D>
constexpr size_t bsweep_smem() {
    return ((size_t)D * LB + 2 * (size_t)C * LB + (size_t)C * LT + 3 * (size_t)D * LC + D) * 4;
}
template <int D>
constexpr size_t grad_s_smem() {
    constexpr size_t LD = D + 4, R0 = C * C > 32 * LD ? C * C : 32 * LD;
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
    constexpr int LD = Cfg<D>::LD, NL = Cfg<D>::NL, R0 = C * LD > C * C ? C * LD : C * C;
    extern __shared__ __align__(16) float smem[];
    float *sQ = smem;           // q (Q~ with a per-channel decay); then T^T, row stride C
    float *sK = sQ + R0;        // k (K~)
    float *sE = sK + C * LD;    // e, then E~, then Y
    float *sZ = sE + C * LD;    // per-channel decay: g, then G; then z, then U_z
    float *sGs = sZ + C * LD;   // scalar decay: G per token
    const int tid = threadIdx.x, u = blockIdx.x;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D;
    f32x4 rz[NL];  // z = beta v (or w v), loaded with the other inputs and staged after T and A
    {
        f32x4 rq[NL], rk[NL], re[NL], rg[CHAN ? NL : 1];
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            rq[l] = rk[l] = re[l] = rz[l] = zero4();
            if (CHAN) rg[l] = zero4();
            if (t < x.n) {
                const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + d, iv = (x.rowv + (size_t)t * a.Hv) * D + d;
                rq[l] = ld4io<IO>(a.q, iq);
                rk[l] = ld4io<IO>(a.k, iq);
                re[l] = BW ? ld4io<IO>(a.bg, iv) : splat(a.beta[x.rowv + (size_t)t * a.Hv]);
                if (CHAN) rg[l] = lds4(a.g + iv);
                rz[l] = (BW ? ld4io<IO>(a.wg, iv) : splat(a.beta[x.rowv + (size_t)t * a.Hv])) * ld4io<IO>(a.v, iv);
            }
        }
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            sts4(sQ + t * LD + d, rq[l]);
            sts4(sK + t * LD + d, rk[l]);
            sts4(sE + t * LD + d, re[l] * rk[l]);
            if (CHAN) sts4(sZ + t * LD + d, rg[l]);
        }
    }
    if (!CHAN && tid < C) sGs[tid] = a.g && tid < x.n ? a.g[x.rowv + (size_t)tid * a.Hv] : 0.f;
    __syncthreads();
    if (CHAN) {
        if (tid < D) {  // per channel: the column into registers, summed, written back
            float gc[C];
#pragma unroll
            for (int t = 0; t < C; ++t) gc[t] = sZ[t * LD + tid];
#pragma unroll
            for (int t = 1; t < C; ++t) gc[t] += gc[t - 1];
#pragma unroll
            for (int t = 0; t < C; ++t) sZ[t * LD + tid] = gc[t];
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
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        int e, t, d;
        rc<D>(l, e, t, d);
        const f32x4 G = CHAN ? lds4(sZ + t * LD + d) : splat(sGs[t]);
        const f32x4 Ge = CHAN ? lds4(sZ + (C - 1) * LD + d) : splat(sGs[C - 1]);
        const f32x4 eg = exp4(G), qv = lds4(sQ + t * LD + d), kv = lds4(sK + t * LD + d);
        if (CHAN) {
            sts4(wG + e, G);
            sts4(sQ + t * LD + d, qv * eg);
            sts4(sK + t * LD + d, kv * exp4(-G));
            sts4(sE + t * LD + d, lds4(sE + t * LD + d) * eg);
        }
    }
    if (!CHAN && tid < C) wG[tid] = sGs[tid];
    if (tid < D) a.wGam[(size_t)u * D + tid] = expf(CHAN ? sZ[(C - 1) * LD + tid] : sGs[C - 1]);
    __syncthreads();
    // Q~^T and Kend^T (row = channel), which the sweeps over chunks read.
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        int e, dd, t;
        rc<C>(l, e, dd, t);
        f32x4 qv, kv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            qv[r] = sQ[(t + r) * LD + dd];
            kv[r] = sK[(t + r) * LD + dd];
        }
        if (CHAN) {
            kv *= expf(sZ[(C - 1) * LD + dd]);  // Kend = K~ exp(G_end)
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                qv[r] *= expf(sGs[t + r]);
                kv[r] *= expf(sGs[C - 1] - sGs[t + r]);
            }
        }
        sts4(a.wQt + ucd + e, qv);
        sts4(a.wKet + ucd + e, kv);
    }

    // T and A: thread = 2 x 4 block of rows r0.., columns c0..
    {
        const int r0 = (tid >> 4) * 2, c0 = (tid & 15) * 4;
        float aT[2][4], aA[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) aT[i][j] = aA[i][j] = 0.f;
        if (c0 <= r0 + 1) {
#pragma unroll 2
            for (int d = 0; d < D; d += 4) {
                f32x4 e4[2], q4[2], k4[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    e4[i] = lds4(sE + (r0 + i) * LD + d);
                    q4[i] = lds4(sQ + (r0 + i) * LD + d);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) k4[j] = lds4(sK + (c0 + j) * LD + d);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        aT[i][j] = dot4(e4[i], k4[j], aT[i][j]);
                        aA[i][j] = dot4(q4[i], k4[j], aA[i][j]);
                    }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = r0 + i;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int jj = c0 + j;
                const float f = !CHAN && jj <= t ? expf(sGs[t] - sGs[jj]) : 1.f;
                aT[i][j] = jj < t ? aT[i][j] * f : 0.f;
                aA[i][j] = jj <= t ? aA[i][j] * f : 0.f;
            }
            const size_t o = (size_t)u * C * C + (size_t)t * C + c0;
            sts4(a.wT + o, f32x4{aT[i][0], aT[i][1], aT[i][2], aT[i][3]});
            sts4(a.wA + o, f32x4{aA[i][0], aA[i][1], aA[i][2], aA[i][3]});
        }
        __syncthreads();  // q, k and e tiles read: T^T goes where q was
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) sQ[(c0 + j) * C + r0 + i] = aT[i][j];
    }
    // Right-hand sides: E~ (scalar decay: the raw e scaled by exp(G_t)) and z.
    {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            sts4(sZ + t * LD + d, rz[l]);
            if (!CHAN) sts4(sE + t * LD + d, lds4(sE + t * LD + d) * expf(sGs[t]));
        }
    }
    __syncthreads();
    // (I + T) X = [E~ | Z], one column per thread.
    if (tid < 2 * D) {
        float *X = tid < D ? sE + tid : sZ + (tid - D);
        float xc[C];
#pragma unroll
        for (int i = 0; i < C; ++i) xc[i] = X[i * LD];
        solve_lower(xc, sQ);
#pragma unroll
        for (int i = 0; i < C; ++i) X[i * LD] = xc[i];
    }
    __syncthreads();
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        int e, t, d;
        rc<D>(l, e, t, d);
        sts4(a.wUz + ucd + e, lds4(sZ + t * LD + d));
    }
#pragma unroll
    for (int l = 0; l < NL; ++l) {  // Y^T
        int e, dd, t;
        rc<C>(l, e, dd, t);
        sts4(a.wYt + ucd + e, f32x4{sE[t * LD + dd], sE[(t + 1) * LD + dd], sE[(t + 2) * LD + dd], sE[(t + 3) * LD + dd]});
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

// 2a. Forward over chunks: the state entering each chunk, and U = U_z - Y S.
//    Wave w: U tile (rows 16 (w / 2), columns 16 (w % 2)); state tiles w and
//    w + 8 of the (D / 16) x 2 tiles of the state.
template <int D>
__device__ __forceinline__ void fsweep(const ChunkBwdArgs &a, float *smem, int item) {
    using K = SwCfg<D>;
    constexpr int NTL = K::NTL, NL = K::NL, LD = D + 4, NST = D / 16 * 2;
    float *sS = smem, *sU = sS + D * LB, *sYt = sU + C * LB, *sKt = sYt + D * LT;  // Y^T [D][LT], Kend^T [D][LC]
    float *sGam = sKt + D * LC;
    const int tid = threadIdx.x, tile = item % NTL, bh = item / NTL, col0 = tile * BV;
    const int w = tid >> 6, l = tid & 63, rt = w >> 1, ct = w & 1;
    const size_t sb = (size_t)bh * D * D;
    for (int i = tid; i < D * BV / 4; i += NS) {
        const int d = 4 * i / BV, j = 4 * i - d * BV;
        sts4(sS + d * LB + j, a.S0 ? lds4(a.S0 + sb + (size_t)d * D + col0 + j) : zero4());
    }
    f32x4 pY[NL], pK[NL];
    float pZ[4], pg;
    const auto fetch = [&](int c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            const int e = 4 * (l2 * NS + tid);
            pY[l2] = lds4(a.wYt + ucd + e);   // [D][C]
            pK[l2] = lds4(a.wKet + ucd + e);  // [D][C]
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) pZ[r] = a.wUz[ucd + (size_t)(rt * 16 + 4 * (l >> 4) + r) * D + col0 + ct * 16 + (l & 15)];
        pg = tid < D ? a.wGam[u * D + tid] : 0.f;
    };
    fetch(0);
    for (int c = 0; c < a.NC; ++c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
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
        if (c + 1 < a.NC) fetch(c + 1);
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            sts4(a.wS + u * D * D + (size_t)d * D + col0 + j, lds4(sS + d * LB + j));
        }
        lds_barrier();
        {  // U = U_z - Y S
            const f32x4 p = mfma_kloop_at<D>(zero4(), sYt + rt * 16, LT, sS + ct * 16, LB);
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
        // S = Gamma . S + Kend^T U
        f32x4 sn[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int st = w + 8 * q, dt = st >> 1, sc = st & 1;
            if (st < NST) {
                const f32x4 p = mfma_kloop<C>(zero4(), sKt + dt * 16 * LC, LC, sU + sc * 16, LB);
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
        for (int q = 0; q < 2; ++q) {
            const int st = w + 8 * q, dt = st >> 1, sc = st & 1;
            if (st < NST)
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[(dt * 16 + 4 * (l >> 4) + r) * LB + sc * 16 + (l & 15)] = sn[q][r];
        }
    }
}

// 2b. Backward over chunks for the same work items: X = dL/d(state leaving
//    the chunk), dU, and X for the chunk before. Tiles per wave as above.
template <typename IO, int D>
__device__ __forceinline__ void bsweep(const ChunkBwdArgs &a, float *smem, int item) {
    using K = SwCfg<D>;
    constexpr int NTL = K::NTL, NL = K::NL, LD = D + 4, NST = D / 16 * 2;
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
    f32x4 pY[NL], pK[NL], pQ[NL], pA[NA], pO[NO];
    float pg;
    const auto fetch = [&](int c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
        const int t0 = c * C, n = min(C, a.T - t0);
#pragma unroll
        for (int l2 = 0; l2 < NL; ++l2) {
            const int e = 4 * (l2 * NS + tid);
            pY[l2] = lds4(a.wYt + ucd + e);   // [D][C]
            pK[l2] = lds4(a.wKet + ucd + e);  // [D][C]
            pQ[l2] = lds4(a.wQt + ucd + e);   // [D][C]
        }
#pragma unroll
        for (int l2 = 0; l2 < NA; ++l2) pA[l2] = lds4(a.wA + u * C * C + 4 * (l2 * NS + tid));
#pragma unroll
        for (int l2 = 0; l2 < NO; ++l2) {
            int e, t, j;
            rcs<BV>(l2, e, t, j);
            pO[l2] = t < n ? ld4io<IO>(a.dO, (((size_t)b * a.T + t0 + t) * a.Hv + h) * D + col0 + j) : zero4();
        }
        pg = tid < D ? a.wGam[u * D + tid] : 0.f;
    };
    fetch(a.NC - 1);
    for (int c = a.NC - 1; c >= 0; --c) {
        const size_t u = (size_t)bh * a.NC + c, ucd = u * C * D;
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
        if (c > 0) fetch(c - 1);
        for (int i = tid; i < D * BV / 4; i += NS) {
            const int d = 4 * i / BV, j = 4 * i - d * BV;
            sts4(a.wdS + u * D * D + (size_t)d * D + col0 + j, lds4(sX + d * LB + j));
        }
        lds_barrier();
        {  // dU = s A^T dO + Kend X
            const f32x4 p = mfma_kloop_at<C>(zero4(), sA + rt * 16, LT, sO + ct * 16, LB);
            const f32x4 k = mfma_kloop_at<D>(zero4(), sKt + rt * 16, LC, sX + ct * 16, LB);
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
        // X = Gamma . X + s Q~^T dO - Y^T dU
        f32x4 xn[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int st = w + 8 * q, dt = st >> 1, sc = st & 1;
            if (st < NST) {
                const f32x4 pq = mfma_kloop<C>(zero4(), sQt + dt * 16 * LC, LC, sO + sc * 16, LB);
                const f32x4 py = mfma_kloop<C>(zero4(), sYt + dt * 16 * LC, LC, sdU + sc * 16, LB);
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
        for (int q = 0; q < 2; ++q) {
            const int st = w + 8 * q, dt = st >> 1, sc = st & 1;
            if (st < NST)
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
template <typename IO, int D>
__global__ __launch_bounds__(NS) void cb_sweeps(ChunkBwdArgs a, int items, int P) {
    extern __shared__ __align__(16) float smem[];
    const int x = (int)blockIdx.x, back = x < P, xl = back ? x : x - P;
    const int wi = (xl & 7) * (P >> 3) + (xl >> 3);
    if (wi >= items) return;
    if (back) bsweep<IO, D>(a, smem, wi);
    else fsweep<D>(a, smem, wi);
}

// ---------------------------------------------------------------------------
// 3. Per unit: dR = L^T dU (solve (I + T)^T dR = dU), dT, dA, and the
//    products with S and dS_next.
template <typename IO, int D>
__global__ __launch_bounds__(NT) void cb_grad_s(ChunkBwdArgs a) {
    constexpr int LD = Cfg<D>::LD, NL = Cfg<D>::NL, R0 = C * C > 32 * LD ? C * C : 32 * LD;
    constexpr int NG = 32 * D / 4, NB = (NG + NT - 1) / NT, NTT = C * C / (4 * NT);  // 4-element groups: S block, T
    extern __shared__ __align__(16) float smem[];
    float *sT = smem;  // T, row stride C; later 32 rows of S
    float *sX = sT + R0, *sU = sX + C * LD, *sO = sU + C * LD, *sB = sO + C * LD;
    const int tid = threadIdx.x, u = blockIdx.x;
    const Unit x = decode(a, u);
    const size_t ucd = (size_t)u * C * D, ucc = (size_t)u * C * C, udd = (size_t)u * D * D;
    {
        f32x4 rX[NL], rU[NL], rO[NL], rT[NTT];
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            rX[l] = lds4(a.wdU + ucd + e);
            rU[l] = lds4(a.wU + ucd + e);
            rO[l] = t < x.n ? ld4io<IO>(a.dO, (x.rowv + (size_t)t * a.Hv) * D + d) : zero4();
        }
#pragma unroll
        for (int l = 0; l < NTT; ++l) rT[l] = lds4(a.wT + ucc + 4 * (l * NT + tid));
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int e, t, d;
            rc<D>(l, e, t, d);
            sts4(sX + t * LD + d, rX[l]);
            sts4(sU + t * LD + d, rU[l]);
            sts4(sO + t * LD + d, rO[l]);
        }
#pragma unroll
        for (int l = 0; l < NTT; ++l) sts4(sT + 4 * (l * NT + tid), rT[l]);  // T, row stride C
    }
    // The first block of S and dS_next rows is fetched into registers now, so
    // that it arrives during the solve; the barriers up to its use order the
    // shared tiles only and do not wait for it.
    f32x4 rb[NB], rs[NB];
    const auto fetch = [&](int blk) {
#pragma unroll
        for (int l = 0; l < NB; ++l) {
            const int g = l * NT + tid;
            if (g < NG) {
                rs[l] = lds4(a.wS + udd + (size_t)blk * 32 * D + 4 * g);
                rb[l] = lds4(a.wdS + udd + (size_t)blk * 32 * D + 4 * g);
            }
        }
    };
    fetch(0);
    lds_barrier();
    if (tid < D) {  // one column of dU per thread
        float *X = sX + tid;
        float xc[C];
#pragma unroll
        for (int i = 0; i < C; ++i) xc[i] = X[i * LD];
        solve_upper(xc, sT);
#pragma unroll
        for (int i = 0; i < C; ++i) X[i * LD] = xc[i];
    }
    lds_barrier();
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        int e, t, d;
        rc<D>(l, e, t, d);
        sts4(a.wdU + ucd + e, lds4(sX + t * LD + d));  // dR replaces dU
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
        if (blk + 1 < D / 32) fetch(blk + 1);
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
    static_assert(C * LD <= 2 * C * LC && NRG * D <= 2048 && NCG <= 32 && NT / 16 == 32, "shared-memory layout");
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
            if (CHAN) {
                const f32x4 G = lds4(wG + e), eg = exp4(G);
                qv *= eg;
                ev *= eg;
                kv *= exp4(-G);
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
    __syncthreads();
    if (!CHAN && tid < C) {
        float cs = 0.f;
        for (int r = 0; r < 32; ++r) cs += sColP[r * C + tid];
        sCol[tid] = cs;
    }
    // X_e = dT' P2, X_q = dA' P2, X_k = dT'^T P1 + dA'^T P3 on the matrix
    // cores: 16 x 16 output tiles, wave w taking tiles w, w + 8, ...; then
    // through shared memory (where P1..P3 were) to the thread layout below.
    {
        constexpr int NTC = D / 16, NTW = C / 16 * NTC / 8;
        const int w = tid >> 6, l = tid & 63;
        f32x4 te[NTW], tq[NTW], tk[NTW];
#pragma unroll
        for (int q = 0; q < NTW; ++q) {
            const int tile = w + 8 * q, rt = tile / NTC, ct = tile - rt * NTC;
            te[q] = mfma_kloop<C>(zero4(), sdT + rt * 16 * LC, LC, sP2 + ct * 16, LD);
            tq[q] = mfma_kloop<C>(zero4(), sdA + rt * 16 * LC, LC, sP2 + ct * 16, LD);
            tk[q] = mfma_kloop_at<C>(zero4(), sdT + rt * 16, LC, sP1 + ct * 16, LD);
            tk[q] = mfma_kloop_at<C>(tk[q], sdA + rt * 16, LC, sP3 + ct * 16, LD);
        }
        __syncthreads();  // dT, dA and the P tiles read
#pragma unroll
        for (int q = 0; q < NTW; ++q) {
            const int tile = w + 8 * q, rt = tile / NTC, ct = tile - rt * NTC;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (rt * 16 + 4 * (l >> 4) + r) * LD + ct * 16 + (l & 15);
                sP1[o] = te[q][r];
                sP2[o] = tq[q][r];
                sP3[o] = tk[q][r];
            }
        }
    }
    __syncthreads();  // X tiles written; dT's space holds dG from here
    const int cg = tid % NCG, rg = tid / NCG, m0 = rg * RT, n0 = 4 * cg;

    f32x4 gend = zero4();
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = m0 + i;
        float dgs = 0.f, dbs = 0.f;
        if (t < x.n) {
            const size_t iq = (x.rowq + (size_t)t * a.Hqk) * D + n0, iv = (x.rowv + (size_t)t * a.Hv) * D + n0;
            const size_t o = ucd + (size_t)t * D + n0;
            const float bt = tied ? a.beta[x.rowv + (size_t)t * a.Hv] : 0.f;
            const f32x4 G = CHAN ? lds4(wG + t * D + n0) : splat(wG[t]);
            const f32x4 Ge = CHAN ? lds4(wG + (C - 1) * D + n0) : splat(wG[C - 1]);
            const f32x4 eg = exp4(G), egend = exp4(Ge - G);
            const f32x4 qv = ld4io<IO>(a.q, iq), kv = ld4io<IO>(a.k, iq), vv = ld4io<IO>(a.v, iv);
            const f32x4 gb = BW ? ld4io<IO>(a.bg, iv) : splat(bt), gw = BW ? ld4io<IO>(a.wg, iv) : splat(bt);
            const f32x4 dEY = lds4(a.wdE + o), dQS = lds4(a.wdQ + o), dKE = lds4(a.wdK + o), dR = lds4(a.wdU + o);
            const f32x4 xe = lds4(sP1 + t * LD + n0), xq = lds4(sP2 + t * LD + n0), xk = lds4(sP3 + t * LD + n0);
            const f32x4 emg = CHAN ? exp4(-G) : splat(1.f);
            const f32x4 de = (CHAN ? xe * eg : xe) + dEY * eg;
            const f32x4 dq = (CHAN ? xq * eg : xq) + dQS * eg;
            const f32x4 ke = kv * egend;
            f32x4 dk = (CHAN ? xk * emg : xk) + dKE * egend;
            f32x4 dG = gb * kv * eg * dEY + qv * eg * dQS - ke * dKE;
            if (CHAN) dG += gb * kv * eg * xe - kv * emg * xk + qv * eg * xq;  // E~, K~, Q~ times their parts
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
    constexpr size_t sweep_smem = bsweep_smem<D>() > fsweep_smem<D>() ? bsweep_smem<D>() : fsweep_smem<D>();
    static_assert(sweep_smem <= 160 * 1024, "the sweeps' tiles exceed a workgroup's local data share");
    static const hipError_t attr = [] {
        const void *fn[4] = {reinterpret_cast<const void *>(&cb_prep<IO, D, CHAN, BW>),
                             reinterpret_cast<const void *>(&cb_sweeps<IO, D>),
                             reinterpret_cast<const void *>(&cb_grad_s<IO, D>),
                             reinterpret_cast<const void *>(&cb_grad_out<IO, D, CHAN, BW>)};
        const size_t bytes[4] = {prep_smem<D>(), sweep_smem, grad_s_smem<D>(), grad_out_smem<D>()};
        for (int i = 0; i < 4; ++i) {
            const hipError_t e = hipFuncSetAttribute(fn[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes[i]);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    const unsigned units = (unsigned)((size_t)a.B * a.Hv * a.NC), items = (unsigned)((size_t)a.B * a.Hv * (D / BV));
    hipLaunchKernelGGL((cb_prep<IO, D, CHAN, BW>), dim3(units), dim3(NT), prep_smem<D>(), s, a);
    const unsigned P = (items + 7) / 8 * 8;
    hipLaunchKernelGGL((cb_sweeps<IO, D>), dim3(2 * P), dim3(NS), sweep_smem, s, a, (int)items, (int)P);
    hipLaunchKernelGGL((cb_grad_s<IO, D>), dim3(units), dim3(NT), grad_s_smem<D>(), s, a);
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
