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

template <typename IO, int D>
struct PrepLayout {
    static constexpr int NT = 256;
    static constexpr int PD = D + 8;  // row stride of [C x D] row-major tiles
    static constexpr int PT = C + 8;  // row stride of [D x C] transposed tiles
    static constexpr int PF = C + 1;  // row stride of fp32 [C x C] matrices
    static constexpr size_t SLOT = a16(cmax((size_t)C * PD, (size_t)D * PT) * sizeof(IO));
    static constexpr size_t F32 = a16(cmax(cmax((size_t)2 * C * PF * 4, (size_t)C * D * 4), (size_t)D * PT * sizeof(IO)));
    static constexpr size_t LA = a16(cmax((size_t)2 * C * PT * sizeof(IO), (size_t)D * PT * sizeof(IO)));
    static constexpr size_t OFF_F32 = 5 * SLOT;
    static constexpr size_t OFF_LA = OFF_F32 + F32;
    static constexpr size_t BYTES = OFF_LA + LA;
};

// 8 consecutive elements widened to float.
__device__ __forceinline__ void load8(const bf16_t *p, float *x) {
    u16x8 u = *reinterpret_cast<const u16x8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = bf2f(u[j]);
}
__device__ __forceinline__ void load8(const float *p, float *x) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
}
__device__ __forceinline__ void store8(bf16_t *p, const float *x) {
    u16x8 u;
#pragma unroll
    for (int j = 0; j < 8; ++j) u[j] = f2bf(x[j]);
    *reinterpret_cast<u16x8 *>(p) = u;
}
__device__ __forceinline__ void store8(float *p, const float *x) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

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

template <typename IO, int D>
__global__ __launch_bounds__(256) void chunk_prep(ChunkArgs a) {
    using E = Elem<IO>;
    using M = Mma<IO>;
    using Lay = PrepLayout<IO, D>;
    constexpr int NT = Lay::NT, PD = Lay::PD, PT = Lay::PT, PF = Lay::PF;
    constexpr int KS = M::KS;
    constexpr int CT = D / 16;  // 16-wide column tiles over D

    extern __shared__ __align__(16) unsigned char smem[];
    IO *sE = reinterpret_cast<IO *>(smem + 0 * Lay::SLOT);    // E~ [C][PD]; later -Y^T [D][PT]
    IO *sK = reinterpret_cast<IO *>(smem + 1 * Lay::SLOT);    // K~ [C][PD]; later U_z^T [D][PT]
    IO *sQ = reinterpret_cast<IO *>(smem + 2 * Lay::SLOT);    // Q~ [C][PD]
    IO *sET = reinterpret_cast<IO *>(smem + 3 * Lay::SLOT);   // E~^T [D][PT]; later Y staging [C][PD]
    IO *sZT = reinterpret_cast<IO *>(smem + 4 * Lay::SLOT);   // Z^T [D][PT]; later W_q staging [C][PD]
    float *sG = reinterpret_cast<float *>(smem + Lay::OFF_F32);  // G [C][D] or [C]
    float *sTf = sG;                                             // T [C][PF] (after sG is dead)
    float *sLf = sG + C * PF;                                    // L [C][PF]
    IO *sOzs = reinterpret_cast<IO *>(smem + Lay::OFF_F32);      // O_z^T staging [D][PT] (after L is dead)
    IO *sL = reinterpret_cast<IO *>(smem + Lay::OFF_LA);         // L in io dtype [C][PT]
    IO *sA = sL + C * PT;                                        // A [C][PT]
    IO *sKTs = sL;                                               // Kend^T staging [D][PT] (before L, A)
    IO *sYT = sE;
    IO *sUzT = sK;
    IO *sYs = sET;
    IO *sWs = sZT;

    const int NC = a.NC;
    const int u = blockIdx.x;
    const int c = u % NC;
    const int bh = u / NC;
    const int b = bh / a.Hv, h = bh - (bh / a.Hv) * a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int t0 = c * C;
    const int n = min(C, a.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;

    IO *ws = static_cast<IO *>(a.ws_io) + (size_t)u * chunk_ws_io_elems(D);
    IO *wY = ws, *wWq = ws + C * D, *wKT = ws + 2 * C * D, *wUzT = ws + 3 * C * D, *wOzT = ws + 4 * C * D;

    // ---- Cumulative log decay inside the chunk (padded tokens add 0). ----
    if (a.decay == DECAY_CHANNEL) {
        if (tid < D) {
            float acc = 0.f;
            const float *gp = a.g + (((size_t)b * a.T + t0) * a.Hv + h) * D + tid;
#pragma unroll 8
            for (int i = 0; i < C; ++i) {
                acc += i < n ? gp[(size_t)i * a.Hv * D] : 0.f;
                sG[i * D + tid] = acc;
            }
        }
    } else if (a.decay == DECAY_SCALAR) {
        if (w == 0) {
            float x = l < n ? a.g[((size_t)b * a.T + t0 + l) * a.Hv + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            sG[l] = x;
        }
    }
    __syncthreads();

    // ---- Decay absorbed into the factors (fp32 math, stored in the io dtype). ----
    {
        constexpr int G8 = D / 8;
        for (int item = tid; item < C * G8; item += NT) {
            const int i = item / G8, c8 = (item - (item / G8) * G8) * 8;
            float qv[8], kv[8], vv[8], ev[8], zv[8];
            if (i < n) {
                const size_t tok = (size_t)b * a.T + t0 + i;
                load8(static_cast<const IO *>(a.q) + (tok * a.Hqk + hq) * D + c8, qv);
                load8(static_cast<const IO *>(a.k) + (tok * a.Hqk + hq) * D + c8, kv);
                load8(static_cast<const IO *>(a.v) + (tok * a.Hv + h) * D + c8, vv);
                if (a.beta) {
                    const float bt = a.beta[tok * a.Hv + h];
#pragma unroll
                    for (int j = 0; j < 8; ++j) { ev[j] = bt * kv[j]; zv[j] = bt * vv[j]; }
                } else {
                    float bg[8], wg[8];
                    load8(static_cast<const IO *>(a.bg) + (tok * a.Hv + h) * D + c8, bg);
                    load8(static_cast<const IO *>(a.wg) + (tok * a.Hv + h) * D + c8, wg);
#pragma unroll
                    for (int j = 0; j < 8; ++j) { ev[j] = bg[j] * kv[j]; zv[j] = wg[j] * vv[j]; }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) qv[j] = kv[j] = vv[j] = ev[j] = zv[j] = 0.f;
            }
            float xe[8], xk[8], xq[8], xend[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float G = 0.f, Gend = 0.f;
                if (a.decay == DECAY_CHANNEL) { G = sG[i * D + c8 + j]; Gend = sG[(C - 1) * D + c8 + j]; }
                else if (a.decay == DECAY_SCALAR) { G = sG[i]; Gend = sG[C - 1]; }
                const float eg = expf(G);
                xe[j] = ev[j] * eg;
                xq[j] = qv[j] * eg;
                xk[j] = kv[j] * expf(-G);
                xend[j] = kv[j] * expf(Gend - G);
            }
            store8(sE + i * PD + c8, xe);
            store8(sK + i * PD + c8, xk);
            store8(sQ + i * PD + c8, xq);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sET[(c8 + j) * PT + i] = E::to(xe[j]);
                sZT[(c8 + j) * PT + i] = E::to(zv[j]);
                sKTs[(c8 + j) * PT + i] = E::to(xend[j]);
            }
        }
        if (tid < D) {
            float Gend = 0.f;
            if (a.decay == DECAY_CHANNEL) Gend = sG[(C - 1) * D + tid];
            else if (a.decay == DECAY_SCALAR) Gend = sG[C - 1];
            a.ws_gamma[(size_t)u * D + tid] = expf(Gend);
        }
    }
    __syncthreads();
    copy_block(wKT, C, sKTs, PT, D, C, tid, NT);

    // ---- Gram products on the matrix cores: T = E~ K~^T, A = Q~ K~^T (lower tiles). ----
    f32x4 gacc[5];
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        const int p = w + 4 * s;
        const int kind = p / 10;
        int ti, tj;
        lower_tile(p - kind * 10, ti, tj);
        const IO *X = kind == 0 ? sE : sQ;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < D / KS; ++ks)
            acc = M::step(acc, X + ti * 16 * PD + ks * KS, PD, sK + tj * 16 * PD + ks * KS, PD);
        gacc[s] = acc;
    }
    __syncthreads();  // Kend^T staging copied out; sG dead
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        const int p = w + 4 * s;
        const int kind = p / 10;
        int ti, tj;
        lower_tile(p - kind * 10, ti, tj);
        const int col = tj * 16 + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = ti * 16 + 4 * lq + r;
            if (kind == 0) sTf[row * PF + col] = col < row ? gacc[s][r] : 0.f;
            else sA[row * PT + col] = E::to(col <= row ? gacc[s][r] : 0.f);
        }
    }
    // Upper tiles of A are zero (products below run K over whole 32-token steps).
    for (int i = tid; i < C * C; i += NT) {
        const int row = i / C, col = i - (i / C) * C;
        if ((col >> 4) > (row >> 4)) sA[row * PT + col] = E::to(0.f);
    }
    __syncthreads();

    // ---- L = (I + T)^-1 in fp32. ----
    // Diagonal 16 x 16 blocks by forward substitution, one column per thread.
    if (tid < 64) {
        const int blk = tid >> 4, j = tid & 15, o = blk * 16;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = i == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) s -= sTf[(o + i) * PF + o + m] * x[m];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sLf[(o + i) * PF + o + j] = x[i];
    }
    __syncthreads();
    // Off-diagonal blocks, one block row at a time:
    //   L_{bi,cj} = -L_{bi,bi} * sum_{m=cj}^{bi-1} T_{bi,m} L_{m,cj}
    {
        const int r = tid >> 4, cc = tid & 15;
        for (int bi = 1; bi < 4; ++bi) {
            float wv[3];
            for (int cj = 0; cj < bi; ++cj) {
                float s = 0.f;
                for (int m = cj; m < bi; ++m)
#pragma unroll
                    for (int kk = 0; kk < 16; ++kk)
                        s += sTf[(bi * 16 + r) * PF + m * 16 + kk] * sLf[(m * 16 + kk) * PF + cj * 16 + cc];
                wv[cj] = s;
            }
            for (int cj = 0; cj < bi; ++cj) sLf[(bi * 16 + r) * PF + cj * 16 + cc] = wv[cj];
            __syncthreads();
            for (int cj = 0; cj < bi; ++cj) {
                float s = 0.f;
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    s -= sLf[(bi * 16 + r) * PF + bi * 16 + kk] * sLf[(bi * 16 + kk) * PF + cj * 16 + cc];
                wv[cj] = s;
            }
            __syncthreads();
            for (int cj = 0; cj < bi; ++cj) sLf[(bi * 16 + r) * PF + cj * 16 + cc] = wv[cj];
            __syncthreads();
        }
    }
    for (int i = tid; i < C * C; i += NT) {
        const int row = i / C, col = i - (i / C) * C;
        sL[row * PT + col] = E::to(col <= row ? sLf[row * PF + col] : 0.f);
    }
    __syncthreads();

    // ---- Y = L E~, U_z = L Z: wave w computes token rows 16w..16w+15. ----
    const int nks = (16 * (w + 1) + KS - 1) / KS;  // L is lower: K runs over tokens <= 16w+15
    f32x4 accY[CT], accU[CT];
#pragma unroll
    for (int tc = 0; tc < CT; ++tc) { accY[tc] = zero4(); accU[tc] = zero4(); }
    for (int ks = 0; ks < nks; ++ks) {
        const typename M::Frag la = M::load(sL + w * 16 * PT + ks * KS, PT);
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
            accY[tc] = M::mma(accY[tc], la, M::load(sET + tc * 16 * PT + ks * KS, PT));
            accU[tc] = M::mma(accU[tc], la, M::load(sZT + tc * 16 * PT + ks * KS, PT));
        }
    }
    // -Y^T and U_z^T for the next products (transposed: 4 consecutive tokens per lane).
#pragma unroll
    for (int tc = 0; tc < CT; ++tc) {
        const int col = tc * 16 + lr, tok = w * 16 + 4 * lq;
        store4f(sYT + col * PT + tok, -accY[tc]);
        store4f(sUzT + col * PT + tok, accU[tc]);
    }
    __syncthreads();  // E~^T and Z^T are dead from here
#pragma unroll
    for (int tc = 0; tc < CT; ++tc)
#pragma unroll
        for (int r = 0; r < 4; ++r) sYs[(w * 16 + 4 * lq + r) * PD + tc * 16 + lr] = E::to(accY[tc][r]);
    __syncthreads();
    copy_block(wY, D, sYs, PD, C, D, tid, NT);
    copy_block(wUzT, C, sUzT, PT, D, C, tid, NT);

    // ---- W_q = s (Q~ - A Y), O_z = s A U_z. ----
    f32x4 accW[CT], accO[CT];
#pragma unroll
    for (int tc = 0; tc < CT; ++tc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) accW[tc][r] = E::from(sQ[(w * 16 + 4 * lq + r) * PD + tc * 16 + lr]);
        accO[tc] = zero4();
    }
    for (int ks = 0; ks < nks; ++ks) {
        const typename M::Frag aa = M::load(sA + w * 16 * PT + ks * KS, PT);
#pragma unroll
        for (int tc = 0; tc < CT; ++tc) {
            accW[tc] = M::mma(accW[tc], aa, M::load(sYT + tc * 16 * PT + ks * KS, PT));
            accO[tc] = M::mma(accO[tc], aa, M::load(sUzT + tc * 16 * PT + ks * KS, PT));
        }
    }
    const float sc = a.scale;
#pragma unroll
    for (int tc = 0; tc < CT; ++tc) {
        const int col = tc * 16 + lr, tok = w * 16 + 4 * lq;
#pragma unroll
        for (int r = 0; r < 4; ++r) sWs[(tok + r) * PD + col] = E::to(sc * accW[tc][r]);
        store4f(sOzs + col * PT + tok, sc * accO[tc]);
    }
    __syncthreads();
    copy_block(wWq, D, sWs, PD, C, D, tid, NT);
    copy_block(wOzT, C, sOzs, PT, D, C, tid, NT);
}

// Sequential sweep over chunks for one (sequence, V head, value tile of BV =
// 16*NCT columns). NW = D/32 waves; wave w keeps state rows 32w..32w+31 in
// accumulator layout and computes token tiles [w*TPW, (w+1)*TPW) of P, R.
template <typename IO, int D, int NCT>
__global__ __launch_bounds__(2 * D) void chunk_sweep(ChunkArgs a, int NVT, int G) {
    using E = Elem<IO>;
    using M = Mma<IO>;
    using F = typename M::Frag;
    constexpr int NW = D / 32, BV = 16 * NCT, TPW = 4 / NW;
    constexpr int KS = M::KS, KD = D / KS, KC = C / KS;
    constexpr int LS = D + 8, LU = C + 8;
    __shared__ __align__(16) IO sST[BV * LS];  // S_c^T in the io dtype
    __shared__ __align__(16) IO sUT[BV * LU];  // U^T in the io dtype

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
    const size_t UE = chunk_ws_io_elems(D);
    IO *o = static_cast<IO *>(a.o);
    for (int c = 0; c < a.NC; ++c) {
        const size_t u = (size_t)bh * a.NC + c;
        const IO *Y = wsb + u * UE, *Wq = Y + C * D, *KT = Wq + C * D, *UzT = KT + D * C, *OzT = UzT + D * C;
        const float *gam = a.ws_gamma + u * D;

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
                const F ya = M::load(Y + T0 * D + ks * KS, D);
                const F wa = M::load(Wq + T0 * D + ks * KS, D);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const F sb = M::load(sST + 16 * ct * LS + ks * KS, LS);
                    accP[ct] = M::mma(accP[ct], ya, sb);
                    accR[ct] = M::mma(accR[ct], wa, sb);
                }
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int col = 16 * ct + lr, tok = T0 + 4 * lq;
                const f32x4 U = load4f(UzT + (size_t)(col0 + col) * C + tok) - accP[ct];
                const f32x4 O = accR[ct] + load4f(OzT + (size_t)(col0 + col) * C + tok);
                store4f(sUT + col * LU + tok, U);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = c * C + tok + r;
                    if (t < a.T) o[(((size_t)b * a.T + t) * a.Hv + h) * D + col0 + col] = E::to(O[r]);
                }
            }
        }
        __syncthreads();

#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int ch0 = 32 * w + 16 * rt;
            const f32x4 g4 = load4f(gam + ch0 + 4 * lq);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= g4;
#pragma unroll
            for (int ks = 0; ks < KC; ++ks) {
                const F ka = M::load(KT + ch0 * C + ks * KS, C);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    S[rt][ct] = M::mma(S[rt][ct], ka, M::load(sUT + 16 * ct * LU + ks * KS, LU));
            }
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

template <typename IO, int D, int NCT>
static hipError_t launch_chunk_t(const ChunkArgs &a, hipStream_t s) {
    using Lay = PrepLayout<IO, D>;
    static_assert(Lay::BYTES <= 160 * 1024, "LDS budget");
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_prep<IO, D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)Lay::BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const size_t units = (size_t)a.B * a.Hv * a.NC;
    if (units > 0) {
        hipLaunchKernelGGL((chunk_prep<IO, D>), dim3((unsigned)units), dim3(256), Lay::BYTES, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NVT = D / (16 * NCT);
    const int G = a.B * a.Hv * NVT;
    const int grid = (G + 7) / 8 * 8;
    hipLaunchKernelGGL((chunk_sweep<IO, D, NCT>), dim3(grid), dim3(2 * D), 0, s, a, NVT, G);
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
