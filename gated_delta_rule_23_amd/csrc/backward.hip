// backward.hip -- gradients of the gated delta-rule recurrence, recurrent form.
//
// The page "Resumo Técnico: Gated DeltaNet-2", section "Treinamento Paralelo
// Eficiente por Blocos", names a backward pass in which the per-channel
// gates enter the gradient accumulation; it prints no formula. What is
// computed here is the exact gradient of the forward recurrence for given
// dL/do and dL/dS_T. Per (sequence, V head), walking the tokens in reverse
// with dS = dL/dS_T:
//
//   dS    += s q_t do_t^T        dq_t = s S_t do_t
//   du_t   = dS^T k_t            dk_t = dS u_t + (beta_t or b_t) . de_t
//   dSbar  = dS - e_t du_t^T     de_t = -Sbar_t du_t,   dz_t = du_t
//   dalpha = rowsum(dSbar . S_{t-1}),   dg_t = alpha_t . dalpha
//   dS     = Diag(alpha_t) dSbar
//
// with Sbar_t = Diag(alpha_t) S_{t-1}, u_t = z_t - Sbar_t^T e_t and
// S_t = Sbar_t + k_t u_t^T, then dv, dw, db, dbeta through e = beta k or b.k
// and z = beta v or w.v.
//
// Three kernels:
//  1. bwd_ckpt_kernel runs the forward recurrence and stores the state that
//     enters every block of kBwdBlock = 4 tokens.
//  2. bwd_kernel walks the blocks from the last: it replays the block from
//     its checkpoint, keeping each state entering a token in shared memory,
//     then runs the reverse recurrence above over the block with dS in
//     registers.
//  3. bwd_reduce_kernel sums what the value-column tiles contributed to the
//     key-axis gradients (dq, dk, de, dalpha) and forms the gate gradients.
//
// A workgroup of kernels 1-2 owns (sequence, V head, kBwdCols = 32 value
// columns) and each of its 4 waves an 8-column slice with every key row:
// lane (rg, c2) holds float4 columns 4 c2 .. 4 c2 + 3 of the slice for state
// rows rg, rg + 32, ... So the per-token sums over the key axis stay inside
// the wave (DPP within 16-lane rows, two shuffles across them): the token
// loop has no barrier. The sums over value columns (dq, dk, de, dalpha, and
// dbeta's value part) are formed per wave, kept in shared memory for the
// block, and added over the 4 waves once per block. Vector ALU only.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

namespace {

constexpr int BL = kBwdBlock;
constexpr int CT = kBwdCols;  // value columns per workgroup
constexpr int NWV = 4;        // waves per workgroup
constexpr int CW = CT / NWV;  // value columns per wave
constexpr int NTB = 64 * NWV;
static_assert(CW == 8, "lane layout: two float4 column groups per wave");

template <int D>
struct BwdShape {
    static constexpr int NRW = D / 32;  // state rows per lane
    static constexpr int TILES = D / CT;
};

// One block of tokens' inputs, staged in shared memory, and the per-wave sums
// over value columns for the block.
template <int D>
struct BwdStage {
    f32x4 rv[BL][D];                                     // per token and key channel: (q, k, e, alpha)
    float z[BL][CT], dO[BL][CT], v[BL][CT], wv[BL][CT];  // the workgroup's value columns; wv = the write gate
    float part[NWV][BL][4][D];                           // per wave: s S_t do, dS u, -Sbar du, dalpha
    float partb[NWV][BL];                                // per wave: v . du
};

// The same inputs in registers, loaded one block ahead of their use.
template <int D>
struct BwdIn {
    static constexpr int NE = (BL * D + NTB - 1) / NTB, NC = (BL * CT + NTB - 1) / NTB;
    f32x4 rv[NE];
    float z[NC], dO[NC], v[NC], wv[NC];
};

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the key axis for this lane's 4 columns: the 32 lanes of the wave
// with the same column group (lane bit 0): lanes 2 apart (quad swap), 4 and 8
// apart (rotations within the 16-lane row), then 16 and 32 apart (shuffles).
__device__ __forceinline__ f32x4 keysum(f32x4 p) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float x = p[c];
        x += dpp<0x4E>(x);   // quad [2,3,0,1]
        x += dpp<0x124>(x);  // row_ror:4
        x += dpp<0x128>(x);  // row_ror:8
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        p[c] = x;
    }
    return p;
}
// Sum over the wave's 8 value columns: the lane's 4, then the neighbour lane's.
__device__ __forceinline__ float colsum8(float x) { return x + dpp<0xB1>(x); }  // quad [1,0,3,2]

template <typename IO, int D, bool BWD>
__device__ __forceinline__ void bwd_load(const BwdArgs &a, BwdIn<D> &in, int b, int h, int hq, int col0, int t0,
                                         int n) {
    using E = Elem<IO>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < BwdIn<D>::NE; ++e) {
        const int x = tid + NTB * e, tok = x / D, i = x - tok * D;
        f32x4 r = f32x4{0.f, 0.f, 0.f, 1.f};
        if (x < BL * D && tok < n) {
            const size_t t = (size_t)b * a.T + t0 + tok;
            const size_t qi = (t * a.Hqk + hq) * D + i, vi = (t * a.Hv + h) * D + i;
            const float kk = E::load(static_cast<const IO *>(a.k) + qi);
            r[0] = BWD ? E::load(static_cast<const IO *>(a.q) + qi) : 0.f;
            r[1] = kk;
            r[2] = (a.beta ? a.beta[t * a.Hv + h] : E::load(static_cast<const IO *>(a.bg) + vi)) * kk;
            if (a.decay == DECAY_SCALAR) r[3] = expf(a.g[t * a.Hv + h]);
            else if (a.decay == DECAY_CHANNEL) r[3] = expf(a.g[vi]);
        }
        in.rv[e] = r;
    }
#pragma unroll
    for (int e = 0; e < BwdIn<D>::NC; ++e) {
        const int x = tid + NTB * e, tok = x / CT, c = x - tok * CT;
        in.z[e] = in.dO[e] = in.v[e] = in.wv[e] = 0.f;
        if (x < BL * CT && tok < n) {
            const size_t t = (size_t)b * a.T + t0 + tok;
            const size_t vi = (t * a.Hv + h) * D + col0 + c;
            in.v[e] = E::load(static_cast<const IO *>(a.v) + vi);
            in.wv[e] = a.beta ? a.beta[t * a.Hv + h] : E::load(static_cast<const IO *>(a.wg) + vi);
            in.z[e] = in.wv[e] * in.v[e];
            if (BWD) in.dO[e] = E::load(static_cast<const IO *>(a.dO) + vi);
        }
    }
}

template <int D>
__device__ __forceinline__ void bwd_put(const BwdIn<D> &in, BwdStage<D> &s) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < BwdIn<D>::NE; ++e) {
        const int x = tid + NTB * e;
        if (x < BL * D) s.rv[x / D][x % D] = in.rv[e];
    }
#pragma unroll
    for (int e = 0; e < BwdIn<D>::NC; ++e) {
        const int x = tid + NTB * e;
        if (x < BL * CT) {
            const int tok = x / CT, c = x - tok * CT;
            s.z[tok][c] = in.z[e];
            s.dO[tok][c] = in.dO[e];
            s.v[tok][c] = in.v[e];
            s.wv[tok][c] = in.wv[e];
        }
    }
}

// Lane coordinates: row group rg, this lane's first column within the
// workgroup's 32.
struct Lane {
    int rg, cc;
    __device__ __forceinline__ Lane() {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        rg = lane >> 1;
        cc = CW * w + 4 * (lane & 1);
    }
};

// One forward step of this lane's part of the state: S <- Sbar + k u^T,
// returning u for its 4 columns.
template <int D>
__device__ __forceinline__ f32x4 fwd_step(f32x4 (&S)[BwdShape<D>::NRW], const BwdStage<D> &s, int tok,
                                          const Lane &L) {
    f32x4 pr = zero4(), rv[BwdShape<D>::NRW];
#pragma unroll
    for (int j = 0; j < BwdShape<D>::NRW; ++j) {
        rv[j] = s.rv[tok][L.rg + 32 * j];
        S[j] *= rv[j][3];
        pr += S[j] * rv[j][2];
    }
    const f32x4 u = load4f(&s.z[tok][L.cc]) - keysum(pr);
#pragma unroll
    for (int j = 0; j < BwdShape<D>::NRW; ++j) S[j] += rv[j][1] * u;
    return u;
}

template <typename IO, int D>
__global__ __launch_bounds__(NTB) void bwd_ckpt_kernel(BwdArgs a) {
    using Sh = BwdShape<D>;
    extern __shared__ __align__(16) unsigned char smem[];
    BwdStage<D> &s = *reinterpret_cast<BwdStage<D> *>(smem);
    const int tile = blockIdx.x % Sh::TILES, bh = blockIdx.x / Sh::TILES, b = bh / a.Hv, h = bh - b * a.Hv;
    const int hq = h / (a.Hv / a.Hqk), col0 = tile * CT;
    const Lane L;
    f32x4 S[Sh::NRW];
#pragma unroll
    for (int j = 0; j < Sh::NRW; ++j)
        S[j] = a.S0 ? load4f(a.S0 + ((size_t)bh * D + L.rg + 32 * j) * D + col0 + L.cc) : zero4();
    const int NB = (a.T + BL - 1) / BL;
    BwdIn<D> in;
    bwd_load<IO, D, false>(a, in, b, h, hq, col0, 0, min(BL, a.T));
    for (int m = 0; m < NB; ++m) {
        float *ck = a.ws_ck + ((size_t)m * a.B * a.Hv + bh) * D * D;
#pragma unroll
        for (int j = 0; j < Sh::NRW; ++j) store4f(ck + (size_t)(L.rg + 32 * j) * D + col0 + L.cc, S[j]);
        const int t0 = m * BL, n = min(BL, a.T - t0);
        __syncthreads();  // the previous block's inputs are no longer read
        bwd_put<D>(in, s);
        __syncthreads();
        if (m + 1 < NB) bwd_load<IO, D, false>(a, in, b, h, hq, col0, t0 + BL, min(BL, a.T - t0 - BL));
        for (int tok = 0; tok < n; ++tok) (void)fwd_step<D>(S, s, tok, L);
    }
}

template <typename IO, int D>
__global__ __launch_bounds__(NTB) void bwd_kernel(BwdArgs a) {
    using Sh = BwdShape<D>;
    constexpr int NRW = Sh::NRW, TILES = Sh::TILES;
    extern __shared__ __align__(16) unsigned char smem[];
    BwdStage<D> &s = *reinterpret_cast<BwdStage<D> *>(smem);
    // The states entering each token of the block, lane-private: [token][row j][thread].
    f32x4 *Sx = reinterpret_cast<f32x4 *>(smem + sizeof(BwdStage<D>));
    const int tile = blockIdx.x % TILES, bh = blockIdx.x / TILES, b = bh / a.Hv, h = bh - b * a.Hv;
    const int hq = h / (a.Hv / a.Hqk), col0 = tile * CT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const Lane L;
    const size_t TH = (size_t)a.B * a.T * a.Hv;

    f32x4 dS[NRW];
#pragma unroll
    for (int j = 0; j < NRW; ++j)
        dS[j] = a.dST ? load4f(a.dST + ((size_t)bh * D + L.rg + 32 * j) * D + col0 + L.cc) : zero4();
    const int NB = (a.T + BL - 1) / BL;
    // Block m's inputs and checkpoint are loaded while block m + 1 is processed.
    const auto ckpt = [&](int m) { return a.ws_ck + ((size_t)m * a.B * a.Hv + bh) * D * D; };
    BwdIn<D> in;
    f32x4 Sn[NRW];
    bwd_load<IO, D, true>(a, in, b, h, hq, col0, (NB - 1) * BL, a.T - (NB - 1) * BL);
#pragma unroll
    for (int j = 0; j < NRW; ++j) Sn[j] = load4f(ckpt(NB - 1) + (size_t)(L.rg + 32 * j) * D + col0 + L.cc);
    for (int m = NB - 1; m >= 0; --m) {
        const int t0 = m * BL, n = min(BL, a.T - t0);
        f32x4 S[NRW];
#pragma unroll
        for (int j = 0; j < NRW; ++j) S[j] = Sn[j];
        __syncthreads();  // the previous block's inputs and sums are no longer read
        bwd_put<D>(in, s);
        __syncthreads();
        if (m > 0) {
            bwd_load<IO, D, true>(a, in, b, h, hq, col0, t0 - BL, BL);
#pragma unroll
            for (int j = 0; j < NRW; ++j) Sn[j] = load4f(ckpt(m - 1) + (size_t)(L.rg + 32 * j) * D + col0 + L.cc);
        }
        // Replay: the state entering each token, and each token's u.
        f32x4 u[BL];
#pragma unroll
        for (int tok = 0; tok < BL; ++tok) {
            if (tok < n) {
#pragma unroll
                for (int j = 0; j < NRW; ++j) Sx[(tok * NRW + j) * NTB + tid] = S[j];
                u[tok] = fwd_step<D>(S, s, tok, L);
            }
        }
        // Reverse recurrence over the block.
#pragma unroll
        for (int tok = BL - 1; tok >= 0; --tok) {
            if (tok < n) {
                const f32x4 dO4 = load4f(&s.dO[tok][L.cc]);
                f32x4 Sp[NRW], Sb[NRW], rv[NRW], pd = zero4();
                float xq[NRW], xk[NRW];
#pragma unroll
                for (int j = 0; j < NRW; ++j) {
                    rv[j] = s.rv[tok][L.rg + 32 * j];  // (q, k, e, alpha)
                    Sp[j] = Sx[(tok * NRW + j) * NTB + tid];
                    Sb[j] = Sp[j] * rv[j][3];
                    const f32x4 St = Sb[j] + rv[j][1] * u[tok];
                    dS[j] += (a.scale * rv[j][0]) * dO4;
                    xq[j] = a.scale * dot4(St, dO4);
                    xk[j] = dot4(dS[j], u[tok]);
                    pd += dS[j] * rv[j][1];
                }
                const f32x4 du = keysum(pd);
#pragma unroll
                for (int j = 0; j < NRW; ++j) {
                    const int r = L.rg + 32 * j;
                    const float xe = -dot4(Sb[j], du);
                    const f32x4 dSb = dS[j] - rv[j][2] * du;
                    const float xa = dot4(dSb, Sp[j]);
                    dS[j] = dSb * rv[j][3];
                    const float q1 = colsum8(xq[j]), k1 = colsum8(xk[j]), e1 = colsum8(xe), a1 = colsum8(xa);
                    if ((lane & 1) == 0) {
                        s.part[w][tok][0][r] = q1;
                        s.part[w][tok][1][r] = k1;
                        s.part[w][tok][2][r] = e1;
                        s.part[w][tok][3][r] = a1;
                    }
                }
                // dz = du: the value-column gradients, from row group 0 (which holds du for its columns).
                const f32x4 v4 = load4f(&s.v[tok][L.cc]);
                if (L.rg == 0) {
                    const size_t vi = (((size_t)b * a.T + t0 + tok) * a.Hv + h) * D + col0 + L.cc;
                    store4f(a.dv + vi, load4f(&s.wv[tok][L.cc]) * du);
                    if (a.dw) store4f(a.dw + vi, v4 * du);
                }
                const float xb = colsum8(dot4(v4, du));
                if (lane == 0) s.partb[w][tok] = xb;
            }
        }
        __syncthreads();  // every wave's sums for the block are in shared memory
        // Add the 4 waves' sums and write this workgroup's partials.
        for (int x = tid; x < n * 4 * D; x += NTB) {
            const int tok = x / (4 * D), qd = (x / D) % 4, r = x % D;
            const float sum = s.part[0][tok][qd][r] + s.part[1][tok][qd][r] + s.part[2][tok][qd][r] +
                              s.part[3][tok][qd][r];
            const size_t row = ((size_t)b * a.T + t0 + tok) * a.Hv + h;
            a.ws_part[((size_t)(qd * TILES + tile) * TH + row) * D + r] = sum;
        }
        if (a.dbeta && tid < n) {
            const size_t row = ((size_t)b * a.T + t0 + tid) * a.Hv + h;
            a.ws_part[(size_t)4 * TILES * TH * D + (size_t)tile * TH + row] =
                s.partb[0][tid] + s.partb[1][tid] + s.partb[2][tid] + s.partb[3][tid];
        }
    }
    if (a.dS0)
#pragma unroll
        for (int j = 0; j < NRW; ++j)
            store4f(a.dS0 + ((size_t)bh * D + L.rg + 32 * j) * D + col0 + L.cc, dS[j]);
}

// One workgroup per (sequence, token, QK head): sums the tiles' partials of
// every V head of the group into dq and dk, and forms that token's gate
// gradients.
template <typename IO, int D>
__global__ __launch_bounds__(128) void bwd_reduce_kernel(BwdArgs a) {
    using E = Elem<IO>;
    constexpr int TILES = BwdShape<D>::TILES;
    __shared__ float red[2][2];
    const int hq = blockIdx.x % a.Hqk;
    const size_t bt = blockIdx.x / a.Hqk;  // b * T + t
    const int i = threadIdx.x, lane = i & 63, wave = i >> 6, grp = a.Hv / a.Hqk;
    const bool on = i < D;
    const size_t TH = (size_t)a.B * a.T * a.Hv;
    const size_t qi = (bt * a.Hqk + hq) * D + i;
    const float kk = on ? E::load(static_cast<const IO *>(a.k) + qi) : 0.f;
    float dq = 0.f, dk = 0.f;
    for (int hh = 0; hh < grp; ++hh) {
        const size_t row = bt * a.Hv + (size_t)hq * grp + hh;
        float pq = 0.f, pk = 0.f, pe = 0.f, pa = 0.f;
        if (on)
#pragma unroll
            for (int t = 0; t < TILES; ++t) {
                pq += a.ws_part[((size_t)(0 * TILES + t) * TH + row) * D + i];
                pk += a.ws_part[((size_t)(1 * TILES + t) * TH + row) * D + i];
                pe += a.ws_part[((size_t)(2 * TILES + t) * TH + row) * D + i];
                pa += a.ws_part[((size_t)(3 * TILES + t) * TH + row) * D + i];
            }
        const float ge = a.beta ? a.beta[row] : (on ? E::load(static_cast<const IO *>(a.bg) + row * D + i) : 0.f);
        dq += pq;
        dk += pk + ge * pe;
        if (a.db && on) a.db[row * D + i] = kk * pe;
        if (a.decay == DECAY_CHANNEL && on) a.dg[row * D + i] = expf(a.g[row * D + i]) * pa;
        if (a.decay == DECAY_SCALAR || a.beta) {
            float sa = pa, sb = kk * pe;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                sa += __shfl_xor(sa, off);
                sb += __shfl_xor(sb, off);
            }
            if (lane == 0) {
                red[0][wave] = sa;
                red[1][wave] = sb;
            }
            __syncthreads();
            if (i == 0) {
                if (a.decay == DECAY_SCALAR) a.dg[row] = expf(a.g[row]) * (red[0][0] + red[0][1]);
                if (a.beta) {
                    float zb = 0.f;
                    for (int t = 0; t < TILES; ++t) zb += a.ws_part[(size_t)4 * TILES * TH * D + (size_t)t * TH + row];
                    a.dbeta[row] = red[1][0] + red[1][1] + zb;
                }
            }
            __syncthreads();
        }
    }
    if (on) {
        a.dq[qi] = dq;
        a.dk[qi] = dk;
    }
}

template <typename IO, int D>
hipError_t launch_backward_t(const BwdArgs &a, hipStream_t s) {
    using Sh = BwdShape<D>;
    constexpr size_t lds_ck = sizeof(BwdStage<D>);
    constexpr size_t lds_bw = sizeof(BwdStage<D>) + (size_t)BL * Sh::NRW * NTB * sizeof(f32x4);
    static_assert(lds_bw <= 160 * 1024, "shared memory");
    static const hipError_t attr = [] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_ckpt_kernel<IO, D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_ck);
        if (e != hipSuccess) return e;
        return hipFuncSetAttribute(reinterpret_cast<const void *>(&bwd_kernel<IO, D>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bw);
    }();
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)a.B * (unsigned)a.Hv * Sh::TILES;
    hipLaunchKernelGGL((bwd_ckpt_kernel<IO, D>), dim3(grid), dim3(NTB), lds_ck, s, a);
    hipLaunchKernelGGL((bwd_kernel<IO, D>), dim3(grid), dim3(NTB), lds_bw, s, a);
    hipLaunchKernelGGL((bwd_reduce_kernel<IO, D>), dim3((unsigned)((size_t)a.B * a.T * a.Hqk)), dim3(128), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(int io, int D, const BwdArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_backward_t<bf16_t, 32>(a, s);
        if (D == 64) return launch_backward_t<bf16_t, 64>(a, s);
        if (D == 128) return launch_backward_t<bf16_t, 128>(a, s);
    } else {
        if (D == 32) return launch_backward_t<float, 32>(a, s);
        if (D == 64) return launch_backward_t<float, 64>(a, s);
        if (D == 128) return launch_backward_t<float, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
