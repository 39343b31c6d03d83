// decode.hip -- fused recurrent decode step (one token per sequence).
//
// The recurrent schedule of the mixer ("Kernel Triton recorrente fundido para
// decode", family analysis page "Uma análise das variantes de atenção linear
// da família DeltaNet"): decay the state, reduce it against the erase key,
// form the residual, write the rank-1 update, reduce against the query. The
// pages' kernel walks tokens inside one program per (sequence, V head, value
// tile); here a decode step is a single token, so the whole step is one pass
// over each state:
//
//   Sbar = Diag(alpha) S            alpha = exp(g)
//   r    = Sbar^T e, p = Sbar^T q   both k-axis reductions in the same pass
//   u    = z - r
//   o    = scale * (p + (q . k) u)  = scale * S_new^T q, the read after the write
//   S    = Sbar + k u^T             written back in place
//
// One workgroup of 256 threads owns one (sequence, V head) state of D x D
// fp32. Thread (ty, tx) holds float4 column group tx of rows ty, ty + RS,
// ... in registers, so every row is read and written as contiguous 16-byte
// accesses, and the state crosses HBM exactly once each way. The k-axis
// reductions combine lanes of a wave by shuffles and the waves through LDS.
// No matrix cores: the step is 0.9 flop per byte of state, bandwidth bound.
// The state is read and written with non-temporal accesses: nothing reuses it
// before the next step, by which time a model has streamed every other
// layer's state through the memory-side cache.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

template <typename IO, int D, int SPLIT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    using E = Elem<IO>;
    constexpr int NT = 256;
    constexpr int DC = D / SPLIT;  // value columns of this workgroup
    constexpr int CG = DC / 4;     // float4 column groups per row
    constexpr int RS = NT / CG;    // row stride between a thread's rows
    constexpr int NR = D / RS;     // rows per thread
    constexpr int NW = NT / 64;
    static_assert(NT % CG == 0 && D % RS == 0 && CG <= 64 && DC % 4 == 0, "tile shape");

    __shared__ float s_q[D], s_k[D], s_e[D], s_al[D];
    __shared__ float s_red[NW][2][DC];
    __shared__ float s_qk;

    const int bh = blockIdx.x / SPLIT, c0 = (blockIdx.x % SPLIT) * DC;
    const int b = bh / a.Hv;
    const int h = bh - b * a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int tid = threadIdx.x, tx = tid % CG, ty = tid / CG;
    const int wave = tid >> 6, lane = tid & 63;

    float *S = a.S + (size_t)bh * D * D + c0;
    f32x4 st[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) st[m] = load_state4(S + (size_t)(ty + m * RS) * D + 4 * tx);

    const IO *qp = static_cast<const IO *>(a.q) + ((size_t)b * a.Hqk + hq) * D;
    const IO *kp = static_cast<const IO *>(a.k) + ((size_t)b * a.Hqk + hq) * D;
    for (int i = tid; i < D; i += NT) {
        const float qi = E::load(qp + i), ki = E::load(kp + i);
        s_q[i] = qi;
        s_k[i] = ki;
        s_e[i] = a.beta ? a.beta[bh] * ki : E::load(static_cast<const IO *>(a.bg) + (size_t)bh * D + i) * ki;
        float al = 1.f;
        if (a.decay == DECAY_SCALAR) al = expf(a.g[bh]);
        else if (a.decay == DECAY_CHANNEL) al = expf(a.g[(size_t)bh * D + i]);
        s_al[i] = al;
    }
    __syncthreads();

    float pr[4] = {0.f, 0.f, 0.f, 0.f}, pp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NR; ++m) {
        const int i = ty + m * RS;
        const float al = s_al[i], e = s_e[i], qv = s_q[i];
        st[m] *= al;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pr[c] += st[m][c] * e;
            pp[c] += st[m][c] * qv;
        }
    }
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pr[c] += __shfl_xor(pr[c], off);
            pp[c] += __shfl_xor(pp[c], off);
        }
    }
    if (lane < CG) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_red[wave][0][4 * tx + c] = pr[c];
            s_red[wave][1][4 * tx + c] = pp[c];
        }
    }
    if (wave == 0) {
        float x = 0.f;
        for (int i = lane; i < D; i += 64) x += s_q[i] * s_k[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if (lane == 0) s_qk = x;
    }
    __syncthreads();

    const IO *vp = static_cast<const IO *>(a.v) + (size_t)bh * D + c0 + 4 * tx;
    const float bt = a.beta ? a.beta[bh] : 0.f;
    const float qk = s_qk;
    float u[4], o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        float r = 0.f, p = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            r += s_red[w][0][4 * tx + c];
            p += s_red[w][1][4 * tx + c];
        }
        const float vv = E::load(vp + c);
        const float z = a.beta ? bt * vv : E::load(static_cast<const IO *>(a.wg) + (size_t)bh * D + c0 + 4 * tx + c) * vv;
        u[c] = z - r;
        o[c] = a.scale * (p + qk * u[c]);
    }
#pragma unroll
    for (int m = 0; m < NR; ++m) {
        const float ki = s_k[ty + m * RS];
#pragma unroll
        for (int c = 0; c < 4; ++c) st[m][c] += ki * u[c];
        store_state4(S + (size_t)(ty + m * RS) * D + 4 * tx, st[m]);
    }
    if (ty == 0) {
        IO *op = static_cast<IO *>(a.o) + (size_t)bh * D + c0 + 4 * tx;
#pragma unroll
        for (int c = 0; c < 4; ++c) op[c] = E::to(o[c]);
    }
}

// 128 x 128 states are split over two workgroups by value columns (32 KiB of
// state each): streaming 32 KiB per workgroup reaches a higher HBM rate on
// MI355X than 64 KiB, and the columns are independent.
template <typename IO, int D>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
    constexpr int SPLIT = D == 128 ? 2 : 1;
    const unsigned grid = (unsigned)a.B * (unsigned)a.Hv * SPLIT;
    hipLaunchKernelGGL((decode_kernel<IO, D, SPLIT>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(int io, int D, const DecodeArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_decode_t<bf16_t, 32>(a, s);
        if (D == 64) return launch_decode_t<bf16_t, 64>(a, s);
        if (D == 128) return launch_decode_t<bf16_t, 128>(a, s);
    } else {
        if (D == 32) return launch_decode_t<float, 32>(a, s);
        if (D == 64) return launch_decode_t<float, 64>(a, s);
        if (D == 128) return launch_decode_t<float, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr

namespace gdr {

// dst[i] = src ? src[i] : 0 for i < n (zero fill or copy of a state block;
// a kernel rather than a memset so the call stays valid under graph capture).
__global__ __launch_bounds__(256) void state_fill_kernel(float *dst, const float *src, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_fill(float *dst, const float *src, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(state_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

}  // namespace gdr
