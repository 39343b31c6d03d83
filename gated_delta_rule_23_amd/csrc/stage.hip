// stage.hip -- the input stage's convolution as a pass of its own, for the
// chunked prefill of per-channel-decay layers (gdr_chunk_fwd_in with
// GDR_DECAY_CHANNEL).
//
// The input stage (page "Gated DeltaNet: o mixer em 48 das 64 camadas",
// section "Conceito": a causal depthwise convolution of kernel 4 over the
// projected q, k and v; normalised keys per the family analysis's notation;
// sigmoid gates and a softplus-shaped decay) is fused into the prefill's load
// stage for scalar-decay layers. With a per-channel decay the prefill's load
// stage already holds seven token-major tiles of the chunk, so there the
// convolution and the normalisation run first, over the whole call, and
// write the processed q, k, v into the call's workspace; the gate and decay
// activations, elementwise, stay in the prefill's load stage. The pass
// streams: each raw row is read once and each processed row written once.
//
//  stage_conv: one thread per 16-byte channel group of one (sequence, head)
//    row of q, k or v and a run of 16 tokens, walked in order with the 3 rows
//    before the current one kept in registers, so each raw row is read once
//    (plus 3 rows before each run); the D / V threads of a row are
//    consecutive lanes, so the norm of q and k is a DPP all-reduce inside the
//    wave. The thread of the last run also writes the outgoing convolution
//    state (the last 3 raw tokens, rows before the call taken from conv_in).
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {
namespace {

constexpr float kNormEps = 1e-12f;  // q, k = x / sqrt(|x|^2 + kNormEps)
constexpr int kRun = 16;            // tokens per thread of the convolution

template <typename IO> struct Vec16;  // 16 bytes of io elements, widened to float and back
template <> struct Vec16<bf16_t> {
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
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void widen(uint4 r, float *f) {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y); f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};

template <typename IO, int D>
__global__ __launch_bounds__(256) void stage_conv(StageArgs a) {
    using W = Vec16<IO>;
    constexpr int V = W::N, CO = D / V;  // channel groups per row
    static_assert(64 % CO == 0, "a row's lanes lie in one wave");
    const int NH = 2 * a.Hqk + a.Hv, NR = (a.T + kRun - 1) / kRun;
    // Thread: channel group cg of head row hh (q heads, then k, then v) for
    // the run of kRun tokens r kRun ..; lanes of a wave cover consecutive
    // head rows of one run, so each step's loads and stores are contiguous.
    const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long rows = (long long)a.B * NR * NH * CO;
    const bool valid = gid < rows;
    const long long g = valid ? gid : rows - 1;  // lanes past the end repeat the last group and store nothing
    const int cg = (int)(g % CO);
    const long long rh = g / CO;
    const int hh = (int)(rh % NH);
    const long long br = rh / NH;
    const int run = (int)(br % NR), b = (int)(br / NR);
    const int x = hh < a.Hqk ? 0 : hh < 2 * a.Hqk ? 1 : 2;
    const int H = x == 2 ? a.Hv : a.Hqk, head = x == 2 ? hh - 2 * a.Hqk : hh - x * a.Hqk;
    const IO *src = static_cast<const IO *>(x == 0 ? a.q : x == 1 ? a.k : a.v);
    IO *dst = static_cast<IO *>(x == 0 ? a.qo : x == 1 ? a.ko : a.vo);
    const size_t ch = (size_t)NH * D, c0 = (size_t)hh * D + V * cg;
    const auto at = [&](int tt) -> size_t { return (((size_t)b * a.T + tt) * H + head) * D + V * cg; };
    const int t0 = run * kRun, n = min(kRun, a.T - t0);

    f32x4 tp[V];  // this thread's channels' taps
#pragma unroll
    for (int c = 0; c < V; ++c) tp[c] = load4f(a.conv_w + (c0 + c) * 4);
    // The 3 raw rows before the run (from the incoming state, or zeros, before the sequence).
    uint4 wnd[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int tt = t0 - 3 + j;
        wnd[j] = tt >= 0 ? *reinterpret_cast<const uint4 *>(src + at(tt))
                 : a.conv_in ? *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.conv_in) +
                                                                 ((size_t)b * 3 + 3 + tt) * ch + c0)
                             : uint4{0u, 0u, 0u, 0u};
    }
    uint4 raw[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) raw[j] = j < n ? *reinterpret_cast<const uint4 *>(src + at(t0 + j)) : uint4{0u, 0u, 0u, 0u};
    float xs[3][V];
#pragma unroll
    for (int j = 0; j < 3; ++j) W::widen(wnd[j], xs[j]);
    // wnd keeps the 3 raw rows before the next token: after the run, the
    // sequence's last 3 when the run ends it.
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
        float cur[V], out[V];
        W::widen(raw[j], cur);
#pragma unroll
        for (int c = 0; c < V; ++c) out[c] = tp[c][0] * xs[0][c] + tp[c][1] * xs[1][c] + tp[c][2] * xs[2][c] + tp[c][3] * cur[c];
        if (x < 2) {  // q and k: normalised over the head
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < V; ++c) ss += out[c] * out[c];
            if constexpr (CO == 32) {
                ss = lanes_allreduce<16>(ss);
                ss += __shfl_xor(ss, 16);
            } else {
                ss = lanes_allreduce<CO>(ss);
            }
            const float f = 1.f / sqrtf(ss + kNormEps);
#pragma unroll
            for (int c = 0; c < V; ++c) out[c] *= f;
        }
        if (valid && j < n) *reinterpret_cast<uint4 *>(dst + at(t0 + j)) = W::pack(out);
#pragma unroll
        for (int c = 0; c < V; ++c) {
            xs[0][c] = xs[1][c];
            xs[1][c] = xs[2][c];
            xs[2][c] = cur[c];
        }
        if (j < n) {
            wnd[0] = wnd[1];
            wnd[1] = wnd[2];
            wnd[2] = raw[j];
        }
    }
    // The outgoing convolution state: the sequence's last 3 raw rows (rows
    // before the call come from the incoming state when T < 3).
    if (valid && a.conv_out && t0 + n == a.T) {
        IO *cout = static_cast<IO *>(a.conv_out) + (size_t)b * 3 * ch + c0;
#pragma unroll
        for (int j = 0; j < 3; ++j) *reinterpret_cast<uint4 *>(cout + (size_t)j * ch) = wnd[j];
    }
}

template <typename IO, int D>
hipError_t launch_stage_t(const StageArgs &a, hipStream_t s) {
    constexpr int CO = D / (16 / (int)sizeof(IO));
    const long long groups = (long long)a.B * ((a.T + kRun - 1) / kRun) * (2 * a.Hqk + a.Hv) * CO;
    if (groups > 0) {
        const long long grid = (groups + 255) / 256;
        if (grid > 0x7fffffffll) return hipErrorInvalidValue;
        hipLaunchKernelGGL((stage_conv<IO, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stage(int io, int D, const StageArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_stage_t<bf16_t, 32>(a, s);
        if (D == 64) return launch_stage_t<bf16_t, 64>(a, s);
        if (D == 128) return launch_stage_t<bf16_t, 128>(a, s);
    } else {
        if (D == 32) return launch_stage_t<float, 32>(a, s);
        if (D == 64) return launch_stage_t<float, 64>(a, s);
        if (D == 128) return launch_stage_t<float, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
