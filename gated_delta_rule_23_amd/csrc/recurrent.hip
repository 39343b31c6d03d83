// recurrent.hip -- fused recurrent forward over a run of tokens.
//
// The recurrent form of the mixer ("Kernel Triton recorrente fundido para
// decode", family analysis page "Uma análise das variantes de atenção linear
// da família DeltaNet"): one program per (sequence, V head, value tile) walks
// the tokens in order with its block of the state held on chip, so the state
// crosses HBM once each way per call, whatever the number of tokens. Per
// token, with alpha = exp(g):
//
//   r = Sbar^T e = S^T (alpha . e)      p = Sbar^T q = S^T (alpha . q)
//   u = z - r                           o = scale * (p + (q . k) u)
//   S = Diag(alpha) S + k u^T
//
// o is the read after the write, scale * S_new^T q, written out as
// p + (q . k) u so that one pass over the state serves both reductions.
//
// Value columns of the state never mix: u_j, o_j and the update of column j
// use column j and the key-axis vectors only. So each wave owns CW columns
// and all D rows of one head, and both key-axis reductions stay inside the
// wave: lane (r, c) holds float4 column group c of rows r*RPL ... r*RPL +
// RPL-1 in registers, and the NRL lanes sharing a column group sum their
// partial results with an all-reduce of DPP row permutations (no LDS, no
// barrier). The waves of a workgroup share only the token inputs, staged in
// LDS TB tokens at a time already combined into alpha.e, alpha.q, k (and
// alpha per key channel), z and q . k; one barrier per staged block.
//
// The state is streamed with non-temporal loads and stores (it is not reused
// within the call, and a model touches every other layer's state before this
// one's next call). Work per token and head is about 4 D^2 flops against
// D^2 fp32 of state that is read and written once per call: a run of a few
// tokens is bound by HBM, a long one by the vector ALUs (long prefills belong
// to the chunked path, whose products run on the matrix cores).
//
// With the input stage (RAW), q, k and v arrive as raw projections: the
// staging pass convolves each token's 4-token window (the depthwise causal
// convolution of kernel 4; tokens before the call from the convolution
// state), normalises q and k over the head, and applies the gate and decay
// activations before staging; the processed values exist only on chip.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

template <int D, int CW, bool CHAN>
struct RecurCfg {
    static constexpr int NCG = CW / 4;             // float4 column groups per wave
    static constexpr int NRL = 64 / NCG;           // lanes sharing a column group
    static constexpr int RPL = D / NRL;            // rows per lane
    static constexpr int NWB = D / CW < 4 ? D / CW : 4;  // waves per workgroup
    static constexpr int NT = 64 * NWB;
    static constexpr int TILES = D / (NWB * CW);   // workgroups per (sequence, V head)
    static constexpr int TB = 8;                   // tokens staged per block
    // Staged token layout (floats). Key-axis arrays are stored per lane row
    // block with 4 floats of padding, so the NRL distinct 16-byte reads of a
    // wave fall in different LDS banks.
    static constexpr int RP = RPL + 4;
    static constexpr int DP = NRL * RP;
    static constexpr int OFF_AE = 0, OFF_AQ = DP, OFF_K = 2 * DP, OFF_AL = 3 * DP;
    static constexpr int OFF_Z = (CHAN ? 4 : 3) * DP;
    static constexpr int OFF_MISC = OFF_Z + D;     // q . k, scalar alpha
    static constexpr int STR = OFF_MISC + 4;
    static_assert(RPL % 4 == 0 && NRL >= 8 && NRL <= 16 && D % (NWB * CW) == 0, "recurrent tile shape");
};

__device__ __forceinline__ f32x4 exp4(f32x4 g) { return f32x4{expf(g[0]), expf(g[1]), expf(g[2]), expf(g[3])}; }

// q and k are normalised as x / sqrt(sum x^2 + kNormEps).
constexpr float kNormEps = 1e-12f;

// Input-stage activations: the logistic function for the gates, softplus
// for the decay.
__device__ __forceinline__ float sigmoid1(float x) { return act_sigmoid(x); }
__device__ __forceinline__ f32x4 sigmoid4(f32x4 x) {
    return f32x4{sigmoid1(x[0]), sigmoid1(x[1]), sigmoid1(x[2]), sigmoid1(x[3])};
}
__device__ __forceinline__ float softplus1(float x) { return act_softplus(x); }

// One 4-channel slice of the input stage for token t of sequence b: the
// depthwise causal convolution of kernel 4 over tokens t-3 .. t (tokens
// before 0 from the convolution state, zeros without one). x points at
// channel group i0 of token 0 of the sequence in a [T, H, D] array (token
// stride ts); cin at the same channels of the state's first row (row
// stride ch) or null; taps at this slice's [4][4] taps (channel-major).
template <typename IO>
__device__ __forceinline__ f32x4 conv4_slice(const IO *x, size_t ts, int t, const IO *cin, size_t ch,
                                             const float *taps) {
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tj = t - 3 + j;
        f32x4 xj{0.f, 0.f, 0.f, 0.f};
        if (tj >= 0) xj = load4f(x + (size_t)tj * ts);
        else if (cin) xj = load4f(cin + (size_t)(3 + tj) * ch);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += taps[4 * c + j] * xj[c];
    }
    return acc;
}

template <typename IO, int D, int CW, bool CHAN, bool RAW>
__global__ __launch_bounds__((RecurCfg<D, CW, CHAN>::NT)) void recurrent_kernel(RecurArgs a) {
    using C = RecurCfg<D, CW, CHAN>;
    constexpr int G = D / 4;  // 4-element groups of one token's key or value vector
    __shared__ __align__(16) float lds[C::TB * C::STR];

    const int tile = blockIdx.x % C::TILES;
    const int bh = blockIdx.x / C::TILES;
    const int b = bh / a.Hv, h = bh - b * a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, r = lane % C::NRL, cg = lane / C::NRL;
    const int col = (tile * C::NWB + wv) * CW + 4 * cg;  // first of this lane's four value columns
    const size_t sbase = (size_t)bh * D * D + (size_t)(r * C::RPL) * D + col;

    f32x4 st[C::RPL];
#pragma unroll
    for (int m = 0; m < C::RPL; ++m) st[m] = a.S0 ? load_state4(a.S0 + sbase + (size_t)m * D) : f32x4{0.f, 0.f, 0.f, 0.f};

    const IO *qg = static_cast<const IO *>(a.q), *kg = static_cast<const IO *>(a.k);
    const IO *vg = static_cast<const IO *>(a.v);
    const IO *bgp = static_cast<const IO *>(a.bg), *wgp = static_cast<const IO *>(a.wg);
    IO *og = static_cast<IO *>(a.o);

    for (int t0 = 0; t0 < a.T; t0 += C::TB) {
        const int nt = a.T - t0 < C::TB ? a.T - t0 : C::TB;
        if (t0 > 0) __syncthreads();  // every wave is done with the previous block
        // Stage: one thread per (token, 4 key/value channels); a token's G
        // threads are consecutive lanes of one wave.
        for (int u = tid; u < nt * G; u += C::NT) {
            const int tt = u / G, i0 = 4 * (u - tt * G);
            const size_t tok = (size_t)b * a.T + t0 + tt;
            const size_t xk = (tok * a.Hqk + hq) * D + i0;
            const size_t xs = tok * a.Hv + h;
            const size_t xv = xs * D + i0;
            f32x4 q, k, v, e, z, al;
            float as = 1.f;
            if constexpr (RAW) {
                // Input stage: convolve the raw projections, normalise q and k
                // over the head (the token's G lanes), gates from their inputs.
                const int t = t0 + tt;
                const size_t ch = (size_t)(2 * a.Hqk + a.Hv) * D;
                const size_t sqk = (size_t)a.Hqk * D, sv = (size_t)a.Hv * D;
                const size_t cq = (size_t)hq * D + i0, ck = sqk + cq, cv = 2 * sqk + (size_t)h * D + i0;
                const IO *cin = static_cast<const IO *>(a.conv_in) + (size_t)b * 3 * ch;
                const bool has_in = a.conv_in != nullptr;
                const size_t seq_qk = (size_t)b * a.T * sqk, seq_v = (size_t)b * a.T * sv;
                q = conv4_slice(qg + seq_qk + cq, sqk, t, has_in ? cin + cq : nullptr, ch, a.conv_w + cq * 4);
                k = conv4_slice(kg + seq_qk + cq, sqk, t, has_in ? cin + ck : nullptr, ch, a.conv_w + ck * 4);
                v = conv4_slice(vg + seq_v + (size_t)h * D + i0, sv, t, has_in ? cin + cv : nullptr, ch,
                                a.conv_w + cv * 4);
                float nq = q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3];
                float nk = k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3];
#pragma unroll
                for (int off = 1; off < G; off <<= 1) {
                    nq += __shfl_xor(nq, off);
                    nk += __shfl_xor(nk, off);
                }
                q *= 1.f / sqrtf(nq + kNormEps);
                k *= 1.f / sqrtf(nk + kNormEps);
                if (a.beta) {
                    const float bt = sigmoid1(a.beta[xs]);
                    e = bt * k;
                    z = bt * v;
                } else {
                    e = sigmoid4(load4f(bgp + xv)) * k;
                    z = sigmoid4(load4f(wgp + xv)) * v;
                }
                const float c = a.decay_scale ? a.decay_scale[h] : 1.f;
                if constexpr (CHAN) {
                    const f32x4 gi = load4f(a.g + xv);
                    al = exp4(f32x4{-c * softplus1(gi[0]), -c * softplus1(gi[1]), -c * softplus1(gi[2]),
                                    -c * softplus1(gi[3])});
                } else {
                    if (a.decay == DECAY_SCALAR) as = expf(-c * softplus1(a.g[xs]));
                    al = f32x4{as, as, as, as};
                }
            } else {
                q = load4f(qg + xk);
                k = load4f(kg + xk);
                v = load4f(vg + xv);
                if (a.beta) {
                    const float bt = a.beta[xs];
                    e = bt * k;
                    z = bt * v;
                } else {
                    e = load4f(bgp + xv) * k;
                    z = load4f(wgp + xv) * v;
                }
                if constexpr (CHAN) {
                    al = exp4(load4f(a.g + xv));
                } else {
                    if (a.decay == DECAY_SCALAR) as = expf(a.g[xs]);
                    al = f32x4{as, as, as, as};
                }
            }
            float *L = lds + tt * C::STR;
            const int p = (i0 / C::RPL) * C::RP + i0 % C::RPL;
            store4f(L + C::OFF_AE + p, al * e);
            store4f(L + C::OFF_AQ + p, al * q);
            store4f(L + C::OFF_K + p, k);
            if constexpr (CHAN) store4f(L + C::OFF_AL + p, al);
            store4f(L + C::OFF_Z + i0, z);
            float qk = q[0] * k[0] + q[1] * k[1] + q[2] * k[2] + q[3] * k[3];
#pragma unroll
            for (int off = 1; off < G; off <<= 1) qk += __shfl_xor(qk, off);
            if (i0 == 0) {
                L[C::OFF_MISC] = qk;
                L[C::OFF_MISC + 1] = as;
            }
        }
        __syncthreads();

        for (int tt = 0; tt < nt; ++tt) {
            const float *L = lds + tt * C::STR;
            const float *Lr = L + r * C::RP;
            f32x4 pr{0.f, 0.f, 0.f, 0.f}, pp{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m4 = 0; m4 < C::RPL / 4; ++m4) {
                const f32x4 ae = load4f(Lr + C::OFF_AE + 4 * m4), aq = load4f(Lr + C::OFF_AQ + 4 * m4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pr += st[4 * m4 + j] * ae[j];
                    pp += st[4 * m4 + j] * aq[j];
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pr[c] = lanes_allreduce<C::NRL>(pr[c]);
                pp[c] = lanes_allreduce<C::NRL>(pp[c]);
            }
            const f32x4 u = load4f(L + C::OFF_Z + col) - pr;
            if (r == 0) {
                const size_t tok = (size_t)b * a.T + t0 + tt;
                store4f(og + (tok * a.Hv + h) * D + col, a.scale * (pp + L[C::OFF_MISC] * u));
            }
            const float as = L[C::OFF_MISC + 1];
#pragma unroll
            for (int m4 = 0; m4 < C::RPL / 4; ++m4) {
                const f32x4 k4 = load4f(Lr + C::OFF_K + 4 * m4);
                f32x4 al4;
                if constexpr (CHAN) al4 = load4f(Lr + C::OFF_AL + 4 * m4);
                else al4 = f32x4{as, as, as, as};
#pragma unroll
                for (int j = 0; j < 4; ++j) st[4 * m4 + j] = st[4 * m4 + j] * al4[j] + k4[j] * u;
            }
        }
    }

#pragma unroll
    for (int m = 0; m < C::RPL; ++m) store_state4(a.ST + sbase + (size_t)m * D, st[m]);

    if constexpr (RAW) {
        // The convolution state after the call: the last 3 raw tokens
        // (token T-3+j in row j; rows before token 0 come from the incoming
        // state). Tile 0 of each V head writes its v channels; the first V
        // head of each QK group also writes the group's q and k channels.
        if (a.conv_out && tile == 0) {
            const bool qk_too = h % (a.Hv / a.Hqk) == 0;
            const size_t ch = (size_t)(2 * a.Hqk + a.Hv) * D;
            const size_t sqk = (size_t)a.Hqk * D, sv = (size_t)a.Hv * D;
            const IO *cin = static_cast<const IO *>(a.conv_in);
            IO *cout = static_cast<IO *>(a.conv_out) + (size_t)b * 3 * ch;
            for (int u = tid; u < 3 * 3 * G; u += C::NT) {
                const int part = u / (3 * G), j = (u / G) % 3, i0 = 4 * (u % G);  // part 0: v, 1: q, 2: k
                if (part > 0 && !qk_too) continue;
                const int tj = a.T - 3 + j;
                const size_t c0 = part == 0 ? 2 * sqk + (size_t)h * D + i0 : (part == 2 ? sqk : 0) + (size_t)hq * D + i0;
                f32x4 x{0.f, 0.f, 0.f, 0.f};
                if (tj >= 0) {
                    const IO *src = part == 0 ? vg + ((size_t)b * a.T + tj) * sv + (size_t)h * D + i0
                                              : (part == 1 ? qg : kg) + ((size_t)b * a.T + tj) * sqk + (size_t)hq * D + i0;
                    x = load4f(src);
                } else if (cin) {
                    x = load4f(cin + ((size_t)b * 3 + 3 + tj) * ch + c0);
                }
                store4f(cout + (size_t)j * ch + c0, x);
            }
        }
    }
}

template <typename IO, int D, int CW, bool CHAN>
static hipError_t launch_rec_t(const RecurArgs &a, hipStream_t s) {
    using C = RecurCfg<D, CW, CHAN>;
    const unsigned grid = (unsigned)a.B * (unsigned)a.Hv * (unsigned)C::TILES;
    if (a.conv_w)
        hipLaunchKernelGGL((recurrent_kernel<IO, D, CW, CHAN, true>), dim3(grid), dim3(C::NT), 0, s, a);
    else
        hipLaunchKernelGGL((recurrent_kernel<IO, D, CW, CHAN, false>), dim3(grid), dim3(C::NT), 0, s, a);
    return hipGetLastError();
}

template <typename IO, int D>
static hipError_t launch_rec_d(const RecurArgs &a, hipStream_t s) {
    const bool chan = a.decay == DECAY_CHANNEL;
    // 32 value columns per wave fill the device once there are about four
    // waves per SIMD; with fewer heads, 16 columns per wave double the waves.
    const bool narrow = D >= 64 && (long long)a.B * a.Hv * (D / 32) < 4096;
    if constexpr (D >= 64) {
        if (narrow) return chan ? launch_rec_t<IO, D, 16, true>(a, s) : launch_rec_t<IO, D, 16, false>(a, s);
    }
    return chan ? launch_rec_t<IO, D, 32, true>(a, s) : launch_rec_t<IO, D, 32, false>(a, s);
}

hipError_t launch_recurrent(int io, int D, const RecurArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_rec_d<bf16_t, 32>(a, s);
        if (D == 64) return launch_rec_d<bf16_t, 64>(a, s);
        if (D == 128) return launch_rec_d<bf16_t, 128>(a, s);
    } else {
        if (D == 32) return launch_rec_d<float, 32>(a, s);
        if (D == 64) return launch_rec_d<float, 64>(a, s);
        if (D == 128) return launch_rec_d<float, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
