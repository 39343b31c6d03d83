// norm_la.hip -- normalised linear attention: the feature-mapped read with a
// normaliser (page "Linear attention e fast weights", section "Conceito").
// Per (sequence b, V head h), with phi applied by the caller,
//   S_t = S_{t-1} + phi(k_t) v_t^T   (d x d),   z_t = z_{t-1} + phi(k_t),
//   o_t = S_t^T phi(q_t) / (z_t^T phi(q_t)),
// the sums running over i <= t. V head h reads QK head h / (Hv / Hqk).
//
// Chunked form, C = 64 tokens: with S and z entering the chunk, Q, K the
// chunk's phi(q), phi(k) rows and V its values,
//   A = tril(Q K^T)  (the token's own key included),
//   O = (Q S + A V) / (Q z + rowsum(A)),   S += K^T V,   z += colsum(K).
// The state is a plain sum, so the sequence also splits into P segments run
// side by side: a first pass forms each segment's sum K^T V and colsum(K)
// (nla_chunks<MODE 0>), nla_scan turns them into the state entering each
// segment (S0 and z0 folded in), and the sweep (nla_chunks<MODE 1>) walks
// each segment's chunks from its start state. Short sequences (or many
// heads) run one segment and skip the first two launches.
//
// A workgroup owns (sequence, V head, segment, 32 value columns); its 4
// waves each take one 16-token block of the chunk for A and O, and D / 32
// of the 16 x 16 tiles of its d x 32 state, which stays in matrix-core
// accumulators in fp32 for the whole segment. All products run on the
// matrix cores: bf16 io on v_mfma_f32_16x16x32_bf16 (the state is rounded
// to bf16 as an operand of Q S, A to bf16 as an operand of A V; the
// normaliser is formed in fp32), fp32 io on v_mfma_f32_16x16x4_f32.
#include "common.hpp"
#include "kernels.hpp"
#include "norm_la.hpp"

namespace gdr {
namespace {

constexpr int C = 64;     // tokens per chunk
constexpr int VT = 32;    // value columns per workgroup
constexpr int NTH = 256;  // threads per workgroup

// Shared-memory tiles (element type IO unless noted), rows padded by 16 bytes:
//   Q, K [C][LQ] token-major (phi(q), phi(k));  Kt [D][LT], Vt [VT][LT]
//   channel-major (token axis contiguous); A [C][LT]; S [VT][LQ] (the state
//   entering the chunk, transposed); z [2][D] fp32 (double-buffered); den
//   [C] fp32. The output of a 16-token block is staged in its own rows of A.
template <typename IO, int D>
struct NlaCfg {
    static constexpr int E = 16 / (int)sizeof(IO);  // elements per 16-byte access
    static constexpr int LQ = D + E, LT = C + E;
    static constexpr size_t OQ = 0, OK = OQ + (size_t)C * LQ * sizeof(IO), OKT = OK + (size_t)C * LQ * sizeof(IO),
                            OVT = OKT + (size_t)D * LT * sizeof(IO), OA = OVT + (size_t)VT * LT * sizeof(IO),
                            OS = OA + (size_t)C * LT * sizeof(IO), OZ = OS + (size_t)VT * LQ * sizeof(IO),
                            ODEN = OZ + 2 * (size_t)D * 4, BYTES = ODEN + (size_t)C * 4;
    static constexpr int LO = VT + 4;  // staged output row (floats)
    static_assert((size_t)16 * LO * 4 <= (size_t)16 * LT * sizeof(IO), "a block's output fits its rows of A");
};

template <typename IO>
__device__ __forceinline__ void put4(IO *p, f32x4 x);
template <>
__device__ __forceinline__ void put4<float>(float *p, f32x4 x) { store4f(p, x); }
template <>
__device__ __forceinline__ void put4<bf16_t>(bf16_t *p, f32x4 x) { store4f(p, x); }

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// MODE 0: per-segment sums K^T V and colsum(K) into the workspace.
// MODE 1: the sweep: outputs, and the final state from the last segment.
template <typename IO, int D, int MODE>
__global__ __launch_bounds__(NTH) void nla_chunks(NlaArgs a) {
    using M = Mma<IO>;
    using Cf = NlaCfg<IO, D>;
    constexpr int E = Cf::E, LQ = Cf::LQ, LT = Cf::LT, KS = M::KS, NVT = D / VT, NSW = D / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    IO *sQ = reinterpret_cast<IO *>(smem + Cf::OQ), *sK = reinterpret_cast<IO *>(smem + Cf::OK);
    IO *sKt = reinterpret_cast<IO *>(smem + Cf::OKT), *sVt = reinterpret_cast<IO *>(smem + Cf::OVT);
    IO *sA = reinterpret_cast<IO *>(smem + Cf::OA), *sS = reinterpret_cast<IO *>(smem + Cf::OS);
    float *sZ = reinterpret_cast<float *>(smem + Cf::OZ), *sDen = reinterpret_cast<float *>(smem + Cf::ODEN);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    int id = blockIdx.x;
    const int vt = id % NVT;
    id /= NVT;
    const int seg = id % a.P, bh = id / a.P, b = bh / a.Hv, h = bh - b * a.Hv, hq = h / (a.Hv / a.Hqk);
    if (MODE == 0 && seg == a.P - 1) return;  // the last segment's sum is not needed
    const int c0 = seg * a.L, c1 = min(a.NC, c0 + a.L), col0 = vt * VT;
    const size_t slab = (size_t)D * D + D;
    float *wseg = a.ws ? a.ws + ((size_t)bh * a.P + seg) * slab : nullptr;

    // This wave's state tiles: tile i is rows 16 * dt.., columns 16 * ct.. of
    // the D x VT tile, (dt, ct) = ((w NSW + i) / 2, (w NSW + i) % 2).
    f32x4 Sacc[NSW];
    const float *Sst = MODE == 1 ? (a.P > 1 ? wseg : a.S0 ? a.S0 + (size_t)bh * D * D : nullptr) : nullptr;
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
        const int dt = (w * NSW + i) >> 1, ct = (w * NSW + i) & 1;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sacc[i][r] = Sst ? Sst[(size_t)(dt * 16 + 4 * lg + r) * D + col0 + ct * 16 + lr] : 0.f;
    }
    if (tid < D) {
        const float *zst = MODE == 1 ? (a.P > 1 ? wseg + (size_t)D * D : a.z0 ? a.z0 + (size_t)bh * D : nullptr) : nullptr;
        sZ[tid] = zst ? zst[tid] : 0.f;
    }
    int zb = 0;  // the z buffer holding z entering the chunk

    for (int c = c0; c < c1; ++c) {
        const int t0 = c * C, n = min(C, a.T - t0);
        if constexpr (MODE == 1)  // S entering the chunk, transposed, as the operand of Q S
#pragma unroll
            for (int i = 0; i < NSW; ++i) {
                const int dt = (w * NSW + i) >> 1, ct = (w * NSW + i) & 1;
                put4<IO>(sS + (ct * 16 + lr) * LQ + dt * 16 + 4 * lg, Sacc[i]);
            }
        // Load the chunk: phi(q) and phi(k) rows (and k channel-major), v's tile channel-major.
        {
            constexpr int GR = D / E, NLD = C * GR / NTH;
            static_assert(C * GR % NTH == 0, "load mapping");
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int idx = i * NTH + tid, t = idx / GR, g = (idx - t * GR) * E;
                const size_t row = (((size_t)b * a.T + t0 + t) * a.Hqk + hq) * D + g;
                uint4 kr = uint4{0u, 0u, 0u, 0u}, qr = uint4{0u, 0u, 0u, 0u};
                if (t < n) {
                    kr = *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.k) + row);
                    if (MODE == 1) qr = *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.q) + row);
                }
                *reinterpret_cast<uint4 *>(sK + t * LQ + g) = kr;
                if (MODE == 1) *reinterpret_cast<uint4 *>(sQ + t * LQ + g) = qr;
                const IO *ke = reinterpret_cast<const IO *>(&kr);
#pragma unroll
                for (int e = 0; e < E; ++e) sKt[(g + e) * LT + t] = ke[e];
            }
            constexpr int GV = VT / E, NLV = (C * GV + NTH - 1) / NTH;
#pragma unroll
            for (int i = 0; i < NLV; ++i) {
                const int idx = i * NTH + tid, t = idx / GV, g = (idx - t * GV) * E;
                if (idx < C * GV) {
                    uint4 vr = uint4{0u, 0u, 0u, 0u};
                    if (t < n)
                        vr = *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.v) +
                                                              (((size_t)b * a.T + t0 + t) * a.Hv + h) * D + col0 + g);
                    const IO *ve = reinterpret_cast<const IO *>(&vr);
#pragma unroll
                    for (int e = 0; e < E; ++e) sVt[(g + e) * LT + t] = ve[e];
                }
            }
        }
        __syncthreads();

        if constexpr (MODE == 1) {
            // A^T tiles of this wave's token block w: rows j (block jt), column
            // t; A_tj = phi(q_t) . phi(k_j) for j <= t, else 0. The row sums
            // of A and phi(q_t) . z give the normaliser.
            const int t = 16 * w + lr;
            float rs = 0.f;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                f32x4 acc = zero4();
                if (jt <= w) {
#pragma unroll
                    for (int ks = 0; ks < D; ks += KS) acc = M::step(acc, sK + jt * 16 * LQ + ks, LQ, sQ + 16 * w * LQ + ks, LQ);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc[r] = 16 * jt + 4 * lg + r <= t ? acc[r] : 0.f;
                    rs += acc[r];
                }
                put4<IO>(sA + t * LT + 16 * jt + 4 * lg, acc);
            }
            float qz = 0.f;
            const float *z = sZ + zb * D;
#pragma unroll
            for (int d = lg * (D / 4); d < (lg + 1) * (D / 4); d += 4) {
                const f32x4 qv = load4f(sQ + t * LQ + d), zv = load4f(z + d);
                qz += qv[0] * zv[0] + qv[1] * zv[1] + qv[2] * zv[2] + qv[3] * zv[3];
            }
            float den = rs + qz;
            den += __shfl_xor(den, 16);
            den += __shfl_xor(den, 32);
            if (lg == 0) sDen[t] = den;
            wave_sync();
            // O rows of block w: (Q S + A V) / den, two 16-column tiles.
            f32x4 num[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < D; ks += KS) acc = M::step(acc, sQ + 16 * w * LQ + ks, LQ, sS + ct * 16 * LQ + ks, LQ);
#pragma unroll
                for (int ks = 0; ks < C; ks += KS) acc = M::step(acc, sA + 16 * w * LT + ks, LT, sVt + ct * 16 * LT + ks, LT);
                num[ct] = acc;
            }
            wave_sync();  // this block's rows of A are read: they take its output
            float *stage = reinterpret_cast<float *>(sA + 16 * w * LT);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 4 * lg + r;
                    stage[tr * Cf::LO + ct * 16 + lr] = num[ct][r] / sDen[16 * w + tr];
                }
            wave_sync();
            constexpr int GO = VT / E, NST = 16 * GO / 64;
#pragma unroll
            for (int i = 0; i < (NST > 0 ? NST : 1); ++i) {
                const int idx = i * 64 + l, tr = idx / GO, g = (idx - tr * GO) * E, tt = 16 * w + tr;
                if (idx < 16 * GO && tt < n) {
                    IO *dst = static_cast<IO *>(a.o) + (((size_t)b * a.T + t0 + tt) * a.Hv + h) * D + col0 + g;
                    const float *src = stage + tr * Cf::LO + g;
#pragma unroll
                    for (int e = 0; e < E; e += 4) put4<IO>(dst + e, load4f(src + e));
                }
            }
        }
        // S += K^T V on this wave's state tiles; z += colsum(K) into the other buffer.
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int dt = (w * NSW + i) >> 1, ct = (w * NSW + i) & 1;
#pragma unroll
            for (int ks = 0; ks < C; ks += KS) Sacc[i] = M::step(Sacc[i], sKt + dt * 16 * LT + ks, LT, sVt + ct * 16 * LT + ks, LT);
        }
        if (tid < D) {
            float s = sZ[zb * D + tid];
            for (int t = 0; t < C; t += 4) {
                const f32x4 kv = load4f(sKt + tid * LT + t);
                s += (kv[0] + kv[1]) + (kv[2] + kv[3]);
            }
            sZ[(zb ^ 1) * D + tid] = s;
        }
        zb ^= 1;
        __syncthreads();  // the tiles, S^T and z are read before the next chunk overwrites them
    }

    // The segment's sum (MODE 0) or, from the last segment, the final state.
    float *Sdst = MODE == 0 ? wseg : seg == a.P - 1 ? a.ST + (size_t)bh * D * D : nullptr;
    if (Sdst) {
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int dt = (w * NSW + i) >> 1, ct = (w * NSW + i) & 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) Sdst[(size_t)(dt * 16 + 4 * lg + r) * D + col0 + ct * 16 + lr] = Sacc[i][r];
        }
        if (vt == 0 && tid < D && (MODE == 0 || !a.z_apart)) {
            float *zdst = MODE == 0 ? wseg + (size_t)D * D : a.zT + (size_t)bh * D;
            zdst[tid] = sZ[zb * D + tid];
        }
    }
}

// The state entering each segment: an exclusive running sum of the
// segments' sums, starting from S0 and z0 (zeros when absent), in place.
template <int D>
__global__ __launch_bounds__(NTH) void nla_scan(NlaArgs a) {
    const size_t slab = (size_t)D * D + D;
    const size_t e = (size_t)blockIdx.x * NTH + threadIdx.x;
    const int bh = blockIdx.y;
    if (e >= slab) return;
    float acc = e < (size_t)D * D ? (a.S0 ? a.S0[(size_t)bh * D * D + e] : 0.f)
                                  : (a.z0 ? a.z0[(size_t)bh * D + (e - (size_t)D * D)] : 0.f);
    float *p = a.ws + (size_t)bh * a.P * slab + e;
    for (int s = 0; s < a.P; ++s) {
        const float x = s < a.P - 1 ? p[(size_t)s * slab] : 0.f;
        p[(size_t)s * slab] = acc;
        acc += x;
    }
}

// z_T = z0 + the sum of the call's phi(k) rows, one thread per (sequence, V
// head, channel): used when z_T is z0 itself with one segment, where the
// sweep's workgroups of a head would otherwise read z0 after another of them
// had written z_T.
template <typename IO, int D>
__global__ __launch_bounds__(NTH) void nla_zsum(NlaArgs a) {
    const size_t i = (size_t)blockIdx.x * NTH + threadIdx.x;
    if (i >= (size_t)a.B * a.Hv * D) return;
    const int d = (int)(i % D), bh = (int)(i / D), b = bh / a.Hv, hq = (bh % a.Hv) / (a.Hv / a.Hqk);
    const IO *k = static_cast<const IO *>(a.k) + ((size_t)b * a.T * a.Hqk + hq) * D + d;
    float s = 0.f;
    for (int t = 0; t < a.T; ++t) s += Elem<IO>::load(k + (size_t)t * a.Hqk * D);
    a.zT[i] = a.z0[i] + s;
}

template <typename IO, int D>
hipError_t launch_t(const NlaArgs &a, hipStream_t s) {
    using Cf = NlaCfg<IO, D>;
    const size_t smem = Cf::BYTES;
    static const hipError_t attr_err = [] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&nla_chunks<IO, D, 0>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::BYTES);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&nla_chunks<IO, D, 1>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::BYTES);
        return e;
    }();
    if (attr_err != hipSuccess) return attr_err;
    const long long items = (long long)a.B * a.Hv * a.P * (D / VT);
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffffll) return hipErrorInvalidValue;
    if (a.P > 1) {
        hipLaunchKernelGGL((nla_chunks<IO, D, 0>), dim3((unsigned)items), dim3(NTH), smem, s, a);
        const unsigned gx = (unsigned)(((size_t)D * D + D + NTH - 1) / NTH);
        hipLaunchKernelGGL((nla_scan<D>), dim3(gx, (unsigned)(a.B * a.Hv)), dim3(NTH), 0, s, a);
    }
    hipLaunchKernelGGL((nla_chunks<IO, D, 1>), dim3((unsigned)items), dim3(NTH), smem, s, a);
    if (a.z_apart) {
        const size_t nz = (size_t)a.B * a.Hv * D;
        hipLaunchKernelGGL((nla_zsum<IO, D>), dim3((unsigned)((nz + NTH - 1) / NTH)), dim3(NTH), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nla(int io, int D, const NlaArgs &a, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_t<bf16_t, 32>(a, s);
        if (D == 64) return launch_t<bf16_t, 64>(a, s);
        if (D == 128) return launch_t<bf16_t, 128>(a, s);
    } else {
        if (D == 32) return launch_t<float, 32>(a, s);
        if (D == 64) return launch_t<float, 64>(a, s);
        if (D == 128) return launch_t<float, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
