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
// A workgroup owns (sequence, V head, segment, VT = 64 value columns; 32 at
// d = 32); its 4 waves each take one 16-token block of the chunk for A and
// O, and a quarter of the 16 x 16 tiles of its d x VT state, which stays in
// matrix-core accumulators in fp32 for the whole segment. All products run on the
// matrix cores: bf16 io on v_mfma_f32_16x16x32_bf16 (the state is rounded
// to bf16 as an operand of Q S, A to bf16 as an operand of A V; the
// normaliser is formed in fp32), fp32 io on v_mfma_f32_16x16x4_f32. The
// chunk's rows stay token-major in shared memory; the products that
// contract over tokens (K^T V, A V) read them with the LDS transpose read.
// The next chunk's rows are fetched into registers while the current one
// is computed.
//
// The decode step (one token per sequence) is a streaming kernel of its
// own, nla_decode: one workgroup per (sequence, V head) reads the state
// once, adds phi(k) v^T, reduces phi(q)^T S over the key axis and writes the
// state back; HBM-bound.
#include "common.hpp"
#include "kernels.hpp"
#include "norm_la.hpp"

namespace gdr {
namespace {

constexpr int C = 64;     // tokens per chunk
template <int D>
constexpr int vtile() { return D >= 64 ? 64 : 32; }  // value columns per workgroup
constexpr int NTH = 256;  // threads per workgroup

// Operands read K-major from token-major shared memory: element (row r, k)
// at M[k * ld + r]. For bfloat16, gfx950's LDS transpose read
// ds_read_b64_tr_b16: inside each group of 16 lanes, lane s supplies the
// address of 4 consecutive 16-bit elements and lane j receives element j % 4
// of the words of lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4, so lane s
// pointing at rows 4 (s % 4) .. + 3 of K-row k0 + s / 4 hands lane j row j
// of K-rows k0 .. k0 + 3 (the same reading as the chunked prefill's).
template <typename IO> struct KmRead;
template <> struct KmRead<bf16_t> {
    __device__ __forceinline__ static u16x8 frag(const bf16_t *M, int ld) {
        const int l = lane_id(), s = l & 15, g = l >> 4;
        const bf16_t *p = M + (8 * g + (s >> 2)) * ld + 4 * (s & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p + 4 * ld));
        return __builtin_bit_cast(u16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};
template <> struct KmRead<float> {
    __device__ __forceinline__ static float frag(const float *M, int ld) {
        const int l = lane_id();
        return M[(l >> 4) * ld + (l & 15)];
    }
};

// Shared-memory tiles (element type IO unless noted), token-major, rows
// padded by 16 bytes: Q, K [C][LQ] (phi(q), phi(k)); V [C][LV] (this
// workgroup's VT value columns); A [C][LT]; S [VT][LQ] (the state entering
// the chunk, transposed); z [2][D] fp32 (double-buffered); den [C] fp32.
// The output of a 16-token block is staged in its own rows of A. The
// segment-sum pass uses K and V only.
template <typename IO, int D>
struct NlaCfg {
    static constexpr int E = 16 / (int)sizeof(IO);  // elements per 16-byte access
    static constexpr int VT = vtile<D>(), NCT = VT / 16;  // value columns; their 16-column tiles
    static constexpr int NSW = D * VT / 1024;            // state tiles per wave (4 waves)
    static constexpr int LQ = D + E, LV = VT + E, LT = C + E;
    static constexpr size_t OK = 0, OV = OK + (size_t)C * LQ * sizeof(IO), OZ = OV + (size_t)C * LV * sizeof(IO),
                            OQ = OZ + 2 * (size_t)D * 4, OA = OQ + (size_t)C * LQ * sizeof(IO),
                            OS = OA + (size_t)C * LT * sizeof(IO), ODEN = OS + (size_t)VT * LQ * sizeof(IO),
                            BYTES0 = OQ, BYTES1 = ODEN + (size_t)C * 4;
    static constexpr int LO = VT + E;  // staged output row (io elements)
    static_assert(LO <= LT, "a block's output fits its rows of A");
    static constexpr int GR = D / E, NLD = C * GR / NTH;   // 16-byte pieces of a q or k row; per thread
    static constexpr int GV = VT / E, NLV = C * GV / NTH;  // of a v row's tile; per thread
    static_assert(C * GR % NTH == 0 && C * GV % NTH == 0 && NLV >= 1, "load mapping");
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

// One chunk's rows in registers: phi(q), phi(k) (16-byte pieces) and v's tile.
template <typename IO, int D, bool WITH_Q>
struct ChunkRegs {
    using Cf = NlaCfg<IO, D>;
    static constexpr int VT = Cf::VT;
    uint4 q[WITH_Q ? Cf::NLD : 1], k[Cf::NLD], v[Cf::NLV];
    __device__ __forceinline__ void load(const NlaArgs &a, int b, int hq, int h, int t0, int n, int col0) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < Cf::NLD; ++i) {
            const int idx = i * NTH + tid, t = idx / Cf::GR, g = (idx - t * Cf::GR) * Cf::E;
            const size_t row = (((size_t)b * a.T + t0 + t) * a.Hqk + hq) * D + g;
            k[i] = t < n ? *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.k) + row) : uint4{0u, 0u, 0u, 0u};
            if constexpr (WITH_Q)
                q[i] = t < n ? *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.q) + row) : uint4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < Cf::NLV; ++i) {
            const int idx = i * NTH + tid, t = idx / Cf::GV, g = (idx - t * Cf::GV) * Cf::E;
            v[i] = t < n ? *reinterpret_cast<const uint4 *>(static_cast<const IO *>(a.v) +
                                                            (((size_t)b * a.T + t0 + t) * a.Hv + h) * D + col0 + g)
                         : uint4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(IO *sQ, IO *sK, IO *sV) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < Cf::NLD; ++i) {
            const int idx = i * NTH + tid, t = idx / Cf::GR, g = (idx - t * Cf::GR) * Cf::E;
            *reinterpret_cast<uint4 *>(sK + t * Cf::LQ + g) = k[i];
            if constexpr (WITH_Q) *reinterpret_cast<uint4 *>(sQ + t * Cf::LQ + g) = q[i];
        }
#pragma unroll
        for (int i = 0; i < Cf::NLV; ++i) {
            const int idx = i * NTH + tid, t = idx / Cf::GV, g = (idx - t * Cf::GV) * Cf::E;
            *reinterpret_cast<uint4 *>(sV + t * Cf::LV + g) = v[i];
        }
    }
};

// MODE 0: per-segment sums K^T V and colsum(K) into the workspace.
// MODE 1: the sweep: outputs, and the final state from the last segment.
template <typename IO, int D, int MODE>
__global__ __launch_bounds__(NTH) void nla_chunks(NlaArgs a) {
    using M = Mma<IO>;
    using Cf = NlaCfg<IO, D>;
    constexpr int LQ = Cf::LQ, LV = Cf::LV, LT = Cf::LT, KS = M::KS, VT = Cf::VT, NCT = Cf::NCT, NVT = D / VT,
                  NSW = Cf::NSW;
    extern __shared__ __align__(16) unsigned char smem[];
    IO *sK = reinterpret_cast<IO *>(smem + Cf::OK), *sV = reinterpret_cast<IO *>(smem + Cf::OV);
    float *sZ = reinterpret_cast<float *>(smem + Cf::OZ);
    IO *sQ = reinterpret_cast<IO *>(smem + Cf::OQ), *sA = reinterpret_cast<IO *>(smem + Cf::OA);
    IO *sS = reinterpret_cast<IO *>(smem + Cf::OS);
    float *sDen = reinterpret_cast<float *>(smem + Cf::ODEN);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
    // Work items in the order value tile, V head of the QK group, segment,
    // (sequence, QK head), so that the items sharing one QK head's rows are
    // consecutive; the grid is a multiple of 8 and consecutive items go to
    // the same XCD (workgroups are dealt to the 8 XCDs in turn), whose L2
    // then serves those rows to all of them.
    const int grp = a.Hv / a.Hqk;
    const int x = blockIdx.x, wi = (x & 7) * (int)(gridDim.x >> 3) + (x >> 3);
    if (wi >= a.B * a.Hv * a.P * NVT) return;
    int id = wi;
    const int vt = id % NVT;
    id /= NVT;
    const int hg = id % grp;
    id /= grp;
    const int seg = id % a.P, bq = id / a.P, b = bq / a.Hqk, hq = bq - b * a.Hqk, h = hq * grp + hg;
    const int bh = b * a.Hv + h;
    if (MODE == 0 && seg == a.P - 1) return;  // the last segment's sum is not needed
    const int c0 = seg * a.L, c1 = min(a.NC, c0 + a.L), col0 = vt * VT;
    const size_t slab = (size_t)D * D + D;
    float *wseg = a.ws ? a.ws + ((size_t)bh * a.P + seg) * slab : nullptr;

    // This wave's state tiles: tile i is rows 16 * dt.., columns 16 * ct.. of
    // the D x VT tile, (dt, ct) = ((w NSW + i) / NCT, (w NSW + i) % NCT).
    f32x4 Sacc[NSW];
    const float *Sst = MODE == 1 ? (a.P > 1 ? wseg : a.S0 ? a.S0 + (size_t)bh * D * D : nullptr) : nullptr;
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
        const int dt = (w * NSW + i) / NCT, ct = (w * NSW + i) % NCT;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Sacc[i][r] = Sst ? Sst[(size_t)(dt * 16 + 4 * lg + r) * D + col0 + ct * 16 + lr] : 0.f;
    }
    if (tid < D) {
        const float *zst = MODE == 1 ? (a.P > 1 ? wseg + (size_t)D * D : a.z0 ? a.z0 + (size_t)bh * D : nullptr) : nullptr;
        sZ[tid] = zst ? zst[tid] : 0.f;
    }
    int zb = 0;  // the z buffer holding z entering the chunk

    ChunkRegs<IO, D, MODE == 1> rg;
    if (c0 < c1) rg.load(a, b, hq, h, c0 * C, min(C, a.T - c0 * C), col0);
    for (int c = c0; c < c1; ++c) {
        const int t0 = c * C, n = min(C, a.T - t0);
        if constexpr (MODE == 1)  // S entering the chunk, transposed, as the operand of Q S
#pragma unroll
            for (int i = 0; i < NSW; ++i) {
                const int dt = (w * NSW + i) / NCT, ct = (w * NSW + i) % NCT;
                put4<IO>(sS + (ct * 16 + lr) * LQ + dt * 16 + 4 * lg, Sacc[i]);
            }
        rg.store(sQ, sK, sV);
        if (c + 1 < c1) rg.load(a, b, hq, h, t0 + C, min(C, a.T - t0 - C), col0);  // in flight meanwhile
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
            // O rows of block w: (Q S + A V) / den, NCT 16-column tiles.
            f32x4 num[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < D; ks += KS) acc = M::step(acc, sQ + 16 * w * LQ + ks, LQ, sS + ct * 16 * LQ + ks, LQ);
#pragma unroll
                for (int ks = 0; ks < C; ks += KS)
                    acc = M::mma(acc, M::load(sA + 16 * w * LT + ks, LT), KmRead<IO>::frag(sV + ks * LV + ct * 16, LV));
                num[ct] = acc;
            }
            wave_sync();  // this block's rows of A are read: they take its output
            IO *stage = sA + 16 * w * LT;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 4 * lg + r;
                    stage[tr * Cf::LO + ct * 16 + lr] = Elem<IO>::to(num[ct][r] / sDen[16 * w + tr]);
                }
            wave_sync();
            constexpr int E = Cf::E, GO = VT / E, NST = (16 * GO + 63) / 64;
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const int idx = i * 64 + l, tr = idx / GO, g = (idx - tr * GO) * E, tt = 16 * w + tr;
                if (idx < 16 * GO && tt < n)
                    *reinterpret_cast<uint4 *>(static_cast<IO *>(a.o) + (((size_t)b * a.T + t0 + tt) * a.Hv + h) * D +
                                               col0 + g) = *reinterpret_cast<const uint4 *>(stage + tr * Cf::LO + g);
            }
        }
        // S += K^T V on this wave's state tiles; z += colsum(K) into the other buffer.
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int dt = (w * NSW + i) / NCT, ct = (w * NSW + i) % NCT;
#pragma unroll
            for (int ks = 0; ks < C; ks += KS)
                Sacc[i] = M::mma(Sacc[i], KmRead<IO>::frag(sK + ks * LQ + dt * 16, LQ),
                                 KmRead<IO>::frag(sV + ks * LV + ct * 16, LV));
        }
        if (tid < D) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
            for (int t = 0; t < C; t += 2) {
                s0 += Elem<IO>::load(sK + t * LQ + tid);
                s1 += Elem<IO>::load(sK + (t + 1) * LQ + tid);
            }
            sZ[(zb ^ 1) * D + tid] = sZ[zb * D + tid] + (s0 + s1);
        }
        zb ^= 1;
        __syncthreads();  // the tiles, S^T and z are read before the next chunk overwrites them
    }

    // The segment's sum (MODE 0) or, from the last segment, the final state.
    float *Sdst = MODE == 0 ? wseg : seg == a.P - 1 ? a.ST + (size_t)bh * D * D : nullptr;
    if (Sdst) {
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
            const int dt = (w * NSW + i) / NCT, ct = (w * NSW + i) % NCT;
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
    float x[32];  // the segments' sums (P <= 32), read before any is overwritten
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = s < a.P - 1 ? p[(size_t)s * slab] : 0.f;
#pragma unroll
    for (int s = 0; s < 32; ++s)
        if (s < a.P) {
            p[(size_t)s * slab] = acc;
            acc += x[s];
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

// The decode step: one workgroup per (sequence, V head). Thread (rg, cg)
// holds rows RPT rg .. of the state's column group cg (4 columns), read and
// written once with streaming accesses; q, k, v of the token and z in
// shared memory. num_c = sum_i q_i (S_ic + k_i v_c), den = q . (z + k).
template <typename IO, int D>
__global__ __launch_bounds__(NTH) void nla_decode(NlaArgs a) {
    constexpr int CG = D / 4, RG = NTH / CG, RPT = D / RG;
    static_assert(RG * RPT == D && RPT >= 1, "decode mapping");
    __shared__ float sq[D], sk[D], sv[D], sz[D], spart[RG][D + 4], sden;
    const int tid = threadIdx.x, cg = tid % CG, rgi = tid / CG;
    const int bh = blockIdx.x, b = bh / a.Hv, h = bh - b * a.Hv, hq = h / (a.Hv / a.Hqk);
    float *S = a.ST + (size_t)bh * D * D;
    f32x4 st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = load_state4(S + (size_t)(rgi * RPT + m) * D + 4 * cg);
    if (tid < D) {
        sq[tid] = Elem<IO>::load(static_cast<const IO *>(a.q) + ((size_t)b * a.Hqk + hq) * D + tid);
        sk[tid] = Elem<IO>::load(static_cast<const IO *>(a.k) + ((size_t)b * a.Hqk + hq) * D + tid);
        sv[tid] = Elem<IO>::load(static_cast<const IO *>(a.v) + ((size_t)b * a.Hv + h) * D + tid);
        sz[tid] = a.z0[(size_t)bh * D + tid];
    }
    __syncthreads();
    if (tid < 64) {  // den = q . (z + k), one wave
        float x = 0.f;
        for (int i = tid; i < D; i += 64) x += sq[i] * (sz[i] + sk[i]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
        if (tid == 0) sden = x;
    }
    const f32x4 vc = load4f(sv + 4 * cg);
    f32x4 part = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rgi * RPT + m;
        st[m] += sk[i] * vc;
        part += sq[i] * st[m];
        store_state4(S + (size_t)i * D + 4 * cg, st[m]);
    }
    store4f(&spart[rgi][4 * cg], part);
    __syncthreads();
    if (tid < D) {
        float num = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) num += spart[r][tid];
        static_cast<IO *>(a.o)[((size_t)b * a.Hv + h) * D + tid] = Elem<IO>::to(num / sden);
        a.zT[(size_t)bh * D + tid] = sz[tid] + sk[tid];
    }
}

template <typename IO, int D>
hipError_t launch_t(const NlaArgs &a, bool decode, hipStream_t s) {
    using Cf = NlaCfg<IO, D>;
    static const hipError_t attr_err = [] {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&nla_chunks<IO, D, 0>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::BYTES0);
        if (e == hipSuccess)
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(&nla_chunks<IO, D, 1>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)Cf::BYTES1);
        return e;
    }();
    if (attr_err != hipSuccess) return attr_err;
    if (decode) {
        if ((long long)a.B * a.Hv > 0x7fffffffll) return hipErrorInvalidValue;
        if (a.B * a.Hv > 0) hipLaunchKernelGGL((nla_decode<IO, D>), dim3((unsigned)(a.B * a.Hv)), dim3(NTH), 0, s, a);
        return hipGetLastError();
    }
    const long long items = (long long)a.B * a.Hv * a.P * (D / Cf::VT);
    if (items <= 0) return hipSuccess;
    if (items > 0x7ffffff0ll) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((items + 7) / 8 * 8);
    if (a.P > 1) {
        hipLaunchKernelGGL((nla_chunks<IO, D, 0>), dim3(grid), dim3(NTH), Cf::BYTES0, s, a);
        const unsigned gx = (unsigned)(((size_t)D * D + D + NTH - 1) / NTH);
        hipLaunchKernelGGL((nla_scan<D>), dim3(gx, (unsigned)(a.B * a.Hv)), dim3(NTH), 0, s, a);
    }
    hipLaunchKernelGGL((nla_chunks<IO, D, 1>), dim3(grid), dim3(NTH), Cf::BYTES1, s, a);
    if (a.z_apart) {
        const size_t nz = (size_t)a.B * a.Hv * D;
        hipLaunchKernelGGL((nla_zsum<IO, D>), dim3((unsigned)((nz + NTH - 1) / NTH)), dim3(NTH), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nla(int io, int D, const NlaArgs &a, bool decode, hipStream_t s) {
    if (io == IO_BF16) {
        if (D == 32) return launch_t<bf16_t, 32>(a, decode, s);
        if (D == 64) return launch_t<bf16_t, 64>(a, decode, s);
        if (D == 128) return launch_t<bf16_t, 128>(a, decode, s);
    } else {
        if (D == 32) return launch_t<float, 32>(a, decode, s);
        if (D == 64) return launch_t<float, 64>(a, decode, s);
        if (D == 128) return launch_t<float, 128>(a, decode, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr
