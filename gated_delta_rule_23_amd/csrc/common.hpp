// common.hpp -- device helpers shared by the libgdr kernels (gfx950 only).
//
// Element types: bfloat16 is stored as uint16_t bit patterns; float32 as float.
// Matrix-core tiles use the 16x16 output shape of gfx950's MFMA:
//   bf16: v_mfma_f32_16x16x32_bf16  (K step 32; each lane feeds 8 bf16 of A and of B)
//   f32:  v_mfma_f32_16x16x4_f32    (K step 4;  each lane feeds 1 float of A and of B)
// Operand convention used everywhere: A is a 16 x K block of a row-major
// matrix (K contiguous), and B is given as B^T, i.e. also 16 x K with K
// contiguous. Lane l supplies row (l % 16) of each and K-slice (l / 16).
// The 16x16 fp32 result: lane l holds rows 4*(l/16) + r, r = 0..3, of
// column (l % 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) unsigned short u16x8;
typedef __attribute__((ext_vector_type(4))) unsigned short u16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

typedef uint16_t bf16_t;

// Compute units of the device in use when first asked (thread-safe; 256 if unknown).
inline int device_cus() {
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            return n;
        return 256;
    }();
    return cus;
}

__device__ __forceinline__ float bf2f(bf16_t u) { return __uint_as_float((uint32_t)u << 16); }

// float -> bfloat16, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    __device__ __forceinline__ static float to(float x) { return x; }
    __device__ __forceinline__ static float from(float x) { return x; }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p) { return bf2f(*p); }
    __device__ __forceinline__ static bf16_t to(float x) { return f2bf(x); }
    __device__ __forceinline__ static float from(bf16_t x) { return bf2f(x); }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// 16x16 tile products on the matrix cores.
//   load(M, ld): this lane's fragment of the 16 x KS block at M (row stride
//                ld elements): row (l % 16), K-slice (l / 16).
//   mma(acc, a, b): acc += A_block * (Bt_block)^T for fragments a of A and
//                b of Bt (B given transposed, K contiguous).
//   step(acc, A, lda, Bt, ldb): load both fragments and multiply.
template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KS = 32;
    using Frag = u16x8;
    __device__ __forceinline__ static Frag load(const bf16_t *M, int ld) {
        const int l = lane_id();
        return *reinterpret_cast<const u16x8 *>(M + (l & 15) * ld + (l >> 4) * 8);
    }
    __device__ __forceinline__ static f32x4 mma(f32x4 acc, Frag a, Frag b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 step(f32x4 acc, const bf16_t *A, int lda, const bf16_t *Bt, int ldb) {
        return mma(acc, load(A, lda), load(Bt, ldb));
    }
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    using Frag = float;
    __device__ __forceinline__ static Frag load(const float *M, int ld) {
        const int l = lane_id();
        return M[(l & 15) * ld + (l >> 4)];
    }
    __device__ __forceinline__ static f32x4 mma(f32x4 acc, Frag a, Frag b) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 step(f32x4 acc, const float *A, int lda, const float *Bt, int ldb) {
        return mma(acc, load(A, lda), load(Bt, ldb));
    }
};

// acc += A[16 x 16] * (Bt[16 x 16])^T: bf16 on v_mfma_f32_16x16x16_bf16 (lane l
// feeds 4 elements: row l % 16, K-slice 4*(l/16)); fp32 as four K=4 steps.
typedef __attribute__((ext_vector_type(4))) short s16x4;
template <typename T> struct Mma16;
template <> struct Mma16<bf16_t> {
    __device__ __forceinline__ static f32x4 step(f32x4 acc, const bf16_t *A, int lda, const bf16_t *Bt, int ldb) {
        const int l = lane_id();
        const s16x4 a = *reinterpret_cast<const s16x4 *>(A + (l & 15) * lda + (l >> 4) * 4);
        const s16x4 b = *reinterpret_cast<const s16x4 *>(Bt + (l & 15) * ldb + (l >> 4) * 4);
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
};
template <> struct Mma16<float> {
    __device__ __forceinline__ static f32x4 step(f32x4 acc, const float *A, int lda, const float *Bt, int ldb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = Mma<float>::step(acc, A + 4 * ks, lda, Bt + 4 * ks, ldb);
        return acc;
    }
};

// Input-stage activations on the hardware's base-2 exp and log (v_exp_f32,
// v_log_f32, about 1 ulp each), written from the definitions:
//   sigmoid(x)  = 1 / (1 + e^-x)
//   softplus(x) = max(x, 0) + ln(1 + e^-|x|)   (no overflow for any x)
__device__ __forceinline__ float act_sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
__device__ __forceinline__ float act_softplus(float x) {
    return fmaxf(x, 0.f) +
           0.6931471805599453f * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(x)));
}

// Sum over NL (4, 8 or 16) consecutive lanes, aligned to NL, result in every
// one of them, by DPP row permutations: swap neighbours, swap pairs, then
// fold each 8-lane half onto its mirror image, and for 16 lanes the two
// halves of the row likewise (each step adds a disjoint partial sum).
template <int NL>
__device__ __forceinline__ float lanes_allreduce(float x) {
    static_assert(NL == 4 || NL == 8 || NL == 16, "DPP row groups");
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    if constexpr (NL >= 8)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
    if constexpr (NL == 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row mirror
    return x;
}

// Four consecutive elements (8 or 16 bytes, aligned) widened to float, and back.
__device__ __forceinline__ f32x4 load4f(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4f(const bf16_t *p) {
    u16x4 u = *reinterpret_cast<const u16x4 *>(p);
    return f32x4{bf2f(u[0]), bf2f(u[1]), bf2f(u[2]), bf2f(u[3])};
}
__device__ __forceinline__ void store4f(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }

// Four consecutive fp32 state entries (16-byte aligned) read or written with a
// non-temporal hint: state blocks are streamed once per call and not reused
// before they would be evicted, so they are kept from displacing other data in
// the caches (MI355X's memory-side cache included).
__device__ __forceinline__ f32x4 load_state4(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void store_state4(float *p, f32x4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store4f(bf16_t *p, f32x4 x) {
    *reinterpret_cast<uint2 *>(p) = uint2{f2bf2(x[0], x[1]), f2bf2(x[2], x[3])};
}

// Four consecutive stored elements kept raw in registers (no conversion at
// load time, so a prefetch does not wait for its data), widened at use.
template <typename T> struct Raw4;
template <> struct Raw4<float> {
    using type = f32x4;
    __device__ __forceinline__ static type load(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
    __device__ __forceinline__ static f32x4 widen(type r) { return r; }
};
template <> struct Raw4<bf16_t> {
    using type = u16x4;
    __device__ __forceinline__ static type load(const bf16_t *p) { return *reinterpret_cast<const u16x4 *>(p); }
    __device__ __forceinline__ static f32x4 widen(type u) { return f32x4{bf2f(u[0]), bf2f(u[1]), bf2f(u[2]), bf2f(u[3])}; }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdr
