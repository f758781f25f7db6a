// Device-side building blocks shared by the codec kernels (gfx950 / CDNA4).
//
// * storage conversions (OCP FP8 e4m3fn, bf16, fp16), written from the formats'
//   definitions;
// * MFMA "k-step" traits: one 16x16 output tile consumes 32 K values per step; each
//   lane supplies 8 consecutive K values of one A row and of one B column. The
//   16x16 result is held as 4 floats per lane: row 4*(lane/16) + i, column lane%16.
//   bf16 and fp16 use one v_mfma_f32_16x16x32 per step; fp32 uses eight
//   v_mfma_f32_16x16x4_f32, lane element u standing for K index 8*(lane/16) + u in
//   both operands (a consistent permutation of K leaves the product unchanged);
// * LDS staging of K chunks with conversion to the compute type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// LDS reads in kernels that also have global->LDS direct loads in flight go through
// these native vector types: a read through HIP's struct vector types (uint2, int4,
// float4, ...) makes the compiler wait for every outstanding direct load first.
template <typename V>
__device__ inline V lds_load(const void* p) {
    return *reinterpret_cast<const V*>(p);
}

// storage tag for OCP FP8 e4m3fn bytes
struct fp8_t {
    uint8_t b;
};

enum : int {
    DEVERR_EMPTY_POOL = 1,
    DEVERR_POS_RANGE = 2,
    DEVERR_REF_CAPACITY = 4,
    DEVERR_IDX_RANGE = 8,
    DEVERR_ROW_RANGE = 16,
};

__device__ inline void flag_error(int* err, int bits) {
    if (err) atomicOr(err, bits);
}

// ------------------------------------------------------------------ FP8 e4m3fn
// value = (-1)^s * 2^(e-7) * (1 + m/8) for e >= 1, (-1)^s * m * 2^-9 for e = 0.
__device__ inline float fp8_to_f32(uint32_t byte) {
    const uint32_t em = byte & 0x7Fu;
    const float mag = (em >= 8u) ? __uint_as_float((em << 20) + (120u << 23))
                                 : (float)em * 0.001953125f;
    return (byte & 0x80u) ? -mag : mag;
}

// Round to nearest, ties to even code; saturate to +-448; keep the sign bit.
__device__ inline uint32_t f32_to_fp8(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {  // |x| >= 448 (also inf / nan): largest finite code
        code = 0x7Eu;
    } else if (a >= 0x3C800000u) {  // |x| >= 2^-6: normal, keep 3 mantissa bits (RNE)
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - (120u << 3);
        if (code > 0x7Eu) code = 0x7Eu;
    } else {  // subnormal: m = rint(|x| * 2^9), m = 8 is the smallest normal code
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    }
    return sign | code;
}

// ------------------------------------------------------------------ generic loads
// Load 8 consecutive elements of a storage type and widen them to float.
template <typename S>
struct Load8;

template <>
struct Load8<float> {
    static __device__ inline void run(const float* p, float* o) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

template <>
struct Load8<bf16_t> {
    static __device__ inline void run(const bf16_t* p, float* o) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = __uint_as_float(w[i] << 16);
            o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};

// Hardware OCP e4m3fn widening (v_cvt_pk_f32_fp8: two bytes of a word per call); it
// agrees with fp8_to_f32 on all 256 codes.
__device__ inline float4 fp8x4_to_f32(uint32_t w) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    return make_float4(lo[0], lo[1], hi[0], hi[1]);
}

// Eight FP8 values (two words) widened exactly to bf16
__device__ inline bf16x8 widen8(uint32_t x, uint32_t y) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)y, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)y, 1.0f, true);
    bf16x8 f;
    f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
    f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
    return f;
}

template <>
struct Load8<fp8_t> {
    static __device__ inline void run(const fp8_t* p, float* o) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        const float4 a = fp8x4_to_f32(v.x), b = fp8x4_to_f32(v.y);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

// Load 4 consecutive elements and widen to float.
template <typename S>
struct Load4;
template <>
struct Load4<float> {
    static __device__ inline float4 run(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <>
struct Load4<fp8_t> {
    static __device__ inline float4 run(const fp8_t* p) { return fp8x4_to_f32(*reinterpret_cast<const uint32_t*>(p)); }
};
template <>
struct Load4<bf16_t> {
    static __device__ inline float4 run(const bf16_t* p) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
    }
};

// ------------------------------------------------------------------ MFMA traits
template <typename T>
struct Mma;

template <>
struct Mma<bf16_t> {
    typedef bf16x8 frag;
    static __device__ inline f32x4 step(f32x4 acc, const frag& a, const frag& b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    static __device__ inline frag from_float(const float* v) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (bf16_t)v[i];
        return f;
    }
};

template <>
struct Mma<f16_t> {
    typedef f16x8 frag;
    static __device__ inline f32x4 step(f32x4 acc, const frag& a, const frag& b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
    }
    static __device__ inline frag from_float(const float* v) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (f16_t)v[i];
        return f;
    }
};

template <>
struct Mma<float> {
    typedef f32x8 frag;
    static __device__ inline f32x4 step(f32x4 acc, const frag& a, const frag& b) {
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], acc, 0, 0, 0);
        return acc;
    }
    static __device__ inline frag from_float(const float* v) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = v[i];
        return f;
    }
};

// LDS row pitch (elements) for a K chunk of KC: 16 bytes of padding per row keeps
// the 16-byte fragment reads of 8 consecutive rows on distinct banks.
template <typename T, int KC>
struct Pitch {
    static constexpr int value = KC + 16 / (int)sizeof(T);
};

template <typename T>
__device__ inline typename Mma<T>::frag lds_frag(const T* p) {
    return *reinterpret_cast<const typename Mma<T>::frag*>(p);
}

// Convert 8 floats to the compute type and store them to LDS (16 or 32 bytes).
template <typename T>
__device__ inline void lds_store8(T* dst, const float* v) {
    *reinterpret_cast<typename Mma<T>::frag*>(dst) = Mma<T>::from_float(v);
}

__device__ inline f32x4 zero4() {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return z;
}

// s / k correctly rounded for the reference-mean sums: s is a sum of at most 8 FP8
// e4m3fn values (a multiple of 2^-9, |s| <= 8 * 448) and k = 1..8. With rk = RN(1/k),
// q = s rk and one FMA correction of the residual, q + (s - q k) rk (Markstein's
// correction step for division on FMA hardware), give the IEEE quotient for every such
// s and k: checked exhaustively against the correctly rounded division, all 2^22 sums
// x 8 k (tests/support/exact_div_check.c).
__device__ inline float div_small(float s, float k, float rk) {
    const float q = s * rk;
    const float e = fmaf(-q, k, s);
    return fmaf(e, rk, q);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

}  // namespace rkv
