// Device helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16 and, for
// fp32 inputs, eight v_mfma_f32_32x32x2_f32 covering the same 16-deep slice):
//   A operand (32 x 16): lane l supplies row  m = l % 32, k = 8*(l/32) .. +7
//   B operand (16 x 32): lane l supplies col  n = l % 32, k = 8*(l/32) .. +7
//   C/D (32 x 32, 16 fp32 per lane): lane l holds column n = l % 32 and rows
//       m = 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
// A 16-deep slice can use any fixed assignment of its 16 k-indices to the two
// half-waves as long as A and B agree, which is what lets the fp32 path reuse
// the bf16 operand layout (8 consecutive elements per lane).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef uint16_t bf16_t;
typedef uint8_t fp8_t;   // OCP fp8 e4m3 bits (the variant without infinities)
// Two OCP fp4 e2m1 values in one byte: element 2c in bits 0-3 of byte c,
// element 2c + 1 in bits 4-7 (sign, two exponent bits with bias 1, one
// mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}).
struct fp4x2_t {
    uint8_t bits;
};
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 128;   // Bk: tokens per key block
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<bf16_t>((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const float2v x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// Eight consecutive elements of one matrix-core operand row/column.
template <typename T> struct Op8;
template <> struct Op8<bf16_t> {
    bf16x8 v;
    __device__ __forceinline__ void load(const void* p) {
        v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
    }
    __device__ __forceinline__ void zero() { v = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }
};
template <> struct Op8<float> {
    float v[8];
    __device__ __forceinline__ void load(const void* p) {
        const float4* q = reinterpret_cast<const float4*>(p);
        float4 a = q[0], b = q[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
};

// acc(32x32) += A(32x16) * B(16x32) for one 16-deep slice.
__device__ __forceinline__ void mma16(floatx16& acc, const Op8<bf16_t>& a, const Op8<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(floatx16& acc, const Op8<float>& a, const Op8<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

// Value held by lane l ^ 32 (the other half-wave). v_permlane32_swap applied
// to (x, x) leaves every lane with lane (l % 32)'s x in the first result and
// lane (l % 32 + 32)'s x in the second, so the other half's value is the
// second result in the lower half and the first in the upper half.
__device__ __forceinline__ float swap_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
}

// max of two scores with IEEE 754-2019 "maximum" semantics (NaN propagates;
// +0 above -0): gfx950 has it as v_maximum3_f32, which needs none of the
// operand canonicalisation fmaxf's IEEE-mode lowering adds for values that
// come straight from the matrix cores. Identical to fmaxf on the finite
// scores used here (+0 and -0 compare equal in every later comparison).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// For a pair of per-half partial values a (row set A) and b (row set B), one
// v_permlane32_swap leaves lane l < 32 with a[l] and a[l + 32] and lane
// l >= 32 with b[l - 32] and b[l]: their max is the full value of row set A in
// the lower half-wave and of row set B in the upper one, with no select.
__device__ __forceinline__ float pair_max_own(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 2^x on the transcendental unit (v_exp_f32), without the library's rescaling
// of arguments below -126: such results may come out as 0 instead of a
// denormal. Every use here is a softmax term 2^(z - max) <= 1 summed with a
// term equal to 1 (or weighted by one), so a lost term below 2^-126 changes no
// result beyond fp32 rounding.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max3f(float a, float b, float c) { return vmax(a, vmax(b, c)); }

__device__ __forceinline__ float max16(const floatx16& a) {
    const float m0 = max3f(a[0], a[1], a[2]);
    const float m1 = max3f(a[3], a[4], a[5]);
    const float m2 = max3f(a[6], a[7], a[8]);
    const float m3 = max3f(a[9], a[10], a[11]);
    const float m4 = max3f(a[12], a[13], a[14]);
    return max3f(max3f(m0, m1, m2), max3f(m3, m4, a[15]), m0);
}

}  // namespace msa
