// Device-side helpers shared by the CSA2 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// Storage dtype codes (same values as the C ABI's csa2_dtype).
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2, DT_FP4 = 3, DT_MXFP4 = 4 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Same rounding (to nearest even) with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// ---------------------------------------------------------------- e4m3
// OCP e4m3fn -> bf16 is exact (3 mantissa bits, exponents 2^-9 .. 2^8 all
// fit bf16).  gfx950 converts two codes per instruction; the scale operand
// is 1.0 so nothing is rounded.

__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t codes, bool hi_word) {
    bf16x2 r = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 e4m3 codes (two dwords) -> 8 bf16 (four dwords).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 c) {
    u32x4 r;
    r[0] = e4m3x2_to_bf16x2(c[0], false);
    r[1] = e4m3x2_to_bf16x2(c[0], true);
    r[2] = e4m3x2_to_bf16x2(c[1], false);
    r[3] = e4m3x2_to_bf16x2(c[1], true);
    return r;
}

// ---------------------------------------------------------------- fp4
// Eight E2M1 codes (one dword; element 2j in the low nibble of byte j) times
// a scale -> eight bf16.  Exact: a level (at most 2 significant bits) times
// an E4M3 or power-of-two scale (at most 4) fits bf16's 8.  gfx950's
// conversion applies only the exponent of its scale operand, so the levels
// are converted with scale 1 and the scale multiplies in float32.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t codes, float scale) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    u32x4 r;
    r[0] = cvt_bf16x2(a[0] * scale, a[1] * scale);
    r[1] = cvt_bf16x2(b[0] * scale, b[1] * scale);
    r[2] = cvt_bf16x2(c[0] * scale, c[1] * scale);
    r[3] = cvt_bf16x2(d[0] * scale, d[1] * scale);
    return r;
}

// E8M0 block scale (OCP microscaling) -> float: 2^(code - 127); 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
    code &= 0xFFu;
    if (code == 0xFFu) return __uint_as_float(0x7FC00000u);
    return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);
}

__device__ __forceinline__ float e4m3_to_f32(uint8_t code) {
    uint32_t two = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(
                                                    static_cast<uint32_t>(code), 1.0f, false));
    return __uint_as_float((two & 0xFFFFu) << 16);
}

// Element of a row in any storage dtype, as float (row-wise scale applied
// by the caller).
__device__ __forceinline__ float load_elem(const void* base, size_t i, int dt) {
    if (dt == DT_F32) return static_cast<const float*>(base)[i];
    if (dt == DT_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
    return e4m3_to_f32(static_cast<const uint8_t*>(base)[i]);
}

__device__ __forceinline__ int dt_bytes(int dt) { return dt == DT_F32 ? 4 : (dt == DT_BF16 ? 2 : 1); }

// ---------------------------------------------------------------- rotary
// cos/sin of the rotary angle t * base^(-2j/r): the angle is formed and
// reduced modulo 2*pi in double precision (t reaches 2^20), the reduced
// angle goes through single-precision sincos.
__device__ __forceinline__ double rope_inv_freq(int j, int rd, float base) {
    return pow(static_cast<double>(base), -2.0 * j / rd);
}

__device__ __forceinline__ void rope_cos_sin(int64_t t, double inv, float& c, float& s) {
    const double th = static_cast<double>(t) * inv;
    const double k = rint(th * 0.15915494309189533577);       // 1 / (2 pi)
    double r = fma(-k, 6.283185307179586232, th);              // 2 pi, high part
    r = fma(-k, 2.4492935982947064e-16, r);                    // 2 pi, low part
    sincosf(static_cast<float>(r), &s, &c);
}

__device__ __forceinline__ void rope_angle(int64_t t, int j, int rd, float base, float& c, float& s) {
    rope_cos_sin(t, rope_inv_freq(j, rd, base), c, s);
}

// ---------------------------------------------------------------- ordering
// Order-preserving float -> uint32 (larger float, larger key).  -inf and NaN
// become 0, which marks "never selectable".

__device__ __forceinline__ uint32_t score_key(float f) {
    if (!(f > -__builtin_huge_valf())) return 0u;  // -inf or NaN
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 -> f32 (gfx950).  Operand layout, lane l = 0..63:
//   A[i][k]: i = l % 16, k in group l / 16 (8 values)
//   B[k][j]: j = l % 16, k in group l / 16 (8 values)
//   C[i][j]: j = l % 16, i = 4 * (l / 16) + v, v = 0..3
// Any assignment of the 32 k values to (group, element) works as long as A
// and B use the same one; the kernels pick it to make loads contiguous.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 -> f32 (gfx950).  Operand layout, lane l = 0..63:
//   A[i][k]: i = l % 32, k in group l / 32 (8 values)
//   B[k][j]: j = l % 32, k in group l / 32 (8 values)
//   C[i][j]: j = l % 32, i = 8 * (v / 4) + 4 * (l / 32) + v % 4, v = 0..15
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------- shuffles

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// x of this lane and x of lane l ^ 16 (resp. l ^ 32), in either order.
// gfx950's v_permlane16_swap exchanges the odd 16-lane rows of its first
// operand with the even rows of its second (v_permlane32_swap: the upper
// half with the lower half); with x in both operands each lane ends up
// holding both values of its pair, in one VALU op and no LDS traffic.
__device__ __forceinline__ void pair_xor16(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void pair_xor32(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48
// max(x, 0) as one signed-integer max of the bits: a negative float has the
// sign bit set, so it compares below 0 (fmaxf on a matrix-unit result costs
// an extra canonicalising max)
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float max4_rows(float x) {
    float a, b;
    pair_xor16(x, a, b);
    x = fmaxf(a, b);
    pair_xor32(x, a, b);
    return fmaxf(a, b);
}

__device__ __forceinline__ float sum4_rows(float x) {
    float a, b;
    pair_xor16(x, a, b);
    x = a + b;
    pair_xor32(x, a, b);
    return a + b;
}

__device__ __forceinline__ float warp_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
    return v;
}

__device__ __forceinline__ float warp_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += shfl_xor_f(v, o);
    return v;
}

__device__ __forceinline__ int warp_sum_i(int v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace csa2
