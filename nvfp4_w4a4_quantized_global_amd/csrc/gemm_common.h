// Operand expansion shared by the GEMM kernels: packed E2M1 codes and E4M3 block
// scales -> exact fp16 MFMA operands.
//
// Every e2m1 * e4m3 product has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16.  An E4M3 byte b shifted left by 7 and
// read as an fp16 is exactly value(b) * 2^-8 (normal and subnormal alike), so a
// block scale costs one shift; operands then carry 2^-8 each and the fp32
// accumulator is multiplied back by 2^16 (exact) before alpha.
// v_cvt_scalef32_pk_f16_fp4 applies only the exponent of its scale operand, so it
// runs at scale 1 and v_pk_mul_f16 applies the block scale.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.h"

namespace nvfp4 {
namespace gemm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BK = 128;                 // K values per tile = one scale-layout tile
constexpr float kAccUnscale = 65536.0f; // undoes the two 2^-8 operand factors

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// fp16 pair (s*2^-8, s*2^-8) for scale byte `sel` of a packed 4-byte scale word.
__device__ __forceinline__ half2_t scale_pair(uint32_t w, int sel) {
  const uint32_t b = (w >> (8 * sel)) & 0xFFu;
  return as_half2((b << 7) | (b << 23));
}

// 8 E2M1 codes (one 32-bit word, value i in bits 4i..4i+3) -> 8 fp16 values times the block scale.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, half2_t sc) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ uint32_t word(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// alpha = fp32(1 / fp32(gsf_a * gsf_b)).  With seg_rows > 0 the activation rows come in
// blocks of seg_rows rows with one global scale each, gsf_a[row / seg_rows].  Rows and
// seg_rows are below 2^31 (the C ABI rejects larger), so the division is a 32-bit one.
__device__ __forceinline__ uint32_t segment_of(int64_t row, int64_t seg_rows) {
  return (uint32_t)row / (uint32_t)seg_rows;
}
__device__ __forceinline__ float alpha_for(const float* gsf_a, const float* gsf_b, int64_t seg_rows, int64_t row) {
  const float ga = seg_rows > 0 ? gsf_a[segment_of(row, seg_rows)] : *gsf_a;
  return __fdiv_rn(1.0f, __fmul_rn(ga, *gsf_b));
}

// The 16 alphas of the rows 8*(e/4) + 4*kh + e%4 (e = 0..15) of a 32-row MFMA output
// group starting at row g0 (rows clamped to m - 1): one value when the group lies in
// one segment, the common case.
__device__ __forceinline__ void group_alphas(const float* gsf_a, const float* gsf_b, int64_t seg_rows, int64_t g0,
                                             int kh, int64_t m, float (&al)[16]) {
  const int64_t first = g0 < m - 1 ? g0 : m - 1;
  const int64_t last = g0 + 31 < m - 1 ? g0 + 31 : m - 1;
  if (seg_rows <= 0 || segment_of(first, seg_rows) == segment_of(last, seg_rows)) {
    const float a = alpha_for(gsf_a, gsf_b, seg_rows, first);
#pragma unroll
    for (int e = 0; e < 16; ++e) al[e] = a;
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t r = g0 + 8 * (e >> 2) + 4 * kh + (e & 3);
      al[e] = alpha_for(gsf_a, gsf_b, seg_rows, r < m - 1 ? r : m - 1);
    }
  }
}

// Two fp32 values -> two bf16, nearest even (v_cvt_pk_bf16_f32; the same bits as
// f32_to_bf16 for every finite value), a in the low half.
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, bf16x2_t));
}

// bf16(y) + bias in fp32, rounded to bf16: the bias add after the GEMM output is rounded.
__device__ __forceinline__ uint32_t add_bias_bf16(uint32_t y_bf16, uint16_t bias_bf16) {
  return f32_to_bf16(__fadd_rn(bf16_to_f32(y_bf16), bf16_to_f32(bias_bf16)));
}

}  // namespace gemm
}  // namespace nvfp4
