// Device-side number formats and small helpers shared by the gfx950 kernels.
//
// Formats follow the NVFP4 description on the pages (cited by title):
// "minimax_h3_nvfp4_decoder" (NVFP4DecoderLinear._activation_global_sf: global
// scale FP4_E4M3_RANGE / amax; from_packed: two FP4 codes per byte) and
// "FastH3-QAD-v2 and NVFP4 VAE Decoders", section "The whole stack in NVFP4"
// (4-bit values plus one FP8 scale per 16).  FP4 is read as E2M1, the FP8 scale
// as E4M3 (bias 7, finite max 448), FP4_E4M3_RANGE as 6 * 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kRange = 2688.0f;         // 6 * 448
constexpr float kAmaxFloor = 1e-12f;      // amax.clamp(min=1e-12)
constexpr int kBlock = 16;                // K values per E4M3 scale
constexpr int kScaleTileK = 128;          // K values per scale-layout tile (8 scale bytes per row)

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Non-negative finite fp32 -> E4M3 byte, nearest even, saturating at 448 (0x7E).
// Below 2^-6 the E4M3 grid is uniform with step 2^-9, so the code is rint(x * 512)
// (x * 512 is exact); above it the fp32 significand is rounded to 3 bits and the
// exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  if (x >= 448.0f) return 0x7Eu;
  if (x < 0.015625f) return (uint32_t)__builtin_rintf(fminf(x, 0.015625f) * 512.0f);
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  return (u >> 20) - (120u << 3);
}

// E4M3 byte (0x00..0x7E) -> fp32, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t e = b >> 3, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// 16 consecutive bf16 values (32 bytes, 16-byte aligned) -> fp32.
__device__ __forceinline__ void load16_bf16(const uint16_t* __restrict__ p, float (&v)[16]) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const uint4 b = reinterpret_cast<const uint4*>(p)[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// SwiGLU product feeding down_proj: bf16(fp32(fp32(g / fp32(1 + exp(-g))) * u)).  exp is
// evaluated in fp32 step by step: clamp to [-80, 80], t = n*ln2 + r by Cody-Waite
// reduction (ln2 = 15-bit head + tail, so n*head is exact), e^r by a degree-6 Taylor
// polynomial in Horner form, then the exact scaling by 2^n.  Each step is one IEEE
// fp32 operation (explicit intrinsics: no contraction), which fixes the result bit for
// bit; it is within 3 ulps of exp.
__device__ __forceinline__ float exp_cw(float t) {
  t = fminf(fmaxf(t, -80.0f), 80.0f);
  const float n = __builtin_rintf(__fmul_rn(t, 0x1.715476p+0f));
  const float r = __fsub_rn(__fsub_rn(t, __fmul_rn(n, 0x1.62e4p-1f)), __fmul_rn(n, 0x1.7f7d1cp-20f));
  float p = 0x1.6c16c2p-10f;                       // 1/720
  p = __fadd_rn(__fmul_rn(p, r), 0x1.111112p-7f);  // 1/120
  p = __fadd_rn(__fmul_rn(p, r), 0x1.555556p-5f);  // 1/24
  p = __fadd_rn(__fmul_rn(p, r), 0x1.555556p-3f);  // 1/6
  p = __fadd_rn(__fmul_rn(p, r), 0.5f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float swiglu_bf16(float g, float u) {
  const float d = __fadd_rn(1.0f, exp_cw(-g));
  return bf16_to_f32(f32_to_bf16(__fmul_rn(__fdiv_rn(g, d), u)));
}

// E2M1 nibble -> fp32, exact: magnitudes 0, .5, 1, 1.5 for codes 0-3, then
// 2^(e-1) * (1 + m/2) for codes 4-7 (e = code >> 1, m = code & 1); bit 3 is the sign.
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const uint32_t mag = c & 7u;
  const float a = mag < 4u ? 0.5f * (float)mag : __uint_as_float(((126u + (mag >> 1)) << 23) | ((mag & 1u) << 22));
  return (c & 8u) ? -a : a;
}

// fp32 -> E2M1 nibble, nearest even, saturating at 6; the sign bit of v is kept.
// Below 1 the grid is uniform (step 0.5), so the magnitude code is rint(2|v|);
// from 1 up, the fp32 significand is rounded to one bit and the exponent rebiased
// (1.0 -> code 2).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ua = u & 0x7FFFFFFFu;
  const float a = __uint_as_float(ua);
  const uint32_t small = (uint32_t)__builtin_rintf(fminf(a, 1.0f) * 2.0f);
  uint32_t big = ((ua + 0x1FFFFFu + ((ua >> 22) & 1u)) >> 22) - 252u;
  big = big > 7u ? 7u : big;
  const uint32_t mag = a < 1.0f ? small : big;
  return mag | ((u >> 28) & 8u);
}

// Eight fp32 values -> eight E2M1 nibbles (value i in bits 4i..4i+3) with the
// hardware conversion at unit scale, which rounds to nearest even, saturates at 6
// and keeps the sign exactly like e2m1_encode (checked exhaustively against it on
// gfx950 around every rounding boundary, for signed zeros, subnormals and
// out-of-range values).
__device__ __forceinline__ uint32_t e2m1_encode8(const float* v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// Per-16-block quantization, the order every kernel uses:
//   sf = (gsf * bmax) / 6; s8 = E4M3(sf); s = decode(s8); r = gsf / s; code = E2M1(v * r).
__device__ __forceinline__ uint32_t block_scale_byte(float gsf, float bmax) {
  const float sf = __fdiv_rn(__fmul_rn(gsf, bmax), 6.0f);
  return e4m3_encode(sf);
}

// One 16-block under global scale gsf: its E4M3 scale byte and its 16 codes (two
// words, value i in bits 4(i%8).. of word i/8).  All codes are 0 when the scale is 0.
__device__ __forceinline__ uint32_t quantize_block16(const float (&v)[16], float gsf, bool valid, uint32_t& w0,
                                                     uint32_t& w1) {
  float bmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(v[i]));
  const uint32_t s8 = valid ? block_scale_byte(gsf, bmax) : 0u;
  w0 = 0;
  w1 = 0;
  if (s8 != 0) {
    const float r = __fdiv_rn(gsf, e4m3_decode(s8));
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __fmul_rn(v[i], r);
    w0 = e2m1_encode8(p);
    w1 = e2m1_encode8(p + 8);
  }
  return s8;
}

__device__ __forceinline__ float global_scale_from_amax(float amax) {
  return __fdiv_rn(kRange, amax > kAmaxFloor ? amax : kAmaxFloor);
}

// In-register Walsh-Hadamard butterflies on 16 consecutive values, strides 1..min(g,16)/2.
__device__ __forceinline__ void fwht16_local(float (&v)[16], int g) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
    if (h < g) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if ((i & h) == 0) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
      }
    }
  }
}

// Butterfly stages with strides 16, 32, 64 across the lanes that hold consecutive
// 16-value chunks of one group (lane ^ 1, ^ 2, ^ 4).  Every lane of the wave must
// execute this (shuffles).
__device__ __forceinline__ void fwht16_cross(float (&v)[16], int g) {
#pragma unroll
  for (int hl = 1; hl < 8; hl <<= 1) {
    if (16 * hl < g) {
      const bool upper = (threadIdx.x & hl) != 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __shfl_xor(v[i], hl, 64);
        v[i] = upper ? p - v[i] : v[i] + p;
      }
    }
  }
}

// Rotation of one 16-value chunk (the lane's part of a group of g <= 128), then the
// rounding to bf16 the activation path applies; returns the bf16 values as fp32.
__device__ __forceinline__ void rotate16_bf16(float (&v)[16], int g, float inv_sqrt_g) {
  fwht16_local(v, g);
  fwht16_cross(v, g);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(f32_to_bf16(__fmul_rn(v[i], inv_sqrt_g)));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

}  // namespace nvfp4
