// Block-scaled NVFP4 x NVFP4 GEMM on gfx950 matrix cores.
//
// What is computed ("minimax_h3_nvfp4_decoder" page, nvfp4_linear_inference: the
// mm_fp4 call with alpha = 1/(global_sf_x*global_sf_w), output in the activation
// dtype, then the bias add):
//   out[i, j] = bf16( alpha * sum_b sx[i,b] sw[j,b] sum_{k in b} qx[i,k] qw[j,k] ),
//   then out = bf16(out + bias[j]).
//
// Why f16 MFMA.  The scale is a non-power-of-two E4M3 per 16 K values.  gfx950's
// scaled FP4/FP8 MFMA applies one power-of-two (E8M0) scale per 32 K values, and an
// FP8 operand cannot hold e2m1*e4m3 exactly (up to 6 significant bits).  Every
// e2m1*e4m3 product is exact in fp16, so both operands are expanded to fp16 in
// registers, straight from the packed codes staged in LDS, and multiplied on the
// f16 MFMA with fp32 accumulation: no precision is lost before the accumulator.
//
// Scaling trick.  An E4M3 byte b shifted left by 7 is, read as an fp16, exactly
// value(b) * 2^-8 for every b (normal and subnormal), so a scale costs one shift.
// Operands then carry 2^-8 each; the accumulator is multiplied back by 2^16
// (exact) before alpha.
//
// Tiling.  256 x 128 output tile per 256-thread workgroup, K tiles of 128 (one
// scale-layout tile: 64 code bytes + 8 scale bytes per row), double-buffered in LDS
// with 80-byte row records (conflict-free 16-byte reads).  Four waves in a 2 x 2
// grid each own 128 x 64 of the output as 4 x 2 tiles of v_mfma_f32_32x32x16_f16.
// A lane of an MFMA tile takes row (lane % 32) and the K half (lane / 32) of the
// 128-wide tile, i.e. 32 contiguous code bytes; the same K assignment on both
// operands keeps the dot products intact.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.h"
#include "nvfp4_launch.h"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int WM = 128, WN = 64;
constexpr int TM = WM / 32, TN = WN / 32;
constexpr int kRowBytes = 80;
constexpr int kStageBytes = (BM + BN) * kRowBytes;

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// fp16 pair (s*2^-8, s*2^-8) for scale byte `sel` of a packed 4-byte scale word.
__device__ __forceinline__ half2_t scale_pair(uint32_t w, int sel) {
  const uint32_t b = (w >> (8 * sel)) & 0xFFu;
  return as_half2((b << 7) | (b << 23));
}

// 8 E2M1 codes (one 32-bit word) -> 8 fp16 values times the block scale.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, half2_t sc) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sc;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sc;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sc;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sc;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Global -> register staging of one K tile of one operand panel.
template <int ROWS>
struct Stage {
  static constexpr int kCodeLoads = ROWS / 64;     // 16-byte chunks per thread
  uint4 codes[kCodeLoads];
  uint2 scale;                                     // this thread's row (thread < ROWS)

  __device__ __forceinline__ void load(const uint8_t* __restrict__ cp, const uint8_t* __restrict__ sp, int64_t rows,
                                       int64_t row0, int64_t half_k, int64_t kt, bool aligned16) {
    const int t = threadIdx.x;
    const int64_t kb = kt * 64 + (t & 3) * 16;
#pragma unroll
    for (int i = 0; i < kCodeLoads; ++i) {
      const int64_t r = row0 + (t >> 2) + 64 * i;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < rows && kb < half_k) {
        const uint8_t* p = cp + r * half_k + kb;
        if (aligned16 && kb + 16 <= half_k) {
          v = *reinterpret_cast<const uint4*>(p);
        } else {
          const uint2 lo = *reinterpret_cast<const uint2*>(p);
          v.x = lo.x; v.y = lo.y;
          if (kb + 16 <= half_k) {
            const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
            v.z = hi.x; v.w = hi.y;
          }
        }
      }
      codes[i] = v;
    }
    scale = make_uint2(0, 0);
    if (t < ROWS) {
      const int64_t r = row0 + t;
      if (r < rows) scale = *reinterpret_cast<const uint2*>(sp + (kt * rows + r) * 8);
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kCodeLoads; ++i)
      *reinterpret_cast<uint4*>(lds + ((t >> 2) + 64 * i) * kRowBytes + (t & 3) * 16) = codes[i];
    if (t < ROWS) *reinterpret_cast<uint2*>(lds + t * kRowBytes + 64) = scale;
  }
};

__global__ void __launch_bounds__(kThreads, 2) gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m, int64_t k,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int64_t n,
    const float* __restrict__ gsf_a, const float* __restrict__ gsf_b, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, int tiles_m, int tiles_n, int aligned16) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run
  // of tiles, M fastest, so the blocks sharing a weight panel share an L2.
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid % tiles_m;
  const int tn = bid / tiles_m;
  const int64_t row0 = (int64_t)tm * BM;
  const int64_t col0 = (int64_t)tn * BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31;        // row within an MFMA tile
  const int kh = lane >> 5;        // K half of the 128-wide tile

  const int64_t half_k = k / 2;
  const int64_t kt_count = (k + BK - 1) / BK;

  float16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Stage<BM> sa;
  Stage<BN> sb;
  sa.load(a_codes, a_scales, m, row0, half_k, 0, aligned16);
  sb.load(b_codes, b_scales, n, col0, half_k, 0, aligned16);
  sa.store(lds);
  sb.store(lds + BM * kRowBytes);
  __syncthreads();

  for (int64_t kt = 0; kt < kt_count; ++kt) {
    const int cur = (int)(kt & 1);
    const bool more = kt + 1 < kt_count;
    if (more) {
      sa.load(a_codes, a_scales, m, row0, half_k, kt + 1, aligned16);
      sb.load(b_codes, b_scales, n, col0, half_k, kt + 1, aligned16);
    }
    const uint8_t* la = lds + cur * kStageBytes;
    const uint8_t* lb = la + BM * kRowBytes;

    uint32_t asc[TM], bsc[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      asc[i] = *reinterpret_cast<const uint32_t*>(la + (wm * WM + i * 32 + lr) * kRowBytes + 64 + 4 * kh);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bsc[j] = *reinterpret_cast<const uint32_t*>(lb + (wn * WN + j * 32 + lr) * kRowBytes + 64 + 4 * kh);

#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 araw[TM], braw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        araw[i] = *reinterpret_cast<const uint4*>(la + (wm * WM + i * 32 + lr) * kRowBytes + 32 * kh + 16 * q);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        braw[j] = *reinterpret_cast<const uint4*>(lb + (wn * WN + j * 32 + lr) * kRowBytes + 32 * kh + 16 * q);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8_t af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const uint32_t w = s == 0 ? araw[i].x : s == 1 ? araw[i].y : s == 2 ? araw[i].z : araw[i].w;
          af[i] = dequant8(w, scale_pair(asc[i], 2 * q + (s >> 1)));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const uint32_t w = s == 0 ? braw[j].x : s == 1 ? braw[j].y : s == 2 ? braw[j].z : braw[j].w;
          bf[j] = dequant8(w, scale_pair(bsc[j], 2 * q + (s >> 1)));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }

    if (more) {
      uint8_t* nxt = lds + (cur ^ 1) * kStageBytes;
      sa.store(nxt);
      sb.store(nxt + BM * kRowBytes);
    }
    __syncthreads();
  }

  // Epilogue: y = bf16(alpha * acc), then bf16(y + bias).
  const float alpha = __fdiv_rn(1.0f, __fmul_rn(*gsf_a, *gsf_b));
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = col0 + wn * WN + j * 32 + lr;
    if (col >= n) continue;
    const float bv = bias != nullptr ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = row0 + wm * WM + i * 32 + 8 * (e >> 2) + 4 * kh + (e & 3);
        if (row < m) {
          const float y = __fmul_rn(alpha, __fmul_rn(acc[i][j][e], 65536.0f));
          uint32_t yb = f32_to_bf16(y);
          if (bias != nullptr) yb = f32_to_bf16(__fadd_rn(bf16_to_f32(yb), bv));
          out[row * n + col] = (uint16_t)yb;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t n,
                       const float* gsf_a, const float* gsf_b, const uint16_t* bias, uint16_t* out, hipStream_t s) {
  const int tiles_m = (int)((m + BM - 1) / BM);
  const int tiles_n = (int)((n + BN - 1) / BN);
  const int aligned16 = ((k / 2) % 16 == 0) && (((uintptr_t)a_codes | (uintptr_t)b_codes) % 16 == 0);
  hipLaunchKernelGGL(gemm_kernel, dim3(tiles_m * tiles_n), dim3(kThreads), 0, s, a_codes, a_scales, m, k, b_codes,
                     b_scales, n, gsf_a, gsf_b, bias, out, tiles_m, tiles_n, aligned16);
  return hipGetLastError();
}

}  // namespace nvfp4
