// Block-scaled NVFP4 x NVFP4 GEMM on gfx950 matrix cores: generic kernel for any
// shape, and the dispatcher that sends large problems to gemm_pipe.hip.
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
// registers (gemm_common.h), straight from the packed codes staged in LDS, and
// multiplied on the f16 MFMA with fp32 accumulation: nothing is rounded before the
// accumulator.
//
// Tiling.  A workgroup of WM x WN waves owns a (WM*TM*32) x (WN*TN*32) output tile;
// each wave owns TM x TN tiles of v_mfma_f32_32x32x16_f16.  K advances in tiles of
// 128 (one scale-layout tile: 64 code bytes + 8 scale bytes per row), in three LDS
// stages of 80-byte row records (conflict-free 16-byte reads).  A lane of an MFMA
// tile takes row (lane % 32) and K half (lane / 32) of the 128-wide tile, i.e. 32
// contiguous code bytes; both operands use the same K assignment, which keeps every
// dot product intact.  The epilogue goes through LDS so that each lane writes 16
// contiguous output bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int kRowBytes = 80;
constexpr int kStages = 3;
constexpr int kValuPerMfma = 4;

// Global -> register staging of one K tile of one operand panel of ROWS rows.
template <int ROWS, int THREADS>
struct Stage {
  static constexpr int kChunks = ROWS * 4 / THREADS;       // 16-byte code chunks per thread
  static constexpr int kScaleRows = (ROWS + THREADS - 1) / THREADS;
  static_assert(ROWS * 4 % THREADS == 0, "code chunks must divide evenly");
  uint4 codes[kChunks];
  uint2 scale[kScaleRows];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ cp, const uint8_t* __restrict__ sp, int64_t rows,
                                       int64_t srows, int64_t row0, int64_t half_k, int64_t kt, bool aligned16) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = t + i * THREADS;
      const int64_t r = row0 + (c >> 2);
      const int64_t kb = kt * 64 + (c & 3) * 16;
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
#pragma unroll
    for (int i = 0; i < kScaleRows; ++i) {
      const int rr = t + i * THREADS;
      const int64_t r = row0 + rr;
      scale[i] = make_uint2(0, 0);
      if (rr < ROWS && r < rows) scale[i] = *reinterpret_cast<const uint2*>(sp + (kt * srows + r) * 8);
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = t + i * THREADS;
      *reinterpret_cast<uint4*>(lds + (c >> 2) * kRowBytes + (c & 3) * 16) = codes[i];
    }
#pragma unroll
    for (int i = 0; i < kScaleRows; ++i) {
      const int rr = t + i * THREADS;
      if (rr < ROWS) *reinterpret_cast<uint2*>(lds + rr * kRowBytes + 64) = scale[i];
    }
  }
};

template <int WM, int WN, int TM, int TN>
struct Cfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int BM = WM * TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kLoopLds = kStages * kStageBytes;
  // epilogue: each wave stages 32 rows x (TN*32) bf16 at a time
  static constexpr int kEpiRowBytes = TN * 32 * 2 + 16;
  static constexpr int kEpiLds = WM * WN * 32 * kEpiRowBytes;
  static constexpr int kLds = kLoopLds > kEpiLds ? kLoopLds : kEpiLds;
};

template <int WM, int WN, int TM, int TN>
__global__ void __launch_bounds__(64 * WM * WN) gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m, int64_t k,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int64_t n,
    const float* __restrict__ gsf_a, const float* __restrict__ gsf_b, int64_t a_seg_rows,
    const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ out, int64_t b_srows, int64_t ldo, int tiles_m, int tiles_n, int aligned16) {
  using C = Cfg<WM, WN, TM, TN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run
  // of tiles, M fastest, so the blocks sharing a weight panel share an L2.
  const int nblk = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int tm = bid % tiles_m;
  const int tn = bid / tiles_m;
  const int64_t row0 = (int64_t)tm * C::BM;
  const int64_t col0 = (int64_t)tn * C::BN;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
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

  // Three LDS stages: while tile kt is multiplied out of stage kt%3, tile kt+1 (held in
  // registers since the previous iteration) is stored to stage (kt+1)%3 and tile kt+2
  // is fetched from global memory.  One barrier per tile.
  auto stage = [&](int64_t t) { return lds + (int)(t % kStages) * C::kStageBytes; };
  Stage<C::BM, C::kThreads> sa;
  Stage<C::BN, C::kThreads> sb;
  sa.load(a_codes, a_scales, m, m, row0, half_k, 0, aligned16);
  sb.load(b_codes, b_scales, n, b_srows, col0, half_k, 0, aligned16);
  sa.store(stage(0));
  sb.store(stage(0) + C::BM * kRowBytes);
  if (kt_count > 1) {
    sa.load(a_codes, a_scales, m, m, row0, half_k, 1, aligned16);
    sb.load(b_codes, b_scales, n, b_srows, col0, half_k, 1, aligned16);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < kt_count; ++kt) {
    if (kt + 1 < kt_count) {
      sa.store(stage(kt + 1));
      sb.store(stage(kt + 1) + C::BM * kRowBytes);
    }
    if (kt + 2 < kt_count) {
      sa.load(a_codes, a_scales, m, m, row0, half_k, kt + 2, aligned16);
      sb.load(b_codes, b_scales, n, b_srows, col0, half_k, kt + 2, aligned16);
    }
    const uint8_t* la = stage(kt) + (wm * TM * 32 + lr) * kRowBytes;
    const uint8_t* lb = stage(kt) + (C::BM + wn * TN * 32 + lr) * kRowBytes;

    uint32_t asc[TM], bsc[TN];
    uint4 araw[2][TM], braw[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) asc[i] = *reinterpret_cast<const uint32_t*>(la + i * 32 * kRowBytes + 64 + 4 * kh);
#pragma unroll
    for (int j = 0; j < TN; ++j) bsc[j] = *reinterpret_cast<const uint32_t*>(lb + j * 32 * kRowBytes + 64 + 4 * kh);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        araw[q][i] = *reinterpret_cast<const uint4*>(la + i * 32 * kRowBytes + 32 * kh + 16 * q);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        braw[q][j] = *reinterpret_cast<const uint4*>(lb + j * 32 * kRowBytes + 32 * kh + 16 * q);
    }

    // Sub-step t covers K values [64*kh + 8t, +8) of the tile on each lane.  The
    // fragments of sub-step t+1 are expanded while the MFMAs of sub-step t run.
    half8_t fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = dequant8(word(araw[0][i], 0), scale_pair(asc[i], 0));
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = dequant8(word(braw[0][j], 0), scale_pair(bsc[j], 0));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      half8_t na[TM], nb[TN];
      if (t < 7) {
        const int u = t + 1;
#pragma unroll
        for (int i = 0; i < TM; ++i) na[i] = dequant8(word(araw[u >> 2][i], u & 3), scale_pair(asc[i], u >> 1));
#pragma unroll
        for (int j = 0; j < TN; ++j) nb[j] = dequant8(word(braw[u >> 2][j], u & 3), scale_pair(bsc[j], u >> 1));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      if (t < 7) {
#pragma unroll
        for (int g = 0; g < TM * TN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // then a few VALU
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = na[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = nb[j];
      }
    }
    __syncthreads();
  }

  // Epilogue: y = bf16(alpha * acc) staged through LDS 32 rows at a time per wave,
  // then bf16(y + bias) written as 16-byte row segments.
  uint8_t* epi = lds + wave * 32 * C::kEpiRowBytes;
  constexpr int kSegs = TN * 32 / 8;                 // 16-byte segments per staged row
  const int64_t wrow0 = row0 + wm * TM * 32;
  const int64_t wcol0 = col0 + wn * TN * 32;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float al[16];
    group_alphas(gsf_a, gsf_b, a_seg_rows, wrow0 + i * 32, kh, m, al);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * kh + (e & 3);
        const float y = __fmul_rn(al[e], __fmul_rn(acc[i][j][e], kAccUnscale));
        *reinterpret_cast<uint16_t*>(epi + r * C::kEpiRowBytes + (j * 32 + lr) * 2) = (uint16_t)f32_to_bf16(y);
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 32 * kSegs / 64; ++p) {
      const int idx = p * 64 + lane;
      const int r = idx / kSegs, sg = idx % kSegs;
      const int64_t row = wrow0 + i * 32 + r;
      const int64_t col = wcol0 + sg * 8;
      const uint4 v = *reinterpret_cast<const uint4*>(epi + r * C::kEpiRowBytes + sg * 16);
      if (row < m && col < n) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if (bias != nullptr) {
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            if (col + h < n) {
              const uint32_t sh = 16 * (h & 1);
              const uint32_t zb = add_bias_bf16((w[h >> 1] >> sh) & 0xFFFFu, bias[col + h]);
              w[h >> 1] = (w[h >> 1] & (0xFFFF0000u >> sh)) | (zb << sh);
            }
          }
        }
        uint16_t* o = out + row * ldo + col;
        if (col + 8 <= n && ((uintptr_t)o & 15) == 0) {
          *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          for (int h = 0; h < 8 && col + h < n; ++h) o[h] = (uint16_t)((w[h >> 1] >> (16 * (h & 1))) & 0xFFFFu);
        }
      }
    }
    __syncthreads();
  }
}

template <int WM, int WN, int TM, int TN>
hipError_t launch_cfg(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k, const uint8_t* b_codes,
                      const uint8_t* b_scales, int64_t n, const float* gsf_a, const float* gsf_b, int64_t a_seg_rows,
                      const uint16_t* bias,
                      uint16_t* out, int64_t b_srows, int64_t ldo, int aligned16, hipStream_t s) {
  using C = Cfg<WM, WN, TM, TN>;
  static bool attr_set[kMaxDevices] = {};
  if (hipError_t e = set_dynamic_lds_once(reinterpret_cast<const void*>(&gemm_kernel<WM, WN, TM, TN>), C::kLds,
                                          attr_set);
      e != hipSuccess)
    return e;
  const int tiles_m = (int)((m + C::BM - 1) / C::BM);
  const int tiles_n = (int)((n + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_kernel<WM, WN, TM, TN>), dim3(tiles_m * tiles_n), dim3(C::kThreads), C::kLds, s, a_codes,
                     a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, b_srows, ldo, tiles_m,
                     tiles_n, aligned16);
  return hipGetLastError();
}

// Generic kernel over output columns [0, n) of a product whose B scale layout has
// b_srows rows per K tile and whose output rows are ldo elements apart.
hipError_t launch_generic(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                          const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                          int64_t b_srows, int64_t ldo, int cus, hipStream_t s) {
  const int aligned16 = ((k / 2) % 16 == 0) && (((uintptr_t)a_codes | (uintptr_t)b_codes) % 16 == 0);
  // Largest tile that still gives every compute unit a tile.
  const int64_t mid = ((m + 255) / 256) * ((n + 127) / 128);
  if (mid >= cus)
    return launch_cfg<2, 2, 4, 2>(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out,
                                  b_srows, ldo,
                                  aligned16, s);
  return launch_cfg<2, 2, 2, 2>(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out,
                                b_srows, ldo,
                                aligned16, s);
}

}  // namespace

hipError_t set_dynamic_lds_once(const void* kernel, int bytes, bool (&done)[kMaxDevices]) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (done[dev]) return hipSuccess;
  if (hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); e != hipSuccess)
    return e;
  done[dev] = true;
  return hipSuccess;
}

int compute_units() {
  static int cached[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

namespace {

// Kernel choice by shape (operands aligned, K a multiple of 32): weight streaming up to
// 32 activation rows, and up to 64 on narrow weights (N < 4096); the pipelined kernel
// (128-row tiles up to M = 128) above that.  Measured, GEMM alone, one box: at M = 48
// and 64 the pipelined kernel takes q_proj [8192, 5120] from 31.9-33.6 to 27.5 us and
// gate [25600, 5120] from 65-70 to 54-55 us, while k_proj [1024, 5120] stays faster
// streamed (14.8 vs 18.4 us); at M = 96 and 128 it takes k_proj from 24.1-25.7 to 18.4 us.
bool prefer_skinny(int64_t m, int64_t n) { return m <= 32 || (m <= 64 && n < 4096); }

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t k, int64_t n) {
  if ((k / 2) % 16 != 0) return 0;
  if (prefer_skinny(m, n)) return gemm_skinny_workspace_bytes(m, k, n, compute_units());
  return gemm_pipe_workspace_bytes(m, k, n, compute_units());
}

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t n,
                       const float* gsf_a, const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias,
                       uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t s) {
  const int cus = compute_units();
  if (prefer_skinny(m, n) && gemm_skinny_supported(m, k, a_codes, a_scales, b_codes, b_scales))
    return launch_gemm_skinny(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out,
                              workspace, workspace_bytes, cus, s);
  if (gemm_pipe_supported(m, k, n, a_codes, a_scales, b_codes, b_scales, cus))
    return launch_gemm_pipe(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out,
                            workspace, workspace_bytes, cus, s);
  return launch_generic(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, n, n, cus,
                        s);
}

}  // namespace nvfp4
