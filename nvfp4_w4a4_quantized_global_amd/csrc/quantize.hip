// Activation / weight side of the NVFP4 linear on gfx950: abs-max reduction for the
// dynamic global scale, the fused (rotate +) quantize pass, the stand-alone block
// Hadamard rotation, and the scale-layout conversions.
//
// What is computed: "minimax_h3_nvfp4_decoder" page, nvfp4_linear_inference (a
// dynamic global scale from the call's 2-D input, then the FP4 quantize) and
// NVFP4DecoderLinear.forward / rotate_activation (the block rotation applied to the
// activation before it).  All of it is HBM-bound streaming: every kernel reads its
// input once with 16-byte loads; a 16-value block (32 bytes of bf16) is one lane's
// unit of work, so the per-block max and the per-block scale never leave registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
// Launch shapes of the two passes.  Each can be set at build time (-D) for tuning sweeps.
#ifndef NVFP4_AMAX_BLOCKS
#define NVFP4_AMAX_BLOCKS 512
#endif
#ifndef NVFP4_AMAX_UNROLL
#define NVFP4_AMAX_UNROLL 4
#endif
#ifndef NVFP4_QUANT_UNITS
#define NVFP4_QUANT_UNITS 2
#endif
#ifndef NVFP4_QUANT_BLOCKS
#define NVFP4_QUANT_BLOCKS 2048
#endif
#ifndef NVFP4_SMALL_QUANT_VALUES
#define NVFP4_SMALL_QUANT_VALUES 131072
#endif
constexpr int kAmaxBlocks = NVFP4_AMAX_BLOCKS;   // partial maxima of the amax pass (<= kMaxAmaxPartials)
static_assert(4 * kAmaxBlocks <= kMaxAmaxPartials, "partials buffer");   // SwiGLU: 4x the grid

struct Chunk16 {
  float v[16];
};

__device__ __forceinline__ void load16_f32(const float* __restrict__ p, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 t = reinterpret_cast<const float4*>(p)[i];
    v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
  }
}

// Block-wide max of a non-negative value; every thread gets the result.
__device__ __forceinline__ float block_max(float x, float* lds) {
  x = wave_max(x);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wid] = x;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

// Pass 1 of the dynamic scale: every block writes the max |v| of its share of the
// (optionally rotated, bf16-rounded) input to partials[blockIdx.x].  Lanes take
// consecutive 16-value chunks, so the lanes holding one rotation group are
// consecutive and aligned (the group divides the row length); each lane keeps
// kAmaxUnroll chunks in flight.
constexpr int kAmaxUnroll = NVFP4_AMAX_UNROLL;

// Stores 16 values that are already bf16-exact as bf16.
__device__ __forceinline__ void store16_bf16(uint16_t* __restrict__ p, const float (&v)[16]) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
  uint4* d = reinterpret_cast<uint4*>(p);
  d[0] = make_uint4(w[0], w[1], w[2], w[3]);
  d[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Loads 16 input values at element offset off: x itself, or with kSwiglu the bf16
// SwiGLU product of x (gate) and u (up).
template <bool kSwiglu>
__device__ __forceinline__ void load_input16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ u,
                                             int64_t off, float (&v)[16]) {
  load16_bf16(x + off, v);
  if (kSwiglu) {
    float w[16];
    load16_bf16(u + off, w);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = swiglu_bf16(v[i], w[i]);
  }
}

// Segments (blockIdx.y) are consecutive row blocks of n_chunks chunks each, reduced
// separately into partials[blockIdx.y * gridDim.x + blockIdx.x].  With kSwiglu the
// input is formed from gate (x) and up and, when xout is not NULL, also stored there,
// so the quantize pass reads the product instead of forming it again.
template <bool kRotate, bool kSwiglu>
__global__ void __launch_bounds__(kThreads) amax_partial_kernel(const uint16_t* __restrict__ x,
                                                                 const uint16_t* __restrict__ up,
                                                                 uint16_t* __restrict__ xout, int64_t n_chunks,
                                                                 int group, float inv_sqrt_g,
                                                                 float* __restrict__ partials) {
  __shared__ float lds[kThreads / 64];
  x += (int64_t)blockIdx.y * n_chunks * 16;
  if (kSwiglu) up += (int64_t)blockIdx.y * n_chunks * 16;
  if (kSwiglu && xout != nullptr) xout += (int64_t)blockIdx.y * n_chunks * 16;
  // memory-bound plain input: several chunks in flight per lane; the ALU-bound SwiGLU
  // product: one, for more waves per SIMD
  constexpr int kUnroll = kSwiglu ? 1 : kAmaxUnroll;
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads; c0 < n_chunks; c0 += stride * kUnroll) {
    float v[kUnroll][16];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + u * stride + threadIdx.x;
      if (c < n_chunks) {
        load_input16<kSwiglu>(x, up, c * 16, v[u]);
        if (kSwiglu && xout != nullptr) store16_bf16(xout + c * 16, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (kRotate) rotate16_bf16(v[u], group, inv_sqrt_g);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[u][i]));
    }
  }
  m = block_max(m, lds);
  if (threadIdx.x == 0) partials[blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// One lane's share of a quantize unit (row, 128-wide K tile): lane j of the unit's eight
// owns 16-block j.  v holds its 16 input values (zeros past the end); the block is
// rotated (all lanes of the wave take part), quantized under global scale gsf, and its
// codes (and, with a16, its fp16 operand form) stored; the unit's 8 scale bytes are
// gathered into lane j == 0 and written as one 8-byte word.
template <bool kRotate>
__device__ __forceinline__ void quantize_unit(float (&v)[16], int64_t row, int64_t kt, int j, int64_t m_rows,
                                              int64_t k, int group, float inv_sqrt_g, float gsf,
                                              uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                              uint16_t* __restrict__ a16) {
  if (kRotate) rotate16_bf16(v, group, inv_sqrt_g);
  const int64_t blk = kt * 8 + j;
  const bool in_row = row < m_rows;
  const bool valid = in_row && blk < k / kBlock;
  uint32_t w0, w1;
  const uint32_t s8 = quantize_block16(v, gsf, valid, w0, w1);
  if (valid) *reinterpret_cast<uint2*>(codes + row * (k / 2) + blk * 8) = make_uint2(w0, w1);
  if (a16 != nullptr && valid) {
    // the block's values in the GEMMs' operand form: fp16 code * scale * 2^-8, exact
    const gemm::half2_t sc = gemm::as_half2((s8 << 7) | (s8 << 23));
    uint4* d = reinterpret_cast<uint4*>(a16 + row * k + blk * kBlock);
    d[0] = __builtin_bit_cast(uint4, gemm::dequant8(w0, sc));
    d[1] = __builtin_bit_cast(uint4, gemm::dequant8(w1, sc));
  }
  uint32_t lo = j < 4 ? s8 << (8 * j) : 0u;
  uint32_t hi = j >= 4 ? s8 << (8 * (j - 4)) : 0u;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    lo |= __shfl_xor(lo, o, 64);
    hi |= __shfl_xor(hi, o, 64);
  }
  if (j == 0 && in_row) *reinterpret_cast<uint2*>(scales + (kt * m_rows + row) * 8) = make_uint2(lo, hi);
}

// Pass 2: quantize.  Eight consecutive lanes own one 128-wide K tile of one row
// (a "unit"; lane j of the eight owns the 16-block j of the tile), so each group of
// eight reads 256 contiguous bytes and writes 64 contiguous code bytes and the 8
// scale bytes that are contiguous in the k-tile-major scale layout.  Blocks take the
// global scale once, then loop over groups of kQuantUnits x 32 units, loading a
// group's units before computing them.
constexpr int kQuantUnits = NVFP4_QUANT_UNITS;
// Grid cap (blocks loop over the units): more blocks in flight pay off once the input
// is several times larger than one pass of the cap; below that the per-block scale
// prologue dominates.
constexpr int kQuantBlocks = NVFP4_QUANT_BLOCKS;
constexpr int kQuantBlocksLarge = 8192;
constexpr int64_t kLargeUnits = (int64_t)1 << 19;

// With a dynamic scale the rows form `segments` consecutive blocks of seg_rows rows,
// each with its own global scale from its own n_partials partial maxima (one segment
// for a plain call); gsf_out receives one scale per segment.
template <bool kRotate, bool kSwiglu>
__global__ void __launch_bounds__(kThreads) quantize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ up, int64_t m_rows, int64_t k, int group,
    float inv_sqrt_g,
    const float* __restrict__ static_gsf, const float* __restrict__ partials, int n_partials, int64_t seg_rows,
    int segments, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gsf_out,
    uint16_t* __restrict__ a16) {
  __shared__ uint32_t seg_amax[kMaxSegments];   // segment maxima, then global scales (bits)
  __shared__ float lds[kThreads / 64];
  const int64_t kt_count = (k + kScaleTileK - 1) / kScaleTileK;
  const int64_t nb = k / kBlock;
  const int j = threadIdx.x & 7;

  const bool dynamic = static_gsf == nullptr;
  const float gsf_static = dynamic ? 0.0f : *static_gsf;
  if (dynamic && segments == 1) {
    float a = 0.0f;
    for (int i = threadIdx.x; i < n_partials; i += kThreads) a = fmaxf(a, partials[i]);
    a = block_max(a, lds);
    if (threadIdx.x == 0) seg_amax[0] = __float_as_uint(global_scale_from_amax(a));
    __syncthreads();
  } else if (dynamic) {
    // max of non-negative floats = max of their bit patterns
    for (int i = threadIdx.x; i < segments; i += kThreads) seg_amax[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < segments * n_partials; i += kThreads)
      atomicMax(&seg_amax[i / n_partials], __float_as_uint(partials[i]));
    __syncthreads();
    for (int i = threadIdx.x; i < segments; i += kThreads)
      seg_amax[i] = __float_as_uint(global_scale_from_amax(__uint_as_float(seg_amax[i])));
    __syncthreads();
  }
  if (gsf_out != nullptr && blockIdx.x == 0) {
    if (dynamic) {
      for (int i = threadIdx.x; i < segments; i += kThreads) gsf_out[i] = __uint_as_float(seg_amax[i]);
    } else if (threadIdx.x == 0) {
      *gsf_out = gsf_static;
    }
  }

  const int64_t units_total = m_rows * kt_count;
  const int64_t per_block = (int64_t)kQuantUnits * (kThreads / 8);
  for (int64_t base = (int64_t)blockIdx.x; base * per_block < units_total; base += gridDim.x) {
    float v[kQuantUnits][16];
    int64_t row[kQuantUnits], kt[kQuantUnits];
#pragma unroll
    for (int u = 0; u < kQuantUnits; ++u) {
      const int64_t unit = (base * kQuantUnits + u) * (kThreads / 8) + (threadIdx.x >> 3);
      row[u] = unit / kt_count;
      kt[u] = unit - row[u] * kt_count;
      const int64_t blk = kt[u] * 8 + j;
      if (row[u] < m_rows && blk < nb) {
        load_input16<kSwiglu>(x, up, row[u] * k + blk * kBlock, v[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[u][i] = 0.0f;
      }
    }

#pragma unroll
    for (int u = 0; u < kQuantUnits; ++u) {
      const bool in_row = row[u] < m_rows;
      const float gsf = dynamic ? __uint_as_float(seg_amax[in_row ? row[u] / seg_rows : 0]) : gsf_static;
      quantize_unit<kRotate>(v[u], row[u], kt[u], j, m_rows, k, group, inv_sqrt_g, gsf, codes, scales, a16);
    }
  }
}

// Dynamic-scale quantize of a small input in one launch: every workgroup computes the
// abs-max of the whole (rotated) input by itself (the input is small and sits in L2),
// forms the global scale and quantizes its share of the units, so the two passes above
// cost one launch and no workgroup waits for another.  The maxima agree bit for bit (a
// max does not depend on order), so every workgroup uses the same scale.  For inputs
// of at most kSmallQuantValues values, where launch and ramp time outweigh the
// streaming; one workgroup per kSmallThreads / 8 units, at most kSmallBlocks.
constexpr int kSmallThreads = 1024;
constexpr int64_t kSmallQuantValues = NVFP4_SMALL_QUANT_VALUES;
#ifndef NVFP4_SMALL_QUANT_BLOCKS
#define NVFP4_SMALL_QUANT_BLOCKS 16
#endif
constexpr int kSmallBlocks = NVFP4_SMALL_QUANT_BLOCKS;
constexpr int kSmallUnroll = 4;   // pass-1 chunks in flight per lane (with a rotation)
constexpr int kSmallRaw = (int)(kSmallQuantValues / kBlock / kSmallThreads);   // without one
static_assert(kSmallRaw >= 1 && kSmallRaw <= 8, "bf16 chunks per lane in flight");

template <bool kRotate>
__global__ void __launch_bounds__(kSmallThreads) quantize_small_kernel(
    const uint16_t* __restrict__ x, int64_t m_rows, int64_t k, int group, float inv_sqrt_g,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ gsf_out,
    uint16_t* __restrict__ a16) {
  __shared__ float lds[kSmallThreads / 64];
  const int t = threadIdx.x;
  // pass 1, the whole input in every workgroup: consecutive lanes take consecutive
  // 16-value chunks (a rotation group's chunks sit in consecutive, aligned lanes).  Past
  // one chunk per lane, kSmallUnroll chunks per lane are loaded before any is reduced.
  const int64_t n_chunks = m_rows * k / kBlock;
  float mx = 0.0f;
  auto chunk_max = [&](float (&v)[16]) {
    if (kRotate) rotate16_bf16(v, group, inv_sqrt_g);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(v[i]));
  };
  if (n_chunks <= kSmallThreads) {
    float v[16];
    if (t < n_chunks) {
      load16_bf16(x + (int64_t)t * kBlock, v);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    chunk_max(v);
  } else if (!kRotate && n_chunks > kSmallUnroll * kSmallThreads) {
    // Past one round of kSmallUnroll chunks per lane, and without a rotation, every
    // chunk of the lane is in flight at once (at most kSmallRaw under the size
    // threshold), kept as bf16, and the abs-max is taken on the magnitude bits, which
    // order as the values do for every bf16 but NaN (an input with NaNs has no defined
    // scale).  Measured, dynamic linear at 16 rows (HIP graph, one box): o_proj 18.0 ->
    // 17.0 us, gate 27.5 -> 26.8, k 11.4 -> 10.9.
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m2 = {0, 0};
    for (int64_t c0 = 0; c0 < n_chunks; c0 += kSmallRaw * kSmallThreads) {
      uint4 r[kSmallRaw][2];
#pragma unroll
      for (int u = 0; u < kSmallRaw; ++u) {
        const int64_t c = c0 + u * kSmallThreads + t;
        if (c < n_chunks) {
          r[u][0] = reinterpret_cast<const uint4*>(x + c * kBlock)[0];
          r[u][1] = reinterpret_cast<const uint4*>(x + c * kBlock)[1];
        } else {
          r[u][0] = r[u][1] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int u = 0; u < kSmallRaw; ++u) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t w[4] = {r[u][h].x, r[u][h].y, r[u][h].z, r[u][h].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[e] & 0x7FFF7FFFu));
        }
      }
    }
    mx = __uint_as_float((uint32_t)(m2.x > m2.y ? m2.x : m2.y) << 16);
  } else {
    for (int64_t c0 = 0; c0 < n_chunks; c0 += kSmallUnroll * kSmallThreads) {
      float v[kSmallUnroll][16];
#pragma unroll
      for (int u = 0; u < kSmallUnroll; ++u) {
        const int64_t c = c0 + u * kSmallThreads + t;
        if (c < n_chunks) {
          load16_bf16(x + c * kBlock, v[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[u][i] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < kSmallUnroll; ++u) chunk_max(v[u]);
    }
  }
  mx = wave_max(mx);
  if ((t & 63) == 0) lds[t >> 6] = mx;
  __syncthreads();
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kSmallThreads / 64; ++i) amax = fmaxf(amax, lds[i]);
  const float gsf = global_scale_from_amax(amax);
  if (t == 0 && blockIdx.x == 0 && gsf_out != nullptr) *gsf_out = gsf;
  // pass 2: this workgroup's units of quantize_kernel, eight lanes each (the input is
  // re-read from L2)
  const int64_t kt_count = (k + kScaleTileK - 1) / kScaleTileK;
  const int64_t units = m_rows * kt_count;
  const int j = t & 7;
  for (int64_t u0 = (int64_t)blockIdx.x * (kSmallThreads / 8); u0 < units;
       u0 += (int64_t)gridDim.x * (kSmallThreads / 8)) {
    const int64_t unit = u0 + (t >> 3);
    const int64_t row = unit / kt_count, kt = unit - row * kt_count;
    const int64_t blk = kt * 8 + j;
    float v[16];
    if (row < m_rows && blk < k / kBlock) {
      load16_bf16(x + row * k + blk * kBlock, v);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    quantize_unit<kRotate>(v, row, kt, j, m_rows, k, group, inv_sqrt_g, gsf, codes, scales, a16);
  }
}

// NVFP4 -> real values: each 16-block fp32(code * scale) / gsf, stored as bf16 (RNE) or
// fp32.  One lane per block: 8 code bytes in, 32 or 64 bytes out.
template <bool kOutBf16>
__global__ void __launch_bounds__(kThreads) dequant_kernel(const uint8_t* __restrict__ packed,
                                                            const uint8_t* __restrict__ scales, int64_t rows, int64_t k,
                                                            const float* __restrict__ gsf, void* __restrict__ out) {
  const int64_t nb = k / kBlock;
  const int64_t blocks = rows * nb;
  const float g = *gsf;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < blocks; b += stride) {
    const int64_t r = b / nb, j = b - r * nb;
    const uint2 c = *reinterpret_cast<const uint2*>(packed + r * (k / 2) + j * 8);
    const float s = e4m3_decode(scales[((j >> 3) * rows + r) * 8 + (j & 7)]);
    const uint32_t w[2] = {c.x, c.y};
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __fdiv_rn(__fmul_rn(e2m1_decode((w[i >> 3] >> (4 * (i & 7))) & 0xFu), s), g);
    if (kOutBf16) {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f32_to_bf16(v[2 * i]) | (f32_to_bf16(v[2 * i + 1]) << 16);
      uint4* d = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + r * k + j * kBlock);
      d[0] = make_uint4(o[0], o[1], o[2], o[3]);
      d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
      float4* d = reinterpret_cast<float4*>(static_cast<float*>(out) + r * k + j * kBlock);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
  }
}

// Calibration: *amax = max over the partial maxima, or max(*amax, that) when
// accumulating over batches.
__global__ void __launch_bounds__(kThreads) amax_finalize_kernel(const float* __restrict__ partials, int n_partials,
                                                                  float* __restrict__ amax, int accumulate) {
  __shared__ float lds[kThreads / 64];
  float a = 0.0f;
  for (int i = threadIdx.x; i < n_partials; i += kThreads) a = fmaxf(a, partials[i]);
  a = block_max(a, lds);
  if (threadIdx.x == 0) *amax = accumulate ? fmaxf(*amax, a) : a;
}

// Static activation scale from a calibrated amax: the stored range is fp32(amax *
// margin) and the scale 2688 / max(range, 1e-12), both in fp32.
__global__ void static_scale_kernel(const float* __restrict__ amax, float margin, float* __restrict__ gsf) {
  if (threadIdx.x == 0) *gsf = global_scale_from_amax(__fmul_rn(*amax, margin));
}

// Stand-alone rotation: x (bf16 or fp32) -> y (bf16 or fp32), one 16-value chunk per lane.
template <typename Tin, bool kOutBf16>
__global__ void __launch_bounds__(kThreads) rotate_kernel(const Tin* __restrict__ x, void* __restrict__ y,
                                                          int64_t n_chunks, int group, float inv_sqrt_g) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads; c0 < n_chunks; c0 += stride) {
    const int64_t c = c0 + threadIdx.x;
    float v[16];
    if (c < n_chunks) {
      if constexpr (sizeof(Tin) == 2) load16_bf16(reinterpret_cast<const uint16_t*>(x) + c * 16, v);
      else load16_f32(reinterpret_cast<const float*>(x) + c * 16, v);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    fwht16_local(v, group);
    fwht16_cross(v, group);
    if (c < n_chunks) {
      if constexpr (kOutBf16) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w[i] = f32_to_bf16(__fmul_rn(v[2 * i], inv_sqrt_g)) | (f32_to_bf16(__fmul_rn(v[2 * i + 1], inv_sqrt_g)) << 16);
        uint4* out = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(y) + c * 16);
        out[0] = make_uint4(w[0], w[1], w[2], w[3]);
        out[1] = make_uint4(w[4], w[5], w[6], w[7]);
      } else {
        float4* out = reinterpret_cast<float4*>(reinterpret_cast<float*>(y) + c * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[i] = make_float4(__fmul_rn(v[4 * i], inv_sqrt_g), __fmul_rn(v[4 * i + 1], inv_sqrt_g),
                               __fmul_rn(v[4 * i + 2], inv_sqrt_g), __fmul_rn(v[4 * i + 3], inv_sqrt_g));
      }
    }
  }
}

// Scale-layout conversion; one thread per (row, 128-K tile): 8 bytes.
template <bool kToCanonical>
__global__ void __launch_bounds__(kThreads) scale_layout_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                                int64_t rows, int64_t k) {
  const int64_t kt_count = (k + kScaleTileK - 1) / kScaleTileK;
  const int64_t nb = k / kBlock;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= rows * kt_count) return;
  const int64_t kt = t / rows;
  const int64_t row = t - kt * rows;
  for (int j = 0; j < 8; ++j) {
    const int64_t b = kt * 8 + j;
    const int64_t lay = (kt * rows + row) * 8 + j;
    if (kToCanonical) {
      if (b < nb) dst[row * nb + b] = src[lay];
    } else {
      dst[lay] = b < nb ? src[row * nb + b] : (uint8_t)0;
    }
  }
}

int64_t grid_for(int64_t n_chunks, int64_t cap) {
  int64_t g = (n_chunks + kThreads - 1) / kThreads;
  if (g > cap) g = cap;
  return g < 1 ? 1 : g;
}

}  // namespace

hipError_t launch_amax_partials(const uint16_t* x, const uint16_t* up, uint16_t* xout, int64_t seg_rows, int64_t k,
                                int segments, int group, float inv_sqrt_g, float* partials, int* n_partials,
                                hipStream_t s) {
  const int64_t n_chunks = seg_rows * k / kBlock;
  // the SwiGLU product costs ~45 VALU operations per value: more blocks in flight
  int64_t cap = (up != nullptr ? 4 * kAmaxBlocks : kAmaxBlocks) / segments;
  if (cap < 1) cap = 1;
  const int unroll = up != nullptr ? 1 : kAmaxUnroll;
  const int grid = (int)grid_for((n_chunks + unroll - 1) / unroll, cap);
  *n_partials = grid;
  const dim3 g3((uint32_t)grid, (uint32_t)segments);
  const bool rot = group > 1;
  if (up != nullptr && rot)
    hipLaunchKernelGGL((amax_partial_kernel<true, true>), g3, dim3(kThreads), 0, s, x, up, xout, n_chunks, group, inv_sqrt_g, partials);
  else if (up != nullptr)
    hipLaunchKernelGGL((amax_partial_kernel<false, true>), g3, dim3(kThreads), 0, s, x, up, xout, n_chunks, group, inv_sqrt_g, partials);
  else if (rot)
    hipLaunchKernelGGL((amax_partial_kernel<true, false>), g3, dim3(kThreads), 0, s, x, up, xout, n_chunks, group, inv_sqrt_g, partials);
  else
    hipLaunchKernelGGL((amax_partial_kernel<false, false>), g3, dim3(kThreads), 0, s, x, up, xout, n_chunks, group, inv_sqrt_g, partials);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, const uint16_t* up, int64_t rows, int64_t k, int group,
                           float inv_sqrt_g, const float* static_gsf, const float* partials, int n_partials,
                           int64_t seg_rows, int segments, uint8_t* codes, uint8_t* scales, float* gsf_out,
                           hipStream_t s, uint16_t* a16) {
  const int64_t kt_count = (k + kScaleTileK - 1) / kScaleTileK;
  const int64_t units = rows * kt_count;
  const int64_t per_block = (int64_t)kQuantUnits * (kThreads / 8);
  int64_t grid = (units + per_block - 1) / per_block;
  const int64_t cap = units > kLargeUnits ? kQuantBlocksLarge : kQuantBlocks;
  if (grid > cap) grid = cap;
  const dim3 g1((uint32_t)grid);
  const bool rot = group > 1;
  if (up != nullptr && rot)
    hipLaunchKernelGGL((quantize_kernel<true, true>), g1, dim3(kThreads), 0, s, x, up, rows, k, group, inv_sqrt_g,
                       static_gsf, partials, n_partials, seg_rows, segments, codes, scales, gsf_out, a16);
  else if (up != nullptr)
    hipLaunchKernelGGL((quantize_kernel<false, true>), g1, dim3(kThreads), 0, s, x, up, rows, k, group, inv_sqrt_g,
                       static_gsf, partials, n_partials, seg_rows, segments, codes, scales, gsf_out, a16);
  else if (rot)
    hipLaunchKernelGGL((quantize_kernel<true, false>), g1, dim3(kThreads), 0, s, x, up, rows, k, group, inv_sqrt_g,
                       static_gsf, partials, n_partials, seg_rows, segments, codes, scales, gsf_out, a16);
  else
    hipLaunchKernelGGL((quantize_kernel<false, false>), g1, dim3(kThreads), 0, s, x, up, rows, k, group, inv_sqrt_g,
                       static_gsf, partials, n_partials, seg_rows, segments, codes, scales, gsf_out, a16);
  return hipGetLastError();
}

bool quantize_small_supported(int64_t rows, int64_t k) { return rows * k <= kSmallQuantValues; }

hipError_t launch_quantize_small(const uint16_t* x, int64_t rows, int64_t k, int group, float inv_sqrt_g,
                                 uint8_t* codes, uint8_t* scales, float* gsf_out, hipStream_t s, uint16_t* a16) {
  const int64_t units = rows * ((k + kScaleTileK - 1) / kScaleTileK);
  const int64_t want = (units + kSmallThreads / 8 - 1) / (kSmallThreads / 8);
  const dim3 grid((uint32_t)std::max<int64_t>(1, std::min<int64_t>(want, kSmallBlocks)));
  if (group > 1)
    hipLaunchKernelGGL(quantize_small_kernel<true>, grid, dim3(kSmallThreads), 0, s, x, rows, k, group, inv_sqrt_g,
                       codes, scales, gsf_out, a16);
  else
    hipLaunchKernelGGL(quantize_small_kernel<false>, grid, dim3(kSmallThreads), 0, s, x, rows, k, group, inv_sqrt_g,
                       codes, scales, gsf_out, a16);
  return hipGetLastError();
}

// x = bf16 SwiGLU product of gate and up, one 16-value chunk per lane.
__global__ void __launch_bounds__(kThreads) swiglu_kernel(const uint16_t* __restrict__ gate,
                                                           const uint16_t* __restrict__ up, uint16_t* __restrict__ x,
                                                           int64_t n_chunks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < n_chunks; c += stride) {
    float v[16];
    load_input16<true>(gate, up, c * 16, v);
    store16_bf16(x + c * 16, v);
  }
}

hipError_t launch_swiglu(const uint16_t* gate, const uint16_t* up, uint16_t* x, int64_t rows, int64_t k, hipStream_t s) {
  const int64_t n_chunks = rows * k / kBlock;
  hipLaunchKernelGGL(swiglu_kernel, dim3((uint32_t)grid_for(n_chunks, 8192)), dim3(kThreads), 0, s, gate, up, x, n_chunks);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, const float* gsf,
                          void* out, bool out_bf16, hipStream_t s) {
  const int grid = (int)grid_for(rows * (k / kBlock), 8192);
  if (out_bf16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid), dim3(kThreads), 0, s, packed, scales, rows, k, gsf, out);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid), dim3(kThreads), 0, s, packed, scales, rows, k, gsf, out);
  return hipGetLastError();
}

hipError_t launch_amax_finalize(const float* partials, int n_partials, float* amax, bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(amax_finalize_kernel, dim3(1), dim3(kThreads), 0, s, partials, n_partials, amax, (int)accumulate);
  return hipGetLastError();
}

hipError_t launch_static_scale(const float* amax, float margin, float* gsf, hipStream_t s) {
  hipLaunchKernelGGL(static_scale_kernel, dim3(1), dim3(64), 0, s, amax, margin, gsf);
  return hipGetLastError();
}

hipError_t launch_rotate(const void* x, bool x_bf16, void* y, bool y_bf16, int64_t rows, int64_t k, int group,
                         float inv_sqrt_g, hipStream_t s) {
  const int64_t n_chunks = rows * k / kBlock;
  const int grid = (int)grid_for(n_chunks, 8192);
  if (x_bf16 && y_bf16)
    hipLaunchKernelGGL((rotate_kernel<uint16_t, true>), dim3(grid), dim3(kThreads), 0, s, (const uint16_t*)x, y, n_chunks, group, inv_sqrt_g);
  else if (x_bf16)
    hipLaunchKernelGGL((rotate_kernel<uint16_t, false>), dim3(grid), dim3(kThreads), 0, s, (const uint16_t*)x, y, n_chunks, group, inv_sqrt_g);
  else if (y_bf16)
    hipLaunchKernelGGL((rotate_kernel<float, true>), dim3(grid), dim3(kThreads), 0, s, (const float*)x, y, n_chunks, group, inv_sqrt_g);
  else
    hipLaunchKernelGGL((rotate_kernel<float, false>), dim3(grid), dim3(kThreads), 0, s, (const float*)x, y, n_chunks, group, inv_sqrt_g);
  return hipGetLastError();
}

hipError_t launch_scale_layout(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t k, bool to_canonical, hipStream_t s) {
  const int64_t kt_count = (k + kScaleTileK - 1) / kScaleTileK;
  const int64_t n = rows * kt_count;
  const int64_t grid = (n + kThreads - 1) / kThreads;
  if (to_canonical)
    hipLaunchKernelGGL(scale_layout_kernel<true>, dim3((uint32_t)grid), dim3(kThreads), 0, s, src, dst, rows, k);
  else
    hipLaunchKernelGGL(scale_layout_kernel<false>, dim3((uint32_t)grid), dim3(kThreads), 0, s, src, dst, rows, k);
  return hipGetLastError();
}

}  // namespace nvfp4
