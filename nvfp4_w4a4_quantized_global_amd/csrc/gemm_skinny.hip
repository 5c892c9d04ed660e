// NVFP4 GEMM for few activation rows (M <= 128): weight streaming.
//
// Same product as gemm.hip ("minimax_h3_nvfp4_decoder" page, nvfp4_linear_inference:
// mm_fp4 with alpha = 1/(global_sf_x*global_sf_w), then the bias add), for the decode
// shapes where the packed weight (N*K/2 code bytes + N*K/16 scale bytes) is the traffic
// that matters: every weight byte is read from HBM exactly once, the activation codes
// come from L2.
//
// Work: a block owns 64 output columns (weight rows) and a range of 256-wide K super
// tiles (two tiles of the scale layout); its four waves take the super tiles
// round-robin and their fp32 results are summed through LDS in wave order.  When that
// leaves too few blocks to fill the GPU, the K range is also split across blocks (fp32
// partials in a workspace, summed in split order by gemm_skinny_reduce), so results
// are bitwise repeatable.
//
// Operands are expanded to fp16 exactly (gemm_common.h) and multiplied on
// v_mfma_f32_16x16x32_f16.  In every MFMA, lane group g = lane / 16 supplies K values
// [64g + 8s, +8) of the super tile at sub-step s for both operands (a consistent
// permutation of K), so each lane loads 32 contiguous code bytes per row and the 16
// lanes of a row together read its whole 128-byte line.
//
// At most 16 rows take gemm_decode_kernel below instead: 16 columns per block, the
// operands streamed through per-wave LDS slots by direct loads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

namespace nvfp4 {
namespace {

using namespace gemm;

typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kCols = 64;            // output columns per block (4 MFMA tiles of 16)
constexpr int kWaves = 4;

// kFusedA (MT == 1): A arrives as bf16 values (a_bf16, [m][k], m <= 16) with a static
// global scale (*gsf_a).  The block first quantizes its K range of A into LDS, each
// 16-block once and exactly as the quantize kernel would, and the waves then read A's
// codes and scales from LDS instead of global memory.
constexpr int kFusedMaxSt = 16;   // super tiles of A one block can stage
template <int MT, bool kFusedA>   // M tiles of 16 rows
__global__ void __launch_bounds__(256) gemm_skinny_kernel(
    const uint16_t* __restrict__ a_bf16,
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m, int64_t k,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int64_t n,
    const float* __restrict__ gsf_a, const float* __restrict__ gsf_b, int64_t a_seg_rows,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int splits, float* __restrict__ partial) {
  __shared__ float red[MT * 4][4][64];     // waves 1..3 hand their sums to wave 0, one at a time

  const int col_group = blockIdx.x / splits;
  const int split = blockIdx.x % splits;
  const int64_t n0 = (int64_t)col_group * kCols;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int64_t half_k = k / 2;
  const int64_t kt_all = (k + BK - 1) / BK;
  const int64_t st_all = (kt_all + 1) / 2;                 // 256-wide super tiles
  const int64_t st_begin = st_all * split / splits;
  const int64_t st_end = st_all * (split + 1) / splits;

  // Row pointers (rows past the end clamp to the last row; their outputs are dropped).
  const uint8_t* brow[4];
  const uint8_t* bsrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t r = min(n0 + 16 * j + l16, n - 1);
    brow[j] = b_codes + r * half_k;
    bsrow[j] = b_scales + r * 8 + 4 * (g & 1);
  }
  const uint8_t* arow[MT];
  const uint8_t* asrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int64_t r = min((int64_t)(16 * i + l16), m - 1);
    if (!kFusedA) {
      arow[i] = a_codes + r * half_k;
      asrow[i] = a_scales + r * 8 + 4 * (g & 1);
    }
  }

  float4_t acc[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // One 256-wide K super tile (two scale-layout tiles) per wave and iteration, so each
  // row's 128 code bytes (a whole cache line) are read by one instruction.  Lane group g
  // takes K values [64g, 64g + 64) of the super tile: 32 code bytes and the 4 scale
  // bytes of its blocks, which sit in scale tile 2t + g/2 at byte offset 4 (g % 2).
  // The next super tile's operands are in flight while this one is multiplied.
  struct Tile {
    uint4 bc[4][2];
    uint32_t bs[4];
    uint4 ac[MT][2];
    uint32_t as[MT];
  };
  auto fetch_b = [&](int64_t st, Tile& T) {
    const int64_t off = st * 128 + 32 * g;           // code byte offset of this lane's 32 bytes
    const int64_t kt = 2 * st + (g >> 1);             // its scale tile
    const bool c0 = off < half_k, c1 = off + 16 < half_k, sv = kt < kt_all;   // partial last super tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      T.bc[j][0] = c0 ? *reinterpret_cast<const uint4*>(brow[j] + off) : make_uint4(0, 0, 0, 0);
      T.bc[j][1] = c1 ? *reinterpret_cast<const uint4*>(brow[j] + off + 16) : make_uint4(0, 0, 0, 0);
      T.bs[j] = sv ? *reinterpret_cast<const uint32_t*>(bsrow[j] + kt * n * 8) : 0u;
    }
  };
  auto fetch_a = [&](int64_t st, Tile& T) {
    const int64_t off = st * 128 + 32 * g;
    const int64_t kt = 2 * st + (g >> 1);
    const bool c0 = off < half_k, c1 = off + 16 < half_k, sv = kt < kt_all;
    (void)c0; (void)c1; (void)sv;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (kFusedA) {
        // staged rows: code bytes [128 ls + 32 g, +32) and scale bytes [16 ls + 4 g, +4)
        const int ls = (int)(st - st_begin);
        T.ac[i][0] = *reinterpret_cast<const uint4*>(arow[i] + ls * 128 + 32 * g);
        T.ac[i][1] = *reinterpret_cast<const uint4*>(arow[i] + ls * 128 + 32 * g + 16);
        T.as[i] = *reinterpret_cast<const uint32_t*>(asrow[i] + ls * 16 + 4 * g);
      } else {
        T.ac[i][0] = c0 ? *reinterpret_cast<const uint4*>(arow[i] + off) : make_uint4(0, 0, 0, 0);
        T.ac[i][1] = c1 ? *reinterpret_cast<const uint4*>(arow[i] + off + 16) : make_uint4(0, 0, 0, 0);
        T.as[i] = sv ? *reinterpret_cast<const uint32_t*>(asrow[i] + kt * m * 8) : 0u;
      }
    }
  };
  auto multiply = [&](const Tile& T) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {                     // K values [64g + 8s, +8): block s/2
      half8_t fb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = dequant8(word(T.bc[j][s >> 2], s & 3), scale_pair(T.bs[j], s >> 1));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const half8_t fa = dequant8(word(T.ac[i][s >> 2], s & 3), scale_pair(T.as[i], s >> 1));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  auto fetch = [&](int64_t st, Tile& T) {
    fetch_b(st, T);
    fetch_a(st, T);
  };
  int64_t st = st_begin + wave;
  Tile cur;
  if (st < st_end) fetch_b(st, cur);   // the first weight loads are in flight while A is staged
  if constexpr (kFusedA) {  // quantize this block's K range of A into LDS
    __shared__ __attribute__((aligned(16))) uint8_t a_codes_lds[16][kFusedMaxSt * 128];
    __shared__ __attribute__((aligned(16))) uint8_t a_scales_lds[16][kFusedMaxSt * 16];
    const float gsf_q = *gsf_a;
    const int nblk = (int)(st_end - st_begin) * 16;        // 16-blocks of this K range per row
    for (int q = threadIdx.x; q < m * nblk; q += 256) {
      const int r = q / nblk, b = q - r * nblk;
      const int64_t e0 = (st_begin * 16 + b) * (int64_t)kBlock;
      float v[16];
      if (e0 < k) {
        load16_bf16(a_bf16 + r * k + e0, v);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
      }
      uint32_t w0, w1;
      a_scales_lds[r][b] = (uint8_t)quantize_block16(v, gsf_q, e0 < k, w0, w1);
      *reinterpret_cast<uint2*>(&a_codes_lds[r][b * 8]) = make_uint2(w0, w1);
    }
    __syncthreads();
    arow[0] = &a_codes_lds[min((int64_t)l16, m - 1)][0];
    asrow[0] = &a_scales_lds[min((int64_t)l16, m - 1)][0];
  }
  if (st < st_end) {
    fetch_a(st, cur);
    for (; st < st_end; st += kWaves) {
      Tile nxt;
      if (st + kWaves < st_end) fetch(st + kWaves, nxt);
      multiply(cur);
      cur = nxt;
    }
  }

  // Sum the four waves' K subsets in wave order: ((w0 + w1) + w2) + w3.
  for (int w = 1; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[i * 4 + j][e][lane] = acc[i][j][e];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += red[i * 4 + j][e][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // 16x16 MFMA output: lane holds column l16 of each tile, rows 4g .. 4g+3.
  const float alpha = __fdiv_rn(1.0f, __fmul_rn(*gsf_a, *gsf_b));   // one activation scale
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t col = n0 + 16 * j + l16;
    if (col >= n) continue;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = 16 * i + 4 * g + e;
        if (row >= m) continue;
        if (splits > 1) {
          partial[((int64_t)split * m + row) * n + col] = acc[i][j][e];
        } else {
          const float al = a_seg_rows > 0 ? alpha_for(gsf_a, gsf_b, a_seg_rows, row) : alpha;
          uint32_t y = f32_to_bf16(__fmul_rn(al, __fmul_rn(acc[i][j][e], kAccUnscale)));
          if (bias != nullptr) y = add_bias_bf16(y, bias[col]);
          out[row * n + col] = (uint16_t)y;
        }
      }
    }
  }
}

// Sums the per-split partials [splits][m][n] in split order, then the epilogue.
__global__ void __launch_bounds__(256) gemm_skinny_reduce(const float* __restrict__ partial, int splits, int64_t m,
                                                          int64_t n, const float* __restrict__ gsf_a,
                                                          const float* __restrict__ gsf_b, int64_t a_seg_rows,
                                                          const uint16_t* __restrict__ bias, uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= m * n) return;
  float acc = 0.0f;
  for (int sp = 0; sp < splits; ++sp) acc += partial[sp * m * n + idx];
  const float alpha = alpha_for(gsf_a, gsf_b, a_seg_rows, idx / n);
  uint32_t y = f32_to_bf16(__fmul_rn(alpha, __fmul_rn(acc, kAccUnscale)));
  if (bias != nullptr) y = add_bias_bf16(y, bias[idx % n]);
  out[idx] = (uint16_t)y;
}

// Block-level K splits: at most two blocks per compute unit (the kernel's registers
// allow two resident), so all blocks run in one round, each block keeping at least one
// 256-wide super tile per wave.
int skinny_splits(int64_t k, int64_t n, int cus) {
  const int64_t groups = (n + kCols - 1) / kCols;
  const int64_t st = ((k + BK - 1) / BK + 1) / 2;
  int64_t sp = (2 * cus) / groups;
  const int64_t max_sp = st / kWaves > 0 ? st / kWaves : 1;
  if (sp > max_sp) sp = max_sp;
  return (int)(sp < 1 ? 1 : sp);
}

// Decode (m <= 16): a block owns 16 weight rows (one MFMA column tile) and a K range
// whose 256-wide super tiles its four waves split into four consecutive quarters.  Each
// wave streams its quarter through a ring of kDecDepth LDS slots with direct
// global -> LDS loads (global_load_lds), one slot per super tile: the 16 weight rows and
// the m (<= 16, clamped) activation rows as whole 128-byte lines (load instruction h
// covers rows 8h .. 8h + 7, lane l: row 8h + l / 8, 16-byte position l % 8), and the
// two K tiles' scale words of both operands.  Chunk c of row r sits at position
// c ^ ((r / 2) % 8), which keeps the 16-byte MFMA-layout reads (lane (n, g): row n,
// bytes 32 g .. 32 g + 31 of the super tile) free of bank conflicts.  The loop has no
// lane-dependent branch and its only waits are the explicit ones on the direct loads,
// so a super tile's loads stay in flight while the previous one is multiplied.  The
// waves' sums are added through LDS in wave order; with a block-level K split, fp32
// partials go to gemm_skinny_reduce.
constexpr int kDecRows = 16;
constexpr int kDecDepth = 2;                  // LDS slots (super tiles in flight) per wave
constexpr int kDecSlot = 2 * 2048 + 2 * 256;  // B lines, A lines (kA16: a16 rows), B and A scale words

__device__ __forceinline__ int dec_swz(int r) { return (r >> 1) & 7; }

// One direct global -> LDS load per lane (16 or 4 bytes; lane l lands at dst + l * bytes;
// dst is wave-uniform and goes to M0).  Written as inline asm so that the compiler does
// not track these loads: it would otherwise make every LDS read of the ring wait for all
// of them (it cannot tell the slots apart across loop iterations).  The kernel waits for
// them itself (dec_wait_*), and nothing else in it uses M0.
__device__ __forceinline__ void dec_dma16(const uint8_t* src, uint8_t* dst) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"((uint32_t)(uintptr_t)dst), "v"(src) : "memory");
}
__device__ __forceinline__ void dec_dma4(const uint8_t* src, uint8_t* dst) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"((uint32_t)(uintptr_t)dst), "v"(src) : "memory");
}
// Waits until at most one super tile's kLoads direct loads (the newer one) are in
// flight; the compiler moves no memory access across it.
template <int kLoads>
__device__ __forceinline__ void dec_wait_one_behind() {
  static_assert(kDecDepth == 2 && (kLoads == 5 || kLoads == 6), "wait count");
  if constexpr (kLoads == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
}
__device__ __forceinline__ void dec_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void dec_lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// kA16: the activation arrives as its fp16 operand form a16 [m][k] (m <= 4) instead of
// codes and scales.  A slot then holds rows 0 .. 3 (clamped to m - 1) of a16 for the
// super tile, 512 bytes each, 16-byte chunk c of row r at position c ^ r (the 16 lanes
// that read one chunk of rows l16 % 4 hit four distinct bank groups), and the kernel
// expands only the weight.  MFMA rows 4 .. 15 multiply rows l16 % 4 again, into output
// rows that are never written.
template <bool kA16>
__global__ void __launch_bounds__(256) gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m, int64_t k,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int64_t n,
    const float* __restrict__ gsf_a, const float* __restrict__ gsf_b, int64_t a_seg_rows,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int splits, float* __restrict__ partial,
    const uint16_t* __restrict__ a16) {
  constexpr int kLoads = kA16 ? 5 : 6;   // direct-load instructions per super tile and wave
  __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][kDecDepth][kDecSlot];
  __shared__ float red[kWaves - 1][4][64];

  const int tile = blockIdx.x / splits;
  const int split = blockIdx.x % splits;
  const int64_t n0 = (int64_t)tile * kDecRows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: K range, LDS slots
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int64_t half_k = k / 2;
  const int64_t kt_all = (k + BK - 1) / BK;
  const int64_t st_all = (kt_all + 1) / 2;
  const int64_t b0 = st_all * split / splits, b1 = st_all * (split + 1) / splits;
  const int64_t s0 = b0 + (b1 - b0) * wave / kWaves, s1 = b0 + (b1 - b0) * (wave + 1) / kWaves;
  const int count = (int)(s1 - s0);

  // Direct-load sources.  Lines: lane l -> row lr (+ 8 for the second instruction) at
  // position p, i.e. logical chunk p ^ dec_swz(row).  Scale words: lane l -> word l % 2
  // of row (l % 32) / 2 in K tile 2 st + l / 32 (128 bytes per operand and K tile).
  const int lr = lane >> 3, p = lane & 7;
  const int lc0 = p ^ dec_swz(lr), lc1 = p ^ dec_swz(lr + 8);
  const uint8_t* bl0 = b_codes + min(n0 + lr, n - 1) * half_k + 16 * lc0;
  const uint8_t* bl1 = b_codes + min(n0 + lr + 8, n - 1) * half_k + 16 * lc1;
  const uint8_t* al0 = a_codes + min((int64_t)lr, m - 1) * half_k + 16 * lc0;
  const uint8_t* al1 = a_codes + min((int64_t)lr + 8, m - 1) * half_k + 16 * lc1;
  const int sr = (lane & 31) >> 1, sh = lane >> 5;
  const uint8_t* bsl = b_scales + min(n0 + sr, n - 1) * 8 + 4 * (lane & 1);
  const uint8_t* asl = kA16 ? nullptr : a_scales + min((int64_t)sr, m - 1) * 8 + 4 * (lane & 1);
  // a16 lines: instruction h, lane l -> row 2 h + l / 32, position l % 32, logical chunk
  // (l % 32) ^ row of the super tile's 256 values
  const int ar0 = lane >> 5, ar1 = 2 + (lane >> 5), ap = lane & 31;
  const int ac0 = ap ^ ar0, ac1 = ap ^ ar1;
  const uint16_t* xl0 = kA16 ? a16 + min((int64_t)ar0, m - 1) * k + 8 * ac0 : nullptr;
  const uint16_t* xl1 = kA16 ? a16 + min((int64_t)ar1, m - 1) * k + 8 * ac1 : nullptr;

  // Loads super tile st into a slot.  Super tiles past the wave's range re-load the last
  // one (the slot is never multiplied); chunks past the end of a row (partial last super
  // tile) re-load the row's first chunk, whose block scales there are the zero padding
  // of the scale layout; the K tile past an odd count of K tiles re-loads the last one's
  // scale words, and the lanes that own it use zero scales instead (multiply).
  auto issue = [&](int64_t st, uint8_t* slot) {
    st = min(st, st_all - 1);
    const int64_t off = st * 128;
    const int64_t o0 = off + 16 * lc0 < half_k ? off : -16 * lc0;
    const int64_t o1 = off + 16 * lc1 < half_k ? off : -16 * lc1;
    dec_dma16(bl0 + o0, slot);
    dec_dma16(bl1 + o1, slot + 1024);
    if (kA16) {
      // values past the end of a row re-load the row's first chunk (zero weight scales)
      const int64_t e = st * 256;
      dec_dma16(reinterpret_cast<const uint8_t*>(xl0 + (e + 8 * ac0 < k ? e : -8 * ac0)), slot + 2048);
      dec_dma16(reinterpret_cast<const uint8_t*>(xl1 + (e + 8 * ac1 < k ? e : -8 * ac1)), slot + 3072);
    } else {
      dec_dma16(al0 + o0, slot + 2048);
      dec_dma16(al1 + o1, slot + 3072);
    }
    const int64_t kt = min(2 * st + sh, kt_all - 1);
    dec_dma4(bsl + kt * n * 8, slot + 4096);
    if (!kA16) dec_dma4(asl + kt * m * 8, slot + 4096 + 256);
  };

  float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Multiplies the super tile st held in a slot: lane (l16, g) takes bytes 32 g .. +31 of
  // weight row l16 and activation row l16, and the scale word of K tile 2 st + g / 2.
  auto multiply = [&](const uint8_t* slot, int64_t st) {
    const int p0 = (2 * g) ^ dec_swz(l16), p1 = (2 * g + 1) ^ dec_swz(l16);
    const uint4 w0 = *reinterpret_cast<const uint4*>(slot + l16 * 128 + 16 * p0);
    const uint4 w1 = *reinterpret_cast<const uint4*>(slot + l16 * 128 + 16 * p1);
    const uint4 x0 = *reinterpret_cast<const uint4*>(slot + 2048 + l16 * 128 + 16 * p0);
    const uint4 x1 = *reinterpret_cast<const uint4*>(slot + 2048 + l16 * 128 + 16 * p1);
    const int so = (g >> 1) * 128 + l16 * 8 + 4 * (g & 1);
    const uint32_t keep = 2 * st + (g >> 1) < kt_all ? ~0u : 0u;   // K tile exists
    const uint32_t bs = *reinterpret_cast<const uint32_t*>(slot + 4096 + so) & keep;
    const uint32_t as = kA16 ? 0u : *reinterpret_cast<const uint32_t*>(slot + 4096 + 256 + so) & keep;
    const int xr = l16 & 3;   // kA16: the a16 row this lane reads
#pragma unroll
    for (int s = 0; s < 8; ++s) {                     // K values [64g + 8s, +8): block s/2
      const half8_t fb = dequant8(word(s < 4 ? w0 : w1, s & 3), scale_pair(bs, s >> 1));
      const half8_t fa =
          kA16 ? *reinterpret_cast<const half8_t*>(slot + 2048 + xr * 512 + 16 * ((8 * g + s) ^ xr))
               : dequant8(word(s < 4 ? x0 : x1, s & 3), scale_pair(as, s >> 1));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb, acc, 0, 0, 0);
    }
  };

  // Super tiles s0 + i and s0 + i + 1 from slots sa and sb.  Each slot is refilled as
  // soon as it has been multiplied, so one super tile's loads are in flight while the
  // other is multiplied.  The loop body has no branch; an odd last super tile is
  // multiplied after the loop.
  auto pair = [&](uint8_t* sa, uint8_t* sb, int i) __attribute__((always_inline)) {
    dec_wait_one_behind<kLoads>();          // super tile s0 + i has landed
    multiply(sa, s0 + i);
    dec_lds_order();                // its reads are done before the slot is refilled
    issue(s0 + i + 2, sa);
    dec_wait_one_behind<kLoads>();
    multiply(sb, s0 + i + 1);
    dec_lds_order();
    issue(s0 + i + 3, sb);
  };
  issue(s0, ring[wave][0]);
  issue(s0 + 1, ring[wave][1]);
  int i = 0;
  for (; i + 1 < count; i += 2) pair(ring[wave][0], ring[wave][1], i);
  if (i < count) {
    dec_wait_one_behind<kLoads>();
    multiply(ring[wave][0], s0 + i);
  }
  dec_wait_all();                   // nothing still landing in this wave's slots

  // Sum the four waves' K quarters in wave order: ((w0 + w1) + w2) + w3.
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave - 1][e][lane] = acc[e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += red[w][e][lane];

  // 16x16 MFMA output: lane holds column l16, rows 4g .. 4g+3.
  const int64_t col = n0 + l16;
  if (col >= n) return;
  const float alpha = __fdiv_rn(1.0f, __fmul_rn(*gsf_a, *gsf_b));   // one activation scale
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t row = 4 * g + e;
    if (row >= m) continue;
    if (splits > 1) {
      partial[((int64_t)split * m + row) * n + col] = acc[e];
    } else {
      const float al = a_seg_rows > 0 ? alpha_for(gsf_a, gsf_b, a_seg_rows, row) : alpha;
      uint32_t y = f32_to_bf16(__fmul_rn(al, __fmul_rn(acc[e], kAccUnscale)));
      if (bias != nullptr) y = add_bias_bf16(y, bias[col]);
      out[row * n + col] = (uint16_t)y;
    }
  }
}

// K splits of gemm_decode_kernel: enough blocks for two per compute unit, each wave
// keeping at least two super tiles.
int decode_splits(int64_t k, int64_t n, int cus) {
  const int64_t tiles = (n + kDecRows - 1) / kDecRows;
  const int64_t st = ((k + BK - 1) / BK + 1) / 2;
  int64_t sp = (2 * cus + tiles - 1) / tiles;
  const int64_t max_sp = st / (2 * kWaves) > 0 ? st / (2 * kWaves) : 1;
  if (sp > max_sp) sp = max_sp;
  return (int)(sp < 1 ? 1 : sp);
}

template <int MT, bool kFusedA = false>
hipError_t launch_mt(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k, const uint8_t* b_codes,
                     const uint8_t* b_scales, int64_t n, const float* gsf_a, const float* gsf_b, const uint16_t* bias,
                     int64_t a_seg_rows, uint16_t* out, int splits, float* partial, hipStream_t s,
                     const uint16_t* a_bf16 = nullptr) {
  const int64_t groups = (n + kCols - 1) / kCols;
  hipLaunchKernelGGL((gemm_skinny_kernel<MT, kFusedA>), dim3((uint32_t)(groups * splits)), dim3(256), 0, s, a_bf16,
                     a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, splits,
                     partial);
  return hipGetLastError();
}

}  // namespace

bool linear_skinny_fused_supported(int64_t m, int64_t k, int64_t n, const void* x, const void* b_codes,
                                   const void* b_scales, int cus) {
  const int64_t st_all = ((k + BK - 1) / BK + 1) / 2;
  const int sp = skinny_splits(k, n, cus);
  const int64_t range = (st_all + sp - 1) / sp;     // super tiles a block stages
  // staging costs about one 16-block per thread and row on the critical path: worth it
  // while it stays within two per thread (measured: one row gains a launch, 16 rows lose),
  // and only for small weights: on larger ones the streaming of gemm_decode_kernel gains
  // more than the launch (measured, one row: k_proj 8.3 vs 9.0 us, q_proj 13.3 vs 11.8 us)
  return m >= 1 && m <= 16 && k % 32 == 0 && (((uintptr_t)x | (uintptr_t)b_codes) & 15) == 0 &&
         ((uintptr_t)b_scales & 3) == 0 && range <= kFusedMaxSt && m * range * 16 <= 2 * 256 &&
         n * k <= ((int64_t)1 << 23);
}

hipError_t launch_linear_skinny_fused(const uint16_t* x, int64_t m, int64_t k, const uint8_t* b_codes,
                                      const uint8_t* b_scales, int64_t n, const float* gsf_x, const float* gsf_w,
                                      const uint16_t* bias, uint16_t* out, void* workspace, size_t workspace_bytes,
                                      int cus, hipStream_t s) {
  // the K range each block stages must fit its LDS: without the workspace for the
  // planned split the caller takes the two-pass path
  const int splits = skinny_splits(k, n, cus);
  const size_t need = splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return hipErrorInvalidValue;
  float* partial = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  hipError_t e = launch_mt<1, true>(nullptr, nullptr, m, k, b_codes, b_scales, n, gsf_x, gsf_w, bias, 0, out, splits,
                                    partial, s, x);
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(gemm_skinny_reduce, dim3((uint32_t)((m * n + 255) / 256)), dim3(256), 0, s, partial, splits, m,
                     n, gsf_x, gsf_w, (int64_t)0, bias, out);
  return hipGetLastError();
}

bool gemm_skinny_supported(int64_t m, int64_t k, const void* a_codes, const void* a_scales, const void* b_codes,
                           const void* b_scales) {
  return m <= 128 && (k / 2) % 16 == 0 && (((uintptr_t)a_codes | (uintptr_t)b_codes) & 15) == 0 &&
         (((uintptr_t)a_scales | (uintptr_t)b_scales) & 3) == 0;
}

size_t gemm_skinny_workspace_bytes(int64_t m, int64_t k, int64_t n, int cus) {
  // m <= 16 also covers the static-scale fused launch, which splits like gemm_skinny_kernel
  int64_t sp = skinny_splits(k, n, cus);
  if (m <= 16) sp = std::max<int64_t>(sp, decode_splits(k, n, cus));
  return sp > 1 ? (size_t)sp * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                              const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                              void* workspace, size_t workspace_bytes, int cus, hipStream_t s) {
  int splits = m <= 16 ? decode_splits(k, n, cus) : skinny_splits(k, n, cus);
  const size_t need = splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) splits = 1;
  float* partial = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  hipError_t e;
  if (m <= 16) {
    const int64_t tiles = (n + kDecRows - 1) / kDecRows;
    hipLaunchKernelGGL(gemm_decode_kernel<false>, dim3((uint32_t)(tiles * splits)), dim3(256), 0, s, a_codes,
                       a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, splits, partial,
                       (const uint16_t*)nullptr);
    e = hipGetLastError();
  } else if (m <= 32) {
    e = launch_mt<2>(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, bias, a_seg_rows, out, splits, partial, s);
  } else if (m <= 64) {
    e = launch_mt<4>(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, bias, a_seg_rows, out, splits, partial, s);
  } else {
    e = launch_mt<8>(a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, bias, a_seg_rows, out, splits, partial, s);
  }
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = m * n;
  hipLaunchKernelGGL(gemm_skinny_reduce, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, s, partial, splits, m,
                     n, gsf_a, gsf_b, a_seg_rows, bias, out);
  return hipGetLastError();
}

bool gemm_decode_a16_supported(int64_t m, int64_t k, const void* a16, const void* b_codes, const void* b_scales) {
  return m >= 1 && m <= kDecodeA16Rows && k % 32 == 0 && (((uintptr_t)a16 | (uintptr_t)b_codes) & 15) == 0 &&
         ((uintptr_t)b_scales & 3) == 0;
}

hipError_t launch_gemm_decode_a16(const uint16_t* a16, int64_t m, int64_t k, const uint8_t* b_codes,
                                  const uint8_t* b_scales, int64_t n, const float* gsf_a, const float* gsf_b,
                                  const uint16_t* bias, uint16_t* out, void* workspace, size_t workspace_bytes,
                                  int cus, hipStream_t s) {
  int splits = decode_splits(k, n, cus);
  const size_t need = splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) splits = 1;
  float* partial = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  const int64_t tiles = (n + kDecRows - 1) / kDecRows;
  hipLaunchKernelGGL(gemm_decode_kernel<true>, dim3((uint32_t)(tiles * splits)), dim3(256), 0, s,
                     (const uint8_t*)nullptr, (const uint8_t*)nullptr, m, k, b_codes, b_scales, n, gsf_a, gsf_b,
                     (int64_t)0, bias, out, splits, partial, a16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = m * n;
  hipLaunchKernelGGL(gemm_skinny_reduce, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, s, partial, splits, m,
                     n, gsf_a, gsf_b, (int64_t)0, bias, out);
  return hipGetLastError();
}

}  // namespace nvfp4
