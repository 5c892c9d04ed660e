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

template <int MT>   // M tiles of 16 rows
__global__ void __launch_bounds__(256) gemm_skinny_kernel(
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
    arow[i] = a_codes + r * half_k;
    asrow[i] = a_scales + r * 8 + 4 * (g & 1);
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
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      T.ac[i][0] = c0 ? *reinterpret_cast<const uint4*>(arow[i] + off) : make_uint4(0, 0, 0, 0);
      T.ac[i][1] = c1 ? *reinterpret_cast<const uint4*>(arow[i] + off + 16) : make_uint4(0, 0, 0, 0);
      T.as[i] = sv ? *reinterpret_cast<const uint32_t*>(asrow[i] + kt * m * 8) : 0u;
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
  if (st < st_end) {
    fetch(st, cur);
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
// whose 256-wide super tiles its waves (four or eight) split into consecutive ranges.
// Each wave streams its range through a ring of kDecDepth LDS slots with direct
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
// them itself (dec_wait, dec_wait_all).  The LDS address is an M0 input operand, so the compiler
// itself sets M0 and knows what it holds.
__device__ __forceinline__ void dec_dma16(const uint8_t* src, uint8_t* dst) {
  asm volatile("global_load_lds_dwordx4 %1, off" :: "{m0}"((uint32_t)(uintptr_t)dst), "v"(src) : "memory");
}
__device__ __forceinline__ void dec_dma4(const uint8_t* src, uint8_t* dst) {
  asm volatile("global_load_lds_dword %1, off" :: "{m0}"((uint32_t)(uintptr_t)dst), "v"(src) : "memory");
}
// Waits until at most one super tile's kCount direct loads (the newer one) are in
// flight; the compiler moves no memory access across it.
template <int kCount>
__device__ __forceinline__ void dec_wait() {
  static_assert(kDecDepth == 2 && (kCount == 3 || kCount == 5 || kCount == 6), "wait count");
  if constexpr (kCount == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if constexpr (kCount == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
}
__device__ __forceinline__ void dec_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void dec_lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// kA16: the activation arrives as its fp16 operand form a16 [m][k] (m <= 4) instead of
// codes and scales.  A slot then holds rows 0 .. 3 (clamped to m - 1) of a16 for the
// super tile, 512 bytes each, 16-byte chunk c of row r at position c ^ r (the 16 lanes
// that read one chunk of rows l16 % 4 hit four distinct bank groups), and the kernel
// expands only the weight.  MFMA rows 4 .. 15 multiply rows l16 % 4 again, into output
// rows that are never written.
//
// kDW: waves per block (4 or 8).  Eight waves split the block's K range eight ways, which
// takes the place of a two-way block-level K split: the partial sums meet in LDS and the
// second launch (gemm_skinny_reduce) is not needed.
//
// kOne (m == 1): the slot carries the one activation row only (512 bytes: the row's 256
// fp16 values, or its 128 code bytes and 16 scale bytes), 2816 bytes in all instead of
// 4608, so seven four-wave blocks fit a compute unit's LDS instead of four.
//
// kFuse (with kA16 and kOne: the linear at one row): a16 points at the bf16 row x itself.
// kFuseStatic: gsf_a points at its static global scale.  kFuseDynamic: every block forms
// the dynamic scale itself from the abs-max of the whole row (read from L2; the same
// value in every block).  Block 0 stores the scale used to gsf_dst unless that is NULL;
// the epilogue, or the split-K reduce (from gsf_dst), applies it.  Each wave loads its K
// range of x (fuse_max_st super tiles at most) into its own LDS region by direct loads
// and turns it there into the fp16 operand form with the quantize kernels' block
// encoder, bit for bit what the quantize pass would have written; the slots then carry
// only the weight (2304 bytes).  The linear is one launch instead of two.
//
// Four waves per SIMD (seven for four-wave blocks with kOne, five with kFuse) bound the
// registers.
//
// Super tiles of x one wave quantizes: its region is 512 bytes each.  Five four-wave
// blocks (six super tiles) or two eight-wave blocks (eight) fit a compute unit's LDS.
constexpr int fuse_max_st(int waves) { return waves == 8 ? 8 : 6; }
constexpr int kFuseStatic = 1, kFuseDynamic = 2;
template <bool kA16, int kDW, bool kOne, int kFuse = 0>
__global__ void __launch_bounds__(64 * kDW)
__attribute__((amdgpu_waves_per_eu(kFuse && kDW == 4 ? 5 : kOne && kDW == 4 ? 7 : 4))) gemm_decode_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m, int64_t k,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int64_t n,
    const float* __restrict__ gsf_a, const float* __restrict__ gsf_b, int64_t a_seg_rows,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int splits, float* __restrict__ partial,
    const uint16_t* __restrict__ a16, float* __restrict__ gsf_dst) {
  // direct-load instructions per super tile and wave; bytes per slot and where the
  // weight's scale words sit in it
  constexpr int kLoads = kFuse ? 3 : kOne || kA16 ? 5 : 6;
  constexpr int kSlot = kFuse ? 2048 + 256 : kOne ? 2048 + 512 + 256 : kDecSlot;
  constexpr int kOffBS = kFuse ? 2048 : kOne ? 2560 : 4096;
  static_assert(kDW == 4 || kDW == 8, "waves per block");
  static_assert(!kFuse || (kA16 && kOne), "the fused row is a one-row fp16 operand");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kDW][kDecDepth][kSlot];
  __shared__ __attribute__((aligned(16))) uint8_t arow[kFuse ? kDW : 1][kFuse ? fuse_max_st(kDW) * 512 : 16];

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
  const int64_t s0 = b0 + (b1 - b0) * wave / kDW, s1 = b0 + (b1 - b0) * (wave + 1) / kDW;
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
  // kOne: 4-byte pieces of row 0 in K order.  a16: lane l takes values 2 l, 2 l + 1 and
  // 128 + 2 l, 129 + 2 l of the super tile; codes: lane l takes bytes 4 (l % 32) .. + 3 of
  // its line (lanes 32 .. 63 repeat lanes 0 .. 31) and scale word l % 4 (K tile
  // 2 st + (l % 4) / 2, word l % 2).
  const int sw4 = lane & 3;

  // Loads super tile st into a slot.  Super tiles past the wave's range re-load the
  // wave's own last one (the slot is never multiplied; those lines are still in L2,
  // while the next wave's first ones would come from HBM a second time); chunks past the
  // end of a row (partial last super tile) re-load the row's first chunk, whose block
  // scales there are the zero padding of the scale layout; the K tile past an odd count
  // of K tiles re-loads the last one's scale words, and the lanes that own it use zero
  // scales instead (multiply).
  const int64_t st_last = min(max(s1 - 1, s0), st_all - 1);
  auto issue = [&](int64_t st, uint8_t* slot) {
    st = min(st, st_last);
    const int64_t off = st * 128;
    const int64_t o0 = off + 16 * lc0 < half_k ? off : -16 * lc0;
    const int64_t o1 = off + 16 * lc1 < half_k ? off : -16 * lc1;
    dec_dma16(bl0 + o0, slot);
    dec_dma16(bl1 + o1, slot + 1024);
    if (kFuse) {
      dec_dma4(bsl + min(2 * st + sh, kt_all - 1) * n * 8, slot + kOffBS);
      return;
    }
    if (kOne) {
      // pieces past the end of the row re-load its first one (zero weight scales there)
      const int64_t kt = min(2 * st + (sw4 >> 1), kt_all - 1);
      if (kA16) {
        const int64_t e0 = st * 256 + 2 * lane, e1 = e0 + 128;
        dec_dma4(reinterpret_cast<const uint8_t*>(a16 + (e0 < k ? e0 : 0)), slot + 2048);
        dec_dma4(reinterpret_cast<const uint8_t*>(a16 + (e1 < k ? e1 : 0)), slot + 2048 + 256);
      } else {
        const int64_t c = off + 4 * (lane & 31);
        dec_dma4(a_codes + (c < half_k ? c : 0), slot + 2048);
        dec_dma4(a_scales + kt * 8 + 4 * (sw4 & 1), slot + 2048 + 256);
      }
      dec_dma4(bsl + min(2 * st + sh, kt_all - 1) * n * 8, slot + kOffBS);
      return;
    }
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
    const int so = (g >> 1) * 128 + l16 * 8 + 4 * (g & 1);
    const uint32_t keep = 2 * st + (g >> 1) < kt_all ? ~0u : 0u;   // K tile exists
    const uint32_t bs = *reinterpret_cast<const uint32_t*>(slot + kOffBS + so) & keep;
    if constexpr (kFuse) {
      // every lane reads row 0 from the wave's quantized region
      const uint8_t* xa = arow[wave] + (st - s0) * 512 + 128 * g;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const half8_t fb = dequant8(word(s < 4 ? w0 : w1, s & 3), scale_pair(bs, s >> 1));
        const half8_t fa = *reinterpret_cast<const half8_t*>(xa + 16 * s);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb, acc, 0, 0, 0);
      }
      return;
    }
    if constexpr (kOne) {
      // every lane reads row 0: K values 64 g + 8 s .. of the super tile
      const uint4 x0 = *reinterpret_cast<const uint4*>(slot + 2048 + 32 * g);
      const uint4 x1 = *reinterpret_cast<const uint4*>(slot + 2048 + 32 * g + 16);
      const uint32_t as = kA16 ? 0u : *reinterpret_cast<const uint32_t*>(slot + 2048 + 256 + 4 * g) & keep;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const half8_t fb = dequant8(word(s < 4 ? w0 : w1, s & 3), scale_pair(bs, s >> 1));
        const half8_t fa = kA16 ? *reinterpret_cast<const half8_t*>(slot + 2048 + 128 * g + 16 * s)
                                : dequant8(word(s < 4 ? x0 : x1, s & 3), scale_pair(as, s >> 1));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb, acc, 0, 0, 0);
      }
      return;
    }
    const uint4 x0 = *reinterpret_cast<const uint4*>(slot + 2048 + l16 * 128 + 16 * p0);
    const uint4 x1 = *reinterpret_cast<const uint4*>(slot + 2048 + l16 * 128 + 16 * p1);
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

  // Super tiles s0 + i and s0 + i + 1 from slots 0 and 1.  Each slot is refilled as soon
  // as it has been multiplied, so one super tile's loads are in flight while the other
  // is multiplied.  The loop body has no branch; an odd last super tile is multiplied
  // after the loop.
  if constexpr (kFuse) {
    // the wave's K range of x as bf16 straight into its region, ahead of the weight
    // loads, two super tiles (1 KB) per load; pieces past the end of the row re-load its
    // start and are not used
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(a16);
    for (int j = 0; j < (count + 1) / 2; ++j) {
      const int64_t e = s0 * 256 + j * 512 + 8 * lane;
      dec_dma16(xb + 2 * (e < k ? e : 0), arow[wave] + j * 1024);
    }
  }
  issue(s0, ring[wave][0]);
  issue(s0 + 1, ring[wave][1]);
  float gsf_x = 0.0f;   // kFuse: the activation's global scale
  if constexpr (kFuse) {
    if constexpr (kFuse == kFuseStatic) {
      gsf_x = *gsf_a;
    } else {
      // every thread takes the abs-max of 8-value pieces of the row, then the waves'
      // maxima meet in LDS (the ordinary loads here also wait for the direct loads above)
      __shared__ float wave_amax[kDW];
      float mx = 0.0f;
      for (int64_t c = threadIdx.x; c < k / 8; c += 64 * kDW) {
        const uint4 q = *reinterpret_cast<const uint4*>(a16 + 8 * c);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx = fmaxf(mx, fabsf(__uint_as_float(w[e] << 16)));
          mx = fmaxf(mx, fabsf(__uint_as_float(w[e] & 0xFFFF0000u)));
        }
      }
      mx = wave_max(mx);
      if (lane == 0) wave_amax[wave] = mx;
      __syncthreads();
      float amax = 0.0f;
#pragma unroll
      for (int w = 0; w < kDW; ++w) amax = fmaxf(amax, wave_amax[w]);
      gsf_x = global_scale_from_amax(amax);
    }
    // x has landed once only the two super tiles' weight loads can be in flight; each
    // lane then turns 16-value blocks of it into their fp16 operand form in place (a
    // block's 32 bf16 bytes become its 32 fp16 bytes); blocks past the end of the row
    // are zero
    dec_wait<2 * kLoads>();
    const int blocks = count * 16;
#pragma unroll
    for (int h = 0; h < (fuse_max_st(kDW) * 16 + 63) / 64; ++h) {
      const int b = h * 64 + lane;
      if (b < blocks) {
        uint8_t* blk = arow[wave] + 32 * b;
        const bool valid = s0 * 256 + (int64_t)b * 16 < k;
        float v[16];
        if (valid) {
          load16_bf16(reinterpret_cast<const uint16_t*>(blk), v);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = 0.0f;
        }
        uint32_t c0, c1;
        const uint32_t s8 = quantize_block16(v, gsf_x, valid, c0, c1);
        const half2_t sc = as_half2((s8 << 7) | (s8 << 23));
        uint4* d = reinterpret_cast<uint4*>(blk);
        d[0] = __builtin_bit_cast(uint4, dequant8(c0, sc));
        d[1] = __builtin_bit_cast(uint4, dequant8(c1, sc));
      }
    }
  }
  int i = 0;
  for (; i + 1 < count; i += 2) {
    dec_wait<kLoads>();                  // super tile s0 + i has landed
    multiply(ring[wave][0], s0 + i);
    dec_lds_order();                     // its reads are done before the slot is refilled
    issue(s0 + i + 2, ring[wave][0]);
    dec_wait<kLoads>();
    multiply(ring[wave][1], s0 + i + 1);
    dec_lds_order();
    issue(s0 + i + 3, ring[wave][1]);
  }
  if (i < count) {
    dec_wait<kLoads>();
    multiply(ring[wave][0], s0 + i);
  }
  dec_wait_all();                   // nothing still landing in this wave's slots

  // Sum the waves' K ranges in wave order: ((w0 + w1) + w2) + ...  Each wave hands its
  // sums over in its own first slot, which no load writes any more.
  float* red = reinterpret_cast<float*>(ring[wave][0]);
  if (wave > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[e * 64 + lane] = acc[e];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kDW; ++w) {
    const float* rw = reinterpret_cast<const float*>(ring[w][0]);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += rw[e * 64 + lane];
  }

  // 16x16 MFMA output: lane holds column l16, rows 4g .. 4g+3.
  const int64_t col = n0 + l16;
  if (col >= n) return;
  if (kFuse && gsf_dst != nullptr && blockIdx.x == 0 && lane == 0) *gsf_dst = gsf_x;
  const float alpha = __fdiv_rn(1.0f, __fmul_rn(kFuse ? gsf_x : *gsf_a, *gsf_b));   // one activation scale
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

// Launch shape of gemm_decode_kernel.  Aim: enough four-wave blocks for two per compute
// unit, each wave keeping at least two super tiles.  Where that takes a K split and the
// rows are short (K <= 16384: at most 8 super tiles per wave of an eight-wave block),
// eight-wave blocks halve the split, which saves the reduce launch at a two-way split
// (measured, one row: o_proj 11.0 -> 10.0 us, k_proj 5.8 -> 4.9 us).  On longer rows the
// fewer, longer blocks leave the compute units unevenly loaded (down_proj, K = 25600:
// 22.0 -> 23.1 us), so those keep four waves.
struct DecodePlan {
  int waves;
  int splits;
};
DecodePlan decode_plan(int64_t k, int64_t n, int cus) {
  const int64_t tiles = (n + kDecRows - 1) / kDecRows;
  const int64_t st = ((k + BK - 1) / BK + 1) / 2;
  int64_t sp = (2 * cus + tiles - 1) / tiles;
  const int64_t max_sp = st / (2 * 4) > 0 ? st / (2 * 4) : 1;
  if (sp > max_sp) sp = max_sp;
  if (sp < 2) return {4, 1};
  if (st > 64) return {4, (int)sp};
  return {8, (int)(sp / 2)};
}

template <bool kA16, int kDW, bool kOne, int kFuse = 0>
void launch_decode_t(dim3 grid, hipStream_t s, const uint8_t* a_codes, const uint8_t* a_scales, int64_t m,
                     int64_t k, const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                     const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out, int splits,
                     float* partial, const uint16_t* x16, float* gsf_dst) {
  hipLaunchKernelGGL((gemm_decode_kernel<kA16, kDW, kOne, kFuse>), grid, dim3(64 * kDW), 0, s, a_codes, a_scales, m, k,
                     b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, splits, partial, x16, gsf_dst);
}

hipError_t launch_decode(bool a16, int fuse, int waves, uint32_t blocks, hipStream_t s, const uint8_t* a_codes,
                         const uint8_t* a_scales, int64_t m, int64_t k, const uint8_t* b_codes,
                         const uint8_t* b_scales, int64_t n, const float* gsf_a, const float* gsf_b,
                         int64_t a_seg_rows, const uint16_t* bias, uint16_t* out, int splits, float* partial,
                         const uint16_t* x16, float* gsf_dst = nullptr) {
#ifndef NVFP4_DECODE_ONE_ROW
#define NVFP4_DECODE_ONE_ROW 1
#endif
  const bool one = NVFP4_DECODE_ONE_ROW && m == 1;
  using Launch = decltype(&launch_decode_t<false, 4, false>);
  // [activation form][one row][eight waves]; the fused forms are one-row fp16 only
  static constexpr Launch kPlain[2][2][2] = {
      {{launch_decode_t<false, 4, false>, launch_decode_t<false, 8, false>},
       {launch_decode_t<false, 4, true>, launch_decode_t<false, 8, true>}},
      {{launch_decode_t<true, 4, false>, launch_decode_t<true, 8, false>},
       {launch_decode_t<true, 4, true>, launch_decode_t<true, 8, true>}}};
  static constexpr Launch kFused[2][2] = {
      {launch_decode_t<true, 4, true, kFuseStatic>, launch_decode_t<true, 8, true, kFuseStatic>},
      {launch_decode_t<true, 4, true, kFuseDynamic>, launch_decode_t<true, 8, true, kFuseDynamic>}};
  const int w8 = waves == 8 ? 1 : 0;
  const Launch fn = fuse != 0 ? kFused[fuse == kFuseDynamic ? 1 : 0][w8] : kPlain[a16 ? 1 : 0][one ? 1 : 0][w8];
  fn(dim3(blocks), s, a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, splits,
     partial, x16, gsf_dst);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k, const uint8_t* b_codes,
                     const uint8_t* b_scales, int64_t n, const float* gsf_a, const float* gsf_b, const uint16_t* bias,
                     int64_t a_seg_rows, uint16_t* out, int splits, float* partial, hipStream_t s) {
  const int64_t groups = (n + kCols - 1) / kCols;
  hipLaunchKernelGGL((gemm_skinny_kernel<MT>), dim3((uint32_t)(groups * splits)), dim3(256), 0, s, a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, splits,
                     partial);
  return hipGetLastError();
}

}  // namespace

bool gemm_skinny_supported(int64_t m, int64_t k, const void* a_codes, const void* a_scales, const void* b_codes,
                           const void* b_scales) {
  return m <= 128 && (k / 2) % 16 == 0 && (((uintptr_t)a_codes | (uintptr_t)b_codes) & 15) == 0 &&
         (((uintptr_t)a_scales | (uintptr_t)b_scales) & 3) == 0;
}

size_t gemm_skinny_workspace_bytes(int64_t m, int64_t k, int64_t n, int cus) {
  // up to 16 rows gemm_decode_kernel runs, split by its own plan
  const int64_t sp = m <= 16 ? decode_plan(k, n, cus).splits : skinny_splits(k, n, cus);
  return sp > 1 ? (size_t)sp * (size_t)m * (size_t)n * sizeof(float) : 0;
}

hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                              const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                              void* workspace, size_t workspace_bytes, int cus, hipStream_t s) {
  const DecodePlan plan = decode_plan(k, n, cus);
  int splits = m <= 16 ? plan.splits : skinny_splits(k, n, cus);
  const size_t need = splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) splits = 1;
  float* partial = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  hipError_t e;
  if (m <= 16) {
    const int64_t tiles = (n + kDecRows - 1) / kDecRows;
    e = launch_decode(false, 0, plan.waves, (uint32_t)(tiles * splits), s, a_codes, a_scales, m, k, b_codes, b_scales,
                      n, gsf_a, gsf_b, a_seg_rows, bias, out, splits, partial, nullptr);
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
  const DecodePlan plan = decode_plan(k, n, cus);
  int splits = plan.splits;
  const size_t need = splits > 1 ? (size_t)splits * (size_t)m * (size_t)n * sizeof(float) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) splits = 1;
  float* partial = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  const int64_t tiles = (n + kDecRows - 1) / kDecRows;
  hipError_t e = launch_decode(true, 0, plan.waves, (uint32_t)(tiles * splits), s, nullptr, nullptr, m, k,
                               b_codes, b_scales, n, gsf_a, gsf_b, 0, bias, out, splits, partial, a16);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = m * n;
  hipLaunchKernelGGL(gemm_skinny_reduce, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, s, partial, splits, m,
                     n, gsf_a, gsf_b, (int64_t)0, bias, out);
  return hipGetLastError();
}

namespace {
// The split a one-row fused launch takes with this workspace.
int fused_splits(int64_t k, int64_t n, size_t workspace_bytes, int cus, int& waves) {
  const DecodePlan plan = decode_plan(k, n, cus);
  waves = plan.waves;
  int splits = plan.splits;
  if (splits > 1 && workspace_bytes < (size_t)splits * (size_t)n * sizeof(float)) splits = 1;
  return splits;
}
}  // namespace

bool linear_decode_fused_supported(int64_t m, int64_t k, int64_t n, bool dynamic, const void* x,
                                   const void* b_codes, const void* b_scales, size_t workspace_bytes, int cus) {
  if (m != 1 || k % 32 != 0 || (((uintptr_t)x | (uintptr_t)b_codes) & 15) != 0 || ((uintptr_t)b_scales & 3) != 0)
    return false;
  // Every block of the dynamic form reads the whole row for its abs-max before its K
  // loop starts: on large weights (many blocks, or long rows) that costs more than the
  // separate single-launch quantize (measured, one row: gate_proj 25600 x 5120 20.8 vs
  // 19.2 us, down_proj 5120 x 25600 23.3 vs 23.3; k_proj 1024 x 5120 5.5 vs 7.4, q_proj
  // 8192 x 5120 8.6 vs 9.8, o_proj 5120 x 8192 9.95 vs 11.6).
  if (dynamic && n * k > ((int64_t)1 << 26)) return false;
  int waves;
  const int splits = fused_splits(k, n, workspace_bytes, cus, waves);
  const int64_t st_all = ((k + BK - 1) / BK + 1) / 2;
  const int64_t per_block = (st_all + splits - 1) / splits;
  return (per_block + waves - 1) / waves <= fuse_max_st(waves);   // every wave's range fits its region
}

hipError_t launch_linear_decode_fused(const uint16_t* x, int64_t k, const uint8_t* b_codes, const uint8_t* b_scales,
                                      int64_t n, const float* gsf_x, float* gsf_used, const float* gsf_w,
                                      const uint16_t* bias, uint16_t* out, void* workspace, size_t workspace_bytes,
                                      int cus, hipStream_t s) {
  if (gsf_x == nullptr && gsf_used == nullptr) return hipErrorInvalidValue;   // the reduce reads the scale there
  int waves;
  const int splits = fused_splits(k, n, workspace_bytes, cus, waves);
  float* partial = splits > 1 ? static_cast<float*>(workspace) : nullptr;
  const int64_t tiles = (n + kDecRows - 1) / kDecRows;
  hipError_t e = launch_decode(true, gsf_x != nullptr ? kFuseStatic : kFuseDynamic, waves, (uint32_t)(tiles * splits), s, nullptr, nullptr, 1, k, b_codes,
                               b_scales, n, gsf_x, gsf_w, 0, bias, out, splits, partial, x, gsf_used);
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(gemm_skinny_reduce, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, partial, splits,
                     (int64_t)1, n, gsf_x != nullptr ? gsf_x : gsf_used, gsf_w, (int64_t)0, bias, out);
  return hipGetLastError();
}

}  // namespace nvfp4
