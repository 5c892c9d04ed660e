// Large-problem NVFP4 GEMM on gfx950: the same product as gemm.hip, tuned for
// problems with at least one 256 x 256 output tile per compute unit.
//
//   out[i, j] = bf16( alpha * sum_b sx[i,b] sw[j,b] sum_{k in b} qx[i,k] qw[j,k] ),
//   then out = bf16(out + bias[j])
// ("minimax_h3_nvfp4_decoder" page, nvfp4_linear_inference: mm_fp4 with
// alpha = 1/(global_sf_x*global_sf_w), then the bias add).
//
// One 256-thread workgroup per 256 x 256 tile, one wave per SIMD, each wave 128 x 128
// (4 x 4 v_mfma_f32_32x32x16_f16 tiles, accumulators in AGPRs).  Expansion of the
// packed operands to fp16 (gemm_common.h) happens in registers, interleaved with the
// MFMAs of the previous sub-step, so the matrix core is fed continuously:
//
//   * codes go global -> LDS directly (global_load_lds_dwordx4), no register staging;
//     a 64-byte row of a K tile is four 16-byte chunks, chunk c of row r stored at
//     slot c ^ (((r >> 1) ^ (r >> 2)) & 3), which keeps the 16-byte LDS reads free
//     of bank conflicts;
//   * block scales (8 bytes per row per K tile) go through registers;
//   * two LDS stages; per 128-wide K tile, eight sub-steps of 16 MFMAs:
//       0, 1  -                                  2  read the second half of this tile
//       3  -                                     4  store the next tile's scales
//       -- LDS barrier: next tile complete in LDS, this tile fully read --
//       5  read the next tile's first half and scales; issue loads for tile + 2
//       6  -                                     7  expand the next tile's first step
//     every sub-step expands the fragments of the following one.
//   * rows past the end of A or B are clamped to the last row: they only feed output
//     rows / columns that are never written;
//   * tiles are numbered in bands of 4 tile rows, N-major inside a band, and each XCD
//     takes a contiguous run of numbers, so the 32 tiles resident on an XCD form a
//     4 x 8 block (12 operand panels in its L2 instead of 18 for a 16 x 2 column).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int kRows = 256;                       // rows of B (output columns) per tile
constexpr int kEpiRowBytes = 128 * 2 + 16;

// Tile geometry for kTM 32-row MFMA tiles per wave along M (2 x 2 waves): A rows per
// tile 64 * kTM (256, or 128 for few activation rows), B rows 256.  One LDS stage holds
// a K tile of both operands: A codes, B codes, A scales, B scales.
template <int kTM>
struct Geo {
  static constexpr int kRowsA = 64 * kTM;
  static constexpr int kOffB = kRowsA * 64;
  static constexpr int kOffAS = kOffB + kRows * 64;
  static constexpr int kOffBS = kOffAS + kRowsA * 8;
  static constexpr int kStage = kOffBS + kRows * 8;    // 36 KB (kTM 4) or 27 KB (kTM 2)
  static constexpr int kLds = 2 * kStage;
  static constexpr int kAcc = kTM * 64;                // accumulator entries per thread
  static_assert(4 * 32 * kEpiRowBytes <= kLds, "epilogue staging fits in the stages");
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// One 16-byte global -> LDS copy per lane.  A plain function, so that the target
// builtin is never part of a template-dependent expression.
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Tile index -> (tile row, tile column): bands of kGroupM tile rows, N-major inside a
// band, so consecutive indices (the tiles resident on one XCD at a time) cover a
// kGroupM x (32 / kGroupM) block and share operand panels in that XCD's L2.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int band = tile / (kGroupM * tiles_n);
  const int first = band * kGroupM;
  const int rows = min(tiles_m - first, kGroupM);
  const int in_band = tile - band * kGroupM * tiles_n;
  tm = first + in_band % rows;
  tn = in_band / rows;
}

// Orders this wave's LDS accesses around a point: everything before it has completed,
// and the compiler moves no memory access across it.
__device__ __forceinline__ void lds_order() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Waits for this wave's global and LDS traffic, then the workgroup barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int kMem, int kN>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int g = 0; g < kN; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
    if (kMem != 0) __builtin_amdgcn_sched_group_barrier(kMem, 1, 0);   // one memory op
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);                 // a few VALU
  }
  __builtin_amdgcn_sched_barrier(0);   // nothing crosses a sub-step boundary
}

// kSplit: the launch for the tiles past the last whole round, each split along K into
// fp32 partials (`splits` blocks per tile); otherwise whole tiles with the epilogue.
// kTM: 32-row MFMA tiles per wave along M (4: 256 x 256 tiles, 2: 128 x 256).  With
// sub = 2 (split launch of 128-row tiles only), tile indices count tiles twice as tall
// (tiles_m of that grid), each cut into two 128-row halves: tile tile0 + u / 2, half u % 2.
template <bool kSplit, int kTM>
__global__ void __launch_bounds__(256, 1) gemm_pipe_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales, int64_t m, int64_t k,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales, int64_t n,
    const float* __restrict__ gsf_a, const float* __restrict__ gsf_b, int64_t a_seg_rows,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int64_t b_srows, int64_t ldo, int tiles_m,
    int tiles_n, int tile0, int splits, int sub,
    float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  using G = Geo<kTM>;
  constexpr int kOffB = G::kOffB, kOffAS = G::kOffAS, kOffBS = G::kOffBS, kStage = G::kStage;
  // Tile indices follow tile_coords.  Without split-K, workgroups (dealt round-robin to
  // the 8 XCDs) are remapped so each XCD gets a contiguous run of tile indices, whose
  // resident tiles then share operand panels in its L2.  With split-K, block b takes K
  // range b % splits of tile b / splits.
  const int nblk = gridDim.x;
  int bid = blockIdx.x;
  int split = 0, half = 0;
  if (kSplit) {
    split = bid % splits;
    bid = bid / splits;
    half = bid % sub;
    bid = bid / sub;
  } else if ((nblk & 7) == 0) {
    bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  }
  bid += tile0;
  int tm, tn;
  tile_coords(bid, tiles_m, tiles_n, tm, tn);
  const int64_t row0 = ((int64_t)tm * sub + half) * G::kRowsA;
  const int64_t col0 = (int64_t)tn * kRows;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (LDS bases go to M0)
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31;
  const int kh = lane >> 5;
  const int64_t half_k = k / 2;
  const int64_t kt_all = (k + BK - 1) / BK;
  const int nsplit = kSplit ? splits : 1;
  const int64_t kt_begin = kt_all * split / nsplit;        // this block's K tiles
  const int64_t kt_end = kt_all * (split + 1) / nsplit;

  // Direct loads: for B, wave w, instruction i fills LDS rows 16*(4w+i) .. +15; for A,
  // rows 16*(kTM w+i) .. +15.  Lane l lands in slot (l & 3) of row (base + l/4) and so
  // fetches logical chunk (l & 3) ^ swz(row).
  const uint8_t* ag[kTM];
  const uint8_t* bg[4];
  int chunk_a[kTM], chunk_b[4];
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    const int r = 16 * (kTM * wave + i) + (lane >> 2);
    chunk_a[i] = (lane & 3) ^ swz(r);
    ag[i] = a_codes + min(row0 + r, m - 1) * half_k + 16 * chunk_a[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * (4 * wave + i) + (lane >> 2);
    chunk_b[i] = (lane & 3) ^ swz(r);
    bg[i] = b_codes + min(col0 + r, n - 1) * half_k + 16 * chunk_b[i];
  }
  // the threads that move A's scale rows: all 256 for 256-row tiles (a constant there)
  const bool a_scale_thread = G::kRowsA >= 256 || t < G::kRowsA;
  const uint8_t* asg = a_scales + min(row0 + (a_scale_thread ? t : 0), m - 1) * 8;
  const uint8_t* bsg = b_scales + min(col0 + t, n - 1) * 8;

  auto stage = [&](int64_t kt) { return lds + (int)(kt & 1) * kStage; };

  // Loads of tile kt into stage kt & 1.  Tiles past the end re-load the last tile (into
  // a stage that is never consumed), and chunks past the end of a row (last tile when
  // K % 128 != 0) re-load the row's first chunk: their block scales are the zero
  // padding of the scale layout, so whatever codes land there contribute nothing.
  // Both are selects, so the loop body has no branches.
  auto gload_codes = [&](int64_t kt) {
    uint8_t* st = stage(kt);
    const int64_t off = min(kt, kt_end - 1) * 64;
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const bool in_row = off + 16 * chunk_a[i] < half_k;
      dma16(ag[i] + (in_row ? off : -16 * chunk_a[i]), st + (kTM * wave + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in_row = off + 16 * chunk_b[i] < half_k;
      dma16(bg[i] + (in_row ? off : -16 * chunk_b[i]), st + kOffB + (4 * wave + i) * 1024);
    }
  };
  uint2 sa_reg, sb_reg;
  auto gload_scales = [&](int64_t kt) {
    const int64_t kc = min(kt, kt_end - 1);
    sa_reg = *reinterpret_cast<const uint2*>(asg + kc * m * 8);
    sb_reg = *reinterpret_cast<const uint2*>(bsg + kc * b_srows * 8);
  };
  auto sstore_scales = [&](int64_t kt) {
    uint8_t* st = stage(kt);
    if (a_scale_thread) *reinterpret_cast<uint2*>(st + kOffAS + t * 8) = sa_reg;
    *reinterpret_cast<uint2*>(st + kOffBS + t * 8) = sb_reg;
  };

  const int arow = wm * (32 * kTM) + lr;
  const int brow = wn * 128 + lr;
  auto rscale = [&](const uint8_t* st, uint32_t (&as)[kTM], uint32_t (&bs)[4]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) as[i] = *reinterpret_cast<const uint32_t*>(st + kOffAS + (arow + 32 * i) * 8 + 4 * kh);
#pragma unroll
    for (int j = 0; j < 4; ++j) bs[j] = *reinterpret_cast<const uint32_t*>(st + kOffBS + (brow + 32 * j) * 8 + 4 * kh);
  };
  // half q of the lane's 32 code bytes: logical chunk 2*kh + q
  auto rhalf = [&](const uint8_t* st, int q, uint4 (&ar)[kTM], uint4 (&br)[4]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int r = arow + 32 * i;
      ar[i] = *reinterpret_cast<const uint4*>(st + r * 64 + 16 * ((2 * kh + q) ^ swz(r)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = brow + 32 * j;
      br[j] = *reinterpret_cast<const uint4*>(st + kOffB + r * 64 + 16 * ((2 * kh + q) ^ swz(r)));
    }
  };
  auto expand = [&](const uint4 (&ar)[kTM], const uint4 (&br)[4], const uint32_t (&as)[kTM],
                    const uint32_t (&bs)[4], int step, half8_t (&fa)[kTM], half8_t (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) fa[i] = dequant8(word(ar[i], step & 3), scale_pair(as[i], step >> 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = dequant8(word(br[j], step & 3), scale_pair(bs[j], step >> 1));
  };

  // acc[i][j] is the 32 x 32 output block (rows 32 i, columns 32 j of the wave's
  // quarter), computed as the transposed product (weight fragments as the MFMA's first
  // operand): entry e of lane l is output row l % 32, column 8 (e / 4) + 4 (l / 32) + e % 4,
  // so each lane holds runs of 4 consecutive columns of one row.
  float16_t acc[kTM][4];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  auto mfma16 = [&](const half8_t (&fa)[kTM], const half8_t (&fb)[4]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };

  // Prologue: the first K tile complete in its stage, the second in flight.
  gload_scales(kt_begin);
  gload_codes(kt_begin);
  sstore_scales(kt_begin);
  gload_scales(kt_begin + 1);
  gload_codes(kt_begin + 1);
  stage_barrier();
  uint32_t asc[kTM], bsc[4];
  uint4 ar0[kTM], br0[4], ar1[kTM], br1[4];
  rscale(stage(kt_begin), asc, bsc);
  rhalf(stage(kt_begin), 0, ar0, br0);
  half8_t fa[kTM], fb[4], na[kTM], nb[4];
  expand(ar0, br0, asc, bsc, 0, fa, fb);

  // Every iteration is the same branch-free body (the last two also prepare tiles that
  // are never multiplied), so each sub-step is one scheduling region.
#pragma clang loop unroll(disable)
  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const uint8_t* cur = stage(kt);
    const uint8_t* nxt = stage(kt + 1);
    // sub-step 0
    expand(ar0, br0, asc, bsc, 1, na, nb);
    mfma16(fa, fb);
    interleave<0, 4 * kTM>();
    // sub-step 1
    expand(ar0, br0, asc, bsc, 2, fa, fb);
    mfma16(na, nb);
    interleave<0, 4 * kTM>();
    // sub-step 2
    rhalf(cur, 1, ar1, br1);
    expand(ar0, br0, asc, bsc, 3, na, nb);
    mfma16(fa, fb);
    interleave<0x100, 4 * kTM>();
    // sub-step 3
    expand(ar1, br1, asc, bsc, 4, fa, fb);
    mfma16(na, nb);
    interleave<0, 4 * kTM>();
    // sub-step 4: the next tile's scales (loaded a tile ago) go to its stage
    sstore_scales(kt + 1);
    expand(ar1, br1, asc, bsc, 5, na, nb);
    mfma16(fa, fb);
    interleave<0x200, 4 * kTM>();
    stage_barrier();
    // sub-step 5
    uint32_t nasc[kTM], nbsc[4];
    rscale(nxt, nasc, nbsc);
    rhalf(nxt, 0, ar0, br0);
    gload_scales(kt + 2);
    gload_codes(kt + 2);
    expand(ar1, br1, asc, bsc, 6, fa, fb);
    mfma16(na, nb);
    interleave<0x100, 4 * kTM>();
    // sub-step 6
    expand(ar1, br1, asc, bsc, 7, na, nb);
    mfma16(fa, fb);
    interleave<0, 4 * kTM>();
    // sub-step 7: the next tile's first fragments
#pragma unroll
    for (int i = 0; i < kTM; ++i) asc[i] = nasc[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) bsc[j] = nbsc[j];
    expand(ar0, br0, asc, bsc, 0, fa, fb);
    mfma16(na, nb);
    interleave<0, 4 * kTM>();
  }
  stage_barrier();   // no load still landing in LDS, every wave done with the stages

  if (kSplit) {
    // Split-K: the raw fp32 accumulators of this K range, in register order (entry q of
    // thread t at ((split * tiles + tile) * kAcc + q) * 256 + t); split_k_reduce finishes.
    const int tiles = gridDim.x / splits;
    float* p = partial + ((int64_t)split * tiles + blockIdx.x / splits) * (G::kAcc * 256) + t;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) p[((i * 4 + j) * 16 + e) * 256] = acc[i][j][e];
    return;
  }

  // Epilogue: bf16(alpha * acc) staged through LDS 32 rows per wave at a time (8-byte
  // writes of 4 consecutive columns), then bf16(y + bias), written as 16-byte row
  // segments.  Each wave stages its own rows in its own LDS region, so only the wave's
  // own LDS order matters between the writes and the reads (lds_order): no workgroup
  // barrier, and nothing waits for the global stores, which drain while the workgroup
  // ends and the next one starts.
  uint8_t* epi = lds + wave * 32 * kEpiRowBytes;
  const int64_t wrow0 = row0 + wm * (32 * kTM);
  const int64_t wcol0 = col0 + wn * 128;
  // Lane l always stores the 8 columns col = wcol0 + 8 (l % 16) .. +7: it loads their
  // bias once, and stores them as one 16-byte segment when they are all inside the
  // output and the row starts are 16-byte aligned.
  const int64_t col = wcol0 + 8 * (lane & 15);
  const bool vec_store = col + 8 <= n && (ldo & 7) == 0 && ((uintptr_t)out & 15) == 0;
  uint32_t bw[4] = {0, 0, 0, 0};
  if (bias != nullptr) {
    if (col + 8 <= n && ((uintptr_t)(bias + col) & 15) == 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(bias + col);
      bw[0] = v.x;
      bw[1] = v.y;
      bw[2] = v.z;
      bw[3] = v.w;
    } else {
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (col + h < n) bw[h >> 1] |= (uint32_t)bias[col + h] << (16 * (h & 1));
    }
  }
  const float alpha0 = a_seg_rows > 0 ? 0.0f : alpha_for(gsf_a, gsf_b, 0, 0);
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    const int64_t arow = wrow0 + i * 32 + lr;    // this lane's accumulator row
    const float al = a_seg_rows > 0 ? alpha_for(gsf_a, gsf_b, a_seg_rows, min(arow, m - 1)) : alpha0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float y[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) y[s4] = __fmul_rn(al, __fmul_rn(acc[i][j][4 * q + s4], kAccUnscale));
        *reinterpret_cast<uint2*>(epi + lr * kEpiRowBytes + (32 * j + 8 * q + 4 * kh) * 2) =
            make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
      }
    }
    lds_order();
    const int64_t row_i = wrow0 + i * 32 + (lane >> 4);
    uint16_t* const out_i = out + row_i * ldo + col;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = 4 * p + (lane >> 4);
      const int64_t row = row_i + 4 * p;
      const uint4 v = *reinterpret_cast<const uint4*>(epi + r * kEpiRowBytes + (lane & 15) * 16);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
      if (bias != nullptr) {
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint32_t sh = 16 * (h & 1);
          const uint32_t zb = add_bias_bf16((w[h >> 1] >> sh) & 0xFFFFu, (uint16_t)(bw[h >> 1] >> sh));
          w[h >> 1] = (w[h >> 1] & (0xFFFF0000u >> sh)) | (zb << sh);
        }
      }
      if (row < m) {
        uint16_t* o = out_i + 4 * p * ldo;
        if (vec_store) {
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(o));
        } else if (col < n) {
          const uint64_t lo = ((uint64_t)w[1] << 32) | w[0], hi = ((uint64_t)w[3] << 32) | w[2];
          const int cnt = n - col < 8 ? (int)(n - col) : 8;
#pragma unroll 1
          for (int h = 0; h < cnt; ++h) o[h] = (uint16_t)((h < 4 ? lo : hi) >> (16 * (h & 3)));
        }
      }
    }
    lds_order();
  }
}

// Sums the split-K partials of `tiles` tiles (starting at tile index tile0) in split
// order, then applies the epilogue of the main kernel: bf16(alpha * acc), then the bias.
// Each thread finishes 8 consecutive columns of one output row: entries 4 q' .. 4 q' + 3
// of accumulator block (i, j) of the main kernel's lanes l and l + 32 (l < 32) of one
// wave; consecutive threads take consecutive l, so the partial reads coalesce.
template <int kTM>
__global__ void __launch_bounds__(256) split_k_reduce(const float* __restrict__ partial, int splits, int tiles,
                                                      int tile0, int sub, int tiles_m, int64_t m, int64_t n,
                                                      const float* __restrict__ gsf_a, const float* __restrict__ gsf_b,
                                                      int64_t a_seg_rows, const uint16_t* __restrict__ bias,
                                                      uint16_t* __restrict__ out, int64_t ldo) {
  using G = Geo<kTM>;
  constexpr int kPerTile = G::kAcc * 256 / 8;     // threads per tile
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int tl = (int)(gid / kPerTile);            // tile within the split launch
  int u = (int)(gid % kPerTile);
  const int l = u & 31;
  u >>= 5;
  const int qq = u & 3;
  u >>= 2;
  const int j = u & 3;
  u >>= 2;
  const int i = u % kTM;
  const int wave = u / kTM;
  // value h of split sp: entry (i * 4 + j) * 16 + 4 qq + h % 4 of thread 64 wave + 32 (h / 4) + l
  const float* src = partial + ((int64_t)tl * G::kAcc + (i * 4 + j) * 16 + 4 * qq) * 256 + wave * 64 + l;
  const int64_t split_stride = (int64_t)tiles * G::kAcc * 256;
  auto load8 = [&](int sp, float (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 8; ++h) v[h] = src[sp * split_stride + (h & 3) * 256 + 32 * (h >> 2)];
  };
  // Sums in split order; four splits' loads are in flight at a time.
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  int sp = 0;
  for (; sp + 4 <= splits; sp += 4) {
    float v[4][8];
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) load8(sp + u4, v[u4]);
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4)
#pragma unroll
      for (int h = 0; h < 8; ++h) acc[h] += v[u4][h];
  }
  for (; sp < splits; ++sp) {
    float v[8];
    load8(sp, v);
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[h] += v[h];
  }
  const int tile = tile0 + tl / sub;
  int tm, tn;
  tile_coords(tile, tiles_m, (int)((n + kRows - 1) / kRows), tm, tn);
  const int64_t row = ((int64_t)tm * sub + tl % sub) * G::kRowsA + (wave >> 1) * (32 * kTM) + i * 32 + l;
  const int64_t col = (int64_t)tn * kRows + (wave & 1) * 128 + j * 32 + 8 * qq;
  if (row >= m || col >= n) return;
  const float alpha = alpha_for(gsf_a, gsf_b, a_seg_rows, row);
  uint16_t y[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    uint32_t v = f32_to_bf16(__fmul_rn(alpha, __fmul_rn(acc[h], kAccUnscale)));
    if (bias != nullptr && col + h < n) v = add_bias_bf16(v, bias[col + h]);
    y[h] = (uint16_t)v;
  }
  uint16_t* o = out + row * ldo + col;
  if (col + 8 <= n && ((uintptr_t)o & 15) == 0) {
    *reinterpret_cast<uint4*>(o) = make_uint4(y[0] | ((uint32_t)y[1] << 16), y[2] | ((uint32_t)y[3] << 16),
                                              y[4] | ((uint32_t)y[5] << 16), y[6] | ((uint32_t)y[7] << 16));
  } else {
    for (int h = 0; h < 8 && col + h < n; ++h) o[h] = y[h];
  }
}

// Few activation rows take 128-row tiles (half the MFMA work of a 256-row tile that
// would mostly multiply clamped rows).
int pipe_tm(int64_t m) { return m <= 128 ? 2 : 4; }

// How a problem is cut: `full` tiles in whole rounds of one tile per compute unit,
// then `rest` tiles, each split `splits` ways along K when that fills the GPU better
// and the workspace allows it.
struct PipePlan {
  int64_t tiles_m, tiles_n, full, rest;
  int splits;
  int tm;                  // kTM of the kernel
  int sub;                 // 2: the split tail runs as 128-row halves (kTM 2) of the rest tiles
  size_t partial_floats;   // per split unit (tile or half)
};

PipePlan pipe_plan(int64_t m, int64_t k, int64_t n, int cus) {
  PipePlan p;
  p.tm = pipe_tm(m);
  const int64_t rows_a = 64 * p.tm;
  p.partial_floats = (size_t)rows_a * kRows;
  p.tiles_m = (m + rows_a - 1) / rows_a;
  p.tiles_n = (n + kRows - 1) / kRows;
  const int64_t tiles = p.tiles_m * p.tiles_n;
  p.full = tiles / cus * cus;
  p.rest = tiles - p.full;
  p.splits = 1;
  p.sub = 1;
  const int64_t kt = (k + BK - 1) / BK;
  if (p.rest > 0) {
    // With 256-row tiles and few of them left, their 128-row halves split half as many
    // ways fill the GPU as well and write half the partials; worth it while K is short
    // enough that the halves' lower MFMA rate costs less than the partials it saves
    // (measured: K = 5120 gains 9 us, K = 8192 loses 2 us, K = 25600 loses 20 us).
    const bool no_empty_half = m % 256 == 0 || m % 256 > 128;   // the last tile row's halves both hold rows
    if (p.tm == 4 && kt <= 48 && no_empty_half && 2 * p.rest <= cus && kt >= 2 * (cus / (2 * p.rest)) &&
        cus / (2 * p.rest) >= 2) {
      p.sub = 2;
      p.partial_floats = (size_t)128 * kRows;
    }
    const int64_t units = p.rest * p.sub;
    int64_t sp = cus / units;               // at most one round: partials <= cus units
    while (sp > 1 && kt < 2 * sp) --sp;     // keep at least two K tiles per split
    p.splits = (int)(sp < 1 ? 1 : sp);
  }
  return p;
}

size_t plan_bytes(const PipePlan& p) {
  return p.splits > 1 ? (size_t)p.splits * (size_t)(p.rest * p.sub) * p.partial_floats * sizeof(float) : 0;
}

// The K-split tail: `units` split tiles (or halves, sub = 2) from tile index tile0 of a
// grid of tiles_m x tiles_n tiles, then the reduce.
template <int kTM>
hipError_t launch_split_tail(const PipePlan& p, int sub, const uint8_t* a_codes, const uint8_t* a_scales, int64_t m,
                             int64_t k, const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                             const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                             float* partial, hipStream_t s) {
  constexpr int kLds = Geo<kTM>::kLds;
  static bool attr_set[kMaxDevices] = {};
  if (hipError_t e = set_dynamic_lds_once(reinterpret_cast<const void*>(&gemm_pipe_kernel<true, kTM>), kLds,
                                          attr_set);
      e != hipSuccess)
    return e;
  const int tm = (int)p.tiles_m, tn = (int)p.tiles_n;
  const int64_t units = p.rest * sub;
  hipLaunchKernelGGL((gemm_pipe_kernel<true, kTM>), dim3((uint32_t)(units * p.splits)), dim3(256), kLds, s, a_codes,
                     a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, n, n, tm, tn,
                     (int)p.full, p.splits, sub, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((split_k_reduce<kTM>), dim3((uint32_t)(units * Geo<kTM>::kAcc / 8)), dim3(256), 0, s, partial,
                     p.splits, (int)units, (int)p.full, sub, tm, m, n, gsf_a, gsf_b, a_seg_rows, bias, out, n);
  return hipGetLastError();
}

template <int kTM>
hipError_t launch_plan(const PipePlan& p, const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                       const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out, float* partial,
                       hipStream_t s) {
  constexpr int kLds = Geo<kTM>::kLds;
  static bool attr_set[kMaxDevices] = {};
  if (hipError_t e = set_dynamic_lds_once(reinterpret_cast<const void*>(&gemm_pipe_kernel<false, kTM>), kLds,
                                          attr_set);
      e != hipSuccess)
    return e;
  const int tm = (int)p.tiles_m, tn = (int)p.tiles_n;
  if (p.full > 0) {
    hipLaunchKernelGGL((gemm_pipe_kernel<false, kTM>), dim3((uint32_t)p.full), dim3(256), kLds, s, a_codes, a_scales,
                       m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, n, n, tm, tn, 0, 1, 1,
                       (float*)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.rest == 0) return hipSuccess;
  if (p.splits == 1) {
    hipLaunchKernelGGL((gemm_pipe_kernel<false, kTM>), dim3((uint32_t)p.rest), dim3(256), kLds, s, a_codes, a_scales,
                       m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out, n, n, tm, tn, (int)p.full, 1,
                       1, (float*)nullptr);
    return hipGetLastError();
  }
  if (kTM == 4 && p.sub == 2)
    return launch_split_tail<2>(p, 2, a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias,
                                out, partial, s);
  return launch_split_tail<kTM>(p, 1, a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias,
                                out, partial, s);
}

}  // namespace

bool gemm_pipe_supported(int64_t m, int64_t k, int64_t n, const void* a_codes, const void* a_scales,
                         const void* b_codes, const void* b_scales, int cus) {
  (void)m;
  (void)n;
  (void)cus;
  const bool aligned = (((uintptr_t)a_codes | (uintptr_t)b_codes | (uintptr_t)a_scales | (uintptr_t)b_scales) & 15) == 0;
  return (k / 2) % 16 == 0 && aligned;
}

size_t gemm_pipe_workspace_bytes(int64_t m, int64_t k, int64_t n, int cus) {
  return plan_bytes(pipe_plan(m, k, n, cus));
}

hipError_t launch_gemm_pipe(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                            const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                            const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                            void* workspace, size_t workspace_bytes, int cus, hipStream_t s) {
  PipePlan p = pipe_plan(m, k, n, cus);
  const size_t need = plan_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) p.splits = 1;
  float* partial = static_cast<float*>(workspace);
  if (p.tm == 2)
    return launch_plan<2>(p, a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out,
                          partial, s);
  return launch_plan<4>(p, a_codes, a_scales, m, k, b_codes, b_scales, n, gsf_a, gsf_b, a_seg_rows, bias, out,
                        partial, s);
}

}  // namespace nvfp4
