// Host-side launchers of the gfx950 kernels (one per kernel family).  Each returns
// hipGetLastError() after queuing its launch on `s`; arguments are checked by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Devices the library keeps per-device state for (compute-unit counts, kernel attributes).
constexpr int kMaxDevices = 64;

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once per device
// (`done` is the caller's per-kernel record); a no-op after the first call there.
hipError_t set_dynamic_lds_once(const void* kernel, int bytes, bool (&done)[kMaxDevices]);

// Upper bound on the number of per-block partial maxima of the amax pass, and on the
// number of segments (row blocks with their own scale) of one call.
constexpr int kMaxAmaxPartials = 8192;
constexpr int kMaxSegments = 1024;

// Partial maxima of `segments` consecutive row blocks of seg_rows rows each (one
// segment for a plain call): partials[seg * (*n_partials) + i].  With `up` not NULL the
// input is the bf16 SwiGLU product of x (gate) and up, computed on the fly and, if
// xout is not NULL, stored there.
hipError_t launch_amax_partials(const uint16_t* x, const uint16_t* up, uint16_t* xout, int64_t seg_rows, int64_t k,
                                int segments, int group, float inv_sqrt_g, float* partials, int* n_partials,
                                hipStream_t s);

// Quantizes rows x [rows][k]; with static_gsf NULL, segment s (rows [s*seg_rows,
// (s+1)*seg_rows)) takes its global scale from its n_partials partial maxima and
// gsf_out[s] receives it.  With a16 not NULL, a16 [rows][k] also receives every
// quantized value as the exact fp16 code * scale * 2^-8 (the operand form of the GEMMs,
// for gemm_decode_a16).
hipError_t launch_quantize(const uint16_t* x, const uint16_t* up, int64_t rows, int64_t k, int group,
                           float inv_sqrt_g, const float* static_gsf, const float* partials, int n_partials,
                           int64_t seg_rows, int segments, uint8_t* codes, uint8_t* scales, float* gsf_out,
                           hipStream_t s, uint16_t* a16 = nullptr);

// Dynamic-scale quantize of a small input (rows * k within quantize_small_supported) in
// one launch: the same codes, scales, global scale (*gsf_out) and a16 as
// launch_amax_partials followed by launch_quantize with one segment.
bool quantize_small_supported(int64_t rows, int64_t k);
hipError_t launch_quantize_small(const uint16_t* x, int64_t rows, int64_t k, int group, float inv_sqrt_g,
                                 uint8_t* codes, uint8_t* scales, float* gsf_out, hipStream_t s,
                                 uint16_t* a16 = nullptr);

// x [rows][k] = bf16 SwiGLU product of gate and up.
hipError_t launch_swiglu(const uint16_t* gate, const uint16_t* up, uint16_t* x, int64_t rows, int64_t k, hipStream_t s);

// NVFP4 [rows][k] (codes + scales in the library layout) -> bf16 or fp32 values
// fp32(code * scale) / gsf.
hipError_t launch_dequant(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, const float* gsf,
                          void* out, bool out_bf16, hipStream_t s);

// *amax = max of n_partials partial maxima (accumulate: max with the value already there).
hipError_t launch_amax_finalize(const float* partials, int n_partials, float* amax, bool accumulate, hipStream_t s);

// *gsf = 2688 / max(fp32(*amax * margin), 1e-12).
hipError_t launch_static_scale(const float* amax, float margin, float* gsf, hipStream_t s);

hipError_t launch_rotate(const void* x, bool x_bf16, void* y, bool y_bf16, int64_t rows, int64_t k, int group,
                         float inv_sqrt_g, hipStream_t s);

hipError_t launch_scale_layout(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t k, bool to_canonical,
                               hipStream_t s);

// alpha = 1 / (gsf_a * gsf_b); with a_seg_rows > 0, row r of A takes gsf_a[r / a_seg_rows]
// (one global scale per block of a_seg_rows rows), otherwise gsf_a[0] for every row.
hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t n,
                       const float* gsf_a, const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias,
                       uint16_t* out, void* workspace, size_t workspace_bytes, hipStream_t s);

// Compute units of the current device (cached per device).
int compute_units();

// The software-pipelined 256 x 256-tile GEMM (gemm_pipe.hip): K a multiple of 32 and
// every operand pointer 16-byte aligned.  Tiles beyond the
// last whole round (one tile per compute unit) are split along K when the workspace
// (gemm_pipe_workspace_bytes) allows; without it they run unsplit.
bool gemm_pipe_supported(int64_t m, int64_t k, int64_t n, const void* a_codes, const void* a_scales,
                         const void* b_codes, const void* b_scales, int cus);
size_t gemm_pipe_workspace_bytes(int64_t m, int64_t k, int64_t n, int cus);
hipError_t launch_gemm_pipe(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                            const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                            const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                            void* workspace, size_t workspace_bytes, int cus, hipStream_t s);

// The decode GEMM for m <= kDecodeA16Rows activation rows given as the fp16 operand
// form a16 [m][k] (launch_quantize's a16 output) instead of codes and scales, so the
// kernel expands only the weight.  One activation scale (gsf_a[0]).  K a multiple of
// 32, b_codes 16-byte and b_scales 4-byte aligned, a16 16-byte aligned.
constexpr int kDecodeA16Rows = 4;
bool gemm_decode_a16_supported(int64_t m, int64_t k, const void* a16, const void* b_codes, const void* b_scales);
hipError_t launch_gemm_decode_a16(const uint16_t* a16, int64_t m, int64_t k, const uint8_t* b_codes,
                                  const uint8_t* b_scales, int64_t n, const float* gsf_a, const float* gsf_b,
                                  const uint16_t* bias, uint16_t* out, void* workspace, size_t workspace_bytes,
                                  int cus, hipStream_t s);

// The weight-streaming GEMM for m <= 128 (gemm_skinny.hip): K a multiple of 32, code
// pointers 16-byte and scale pointers 4-byte aligned.  Splits K across blocks when the
// workspace (gemm_skinny_workspace_bytes) allows.
bool gemm_skinny_supported(int64_t m, int64_t k, const void* a_codes, const void* a_scales, const void* b_codes,
                           const void* b_scales);
size_t gemm_skinny_workspace_bytes(int64_t m, int64_t k, int64_t n, int cus);
hipError_t launch_gemm_skinny(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, const float* gsf_a,
                              const float* gsf_b, int64_t a_seg_rows, const uint16_t* bias, uint16_t* out,
                              void* workspace, size_t workspace_bytes, int cus, hipStream_t s);

// The whole linear for up to 16 activation rows with a static scale, in the
// weight-streaming kernel: each block quantizes its K range of the bf16 rows x [m][k]
// into LDS (same codes and scales as launch_quantize) instead of a separate pass.
// Needs the workspace of gemm_skinny_workspace_bytes (hipErrorInvalidValue without).
// The linear at one activation row in one launch: each wave of the decode GEMM quantizes
// its K range of the bf16 row itself (bit-identical to the quantize pass then the GEMM).
// gsf_x: the static scale, or NULL for the dynamic one, which every block forms from the
// row's abs-max.  gsf_used (NULL allowed only with a static scale) receives the scale
// used.  Needs the split-K partials of gemm_workspace_bytes when the decode plan splits
// K, else runs unsplit while every wave's range fits its LDS region.
bool linear_decode_fused_supported(int64_t m, int64_t k, int64_t n, bool dynamic, const void* x,
                                   const void* b_codes, const void* b_scales, size_t workspace_bytes, int cus);
hipError_t launch_linear_decode_fused(const uint16_t* x, int64_t k, const uint8_t* b_codes, const uint8_t* b_scales,
                                      int64_t n, const float* gsf_x, float* gsf_used, const float* gsf_w,
                                      const uint16_t* bias, uint16_t* out, void* workspace, size_t workspace_bytes,
                                      int cus, hipStream_t s);

// Workspace the GEMM dispatcher can use for an [m, k] x [n, k] product (0 if none).
size_t gemm_workspace_bytes(int64_t m, int64_t k, int64_t n);

}  // namespace nvfp4
