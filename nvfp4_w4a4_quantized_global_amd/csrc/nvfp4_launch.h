// Host-side launchers of the gfx950 kernels (one per kernel family).  Each returns
// hipGetLastError() after queuing its launch on `s`; arguments are checked by the
// C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Upper bound on the number of per-block partial maxima of the amax pass.
constexpr int kMaxAmaxPartials = 1024;

hipError_t launch_amax_partials(const uint16_t* x, int64_t rows, int64_t k, int group, float inv_sqrt_g,
                                float* partials, int* n_partials, hipStream_t s);

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t k, int group, float inv_sqrt_g,
                           const float* static_gsf, const float* partials, int n_partials,
                           uint8_t* codes, uint8_t* scales, float* gsf_out, hipStream_t s);

hipError_t launch_rotate(const void* x, bool x_bf16, void* y, bool y_bf16, int64_t rows, int64_t k, int group,
                         float inv_sqrt_g, hipStream_t s);

hipError_t launch_scale_layout(const uint8_t* src, uint8_t* dst, int64_t rows, int64_t k, bool to_canonical,
                               hipStream_t s);

hipError_t launch_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                       const uint8_t* b_codes, const uint8_t* b_scales, int64_t n,
                       const float* gsf_a, const float* gsf_b, const uint16_t* bias, uint16_t* out, hipStream_t s);

// The software-pipelined large-tile GEMM (gemm_pipe.hip): usable when the problem has
// at least one 256 x 256 tile per compute unit, K is a multiple of 32 and every
// operand pointer is 16-byte aligned.  It computes output columns [0, n) of a
// product whose B scale layout holds b_srows rows per K tile and whose output rows
// are ldo elements apart.
bool gemm_pipe_supported(int64_t m, int64_t k, int64_t n, const void* a_codes, const void* a_scales,
                         const void* b_codes, const void* b_scales, int cus);
hipError_t launch_gemm_pipe(const uint8_t* a_codes, const uint8_t* a_scales, int64_t m, int64_t k,
                            const uint8_t* b_codes, const uint8_t* b_scales, int64_t n, int64_t b_srows,
                            const float* gsf_a, const float* gsf_b, const uint16_t* bias, uint16_t* out,
                            int64_t ldo, hipStream_t s);

}  // namespace nvfp4
