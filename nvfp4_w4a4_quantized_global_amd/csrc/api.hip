// C ABI of libnvfp4.so: argument checks, workspace carving and kernel launches.
// The contract of every call is in include/nvfp4.h.  Checks mirror the
// ValueErrors of NVFP4DecoderLinear.__init__ / .from_packed on the
// "minimax_h3_nvfp4_decoder" page (in_features divisible by the 16-value block,
// rotation group dividing in_features, packed weight [out, in/2]).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/nvfp4.h"
#include "nvfp4_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Profiler ranges (roctx): one around each entry-point call, one around each stage
// inside it (nvfp4.amax, nvfp4.quantize, nvfp4.gemm), so that a marker trace ties every
// kernel to the call and stage that queued it.  Without a profiler a push or pop is a
// call into an empty dispatch table.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

size_t align_up(size_t v) { return (v + NVFP4_WORKSPACE_ALIGN - 1) / NVFP4_WORKSPACE_ALIGN * NVFP4_WORKSPACE_ALIGN; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // rows and K each below 2^31

int check_rows_k(const char* fn, int64_t rows, int64_t k, bool allow_empty) {
  if (rows < 0 || (!allow_empty && rows == 0) || rows >= kMaxDim)
    return fail(NVFP4_ERR_SHAPE, "%s: rows must be in [%d, 2^31), got %lld", fn, allow_empty ? 0 : 1, (long long)rows);
  if (k <= 0 || k >= kMaxDim) return fail(NVFP4_ERR_SHAPE, "%s: K must be in [16, 2^31), got %lld", fn, (long long)k);
  if (k % NVFP4_BLOCK_SIZE)
    return fail(NVFP4_ERR_SHAPE, "%s: NVFP4 needs K divisible by %d, got %lld", fn, NVFP4_BLOCK_SIZE, (long long)k);
  if ((double)rows * (double)k >= 9.0e18) return fail(NVFP4_ERR_SHAPE, "%s: rows*K overflows", fn);
  return NVFP4_OK;
}

int check_group(const char* fn, int g, int64_t k, bool allow_none) {
  if (allow_none && g == 0) return NVFP4_OK;
  if (g < 2 || g > NVFP4_MAX_ROTATION_GROUP || (g & (g - 1)))
    return fail(NVFP4_ERR_ARG, "%s: rotation group must be a power of two in [2, %d]%s, got %d", fn,
                NVFP4_MAX_ROTATION_GROUP, allow_none ? " or 0" : "", g);
  if (k % g) return fail(NVFP4_ERR_ARG, "%s: rotation group %d does not divide K %lld", fn, g, (long long)k);
  return NVFP4_OK;
}

float inv_sqrt(int g) { return g > 1 ? (float)(1.0 / sqrt((double)g)) : 1.0f; }

// Alignment the kernels rely on: bf16 / fp32 inputs are read in 16-byte pieces, codes
// and scales in 8-byte pieces, outputs and biases element by element wherever a wider
// access would be misaligned, global scales as fp32 words.  NULL passes (optional
// pointers are checked for presence elsewhere).
int check_align(const char* fn, const char* what, const void* p, unsigned bytes) {
  if ((uintptr_t)p % bytes) return fail(NVFP4_ERR_ARG, "%s: %s must be %u-byte aligned", fn, what, bytes);
  return NVFP4_OK;
}
int check_aligned(const char* fn, const char* what, const void* p) { return check_align(fn, what, p, 16); }

// Packed codes and block scales of one operand (8-byte pieces).
int check_nvfp4_operand(const char* fn, const char* codes_name, const void* codes, const char* scales_name,
                        const void* scales) {
  if (int rc = check_align(fn, codes_name, codes, 8)) return rc;
  return check_align(fn, scales_name, scales, 8);
}

// bf16 output and optional bias (element alignment), fp32 global scales.
int check_epilogue(const char* fn, const void* out, const void* bias, const float* gsf_a, const float* gsf_b) {
  if (int rc = check_align(fn, "out", out, 2)) return rc;
  if (int rc = check_align(fn, "bias", bias, 2)) return rc;
  if (int rc = check_align(fn, "global_sf_x", gsf_a, 4)) return rc;
  return check_align(fn, "global_sf_w", gsf_b, 4);
}

struct LinearWorkspace {
  uint8_t* codes;
  uint8_t* scales;
  float* partials;
  float* gsf;
  void* gemm;
  uint16_t* a16;   // the activation's fp16 operand form (m <= kDecodeA16Rows), or NULL
  size_t gemm_bytes;
  size_t bytes;
};

// Layout of an nvfp4_linear workspace: codes, scales, amax partials, one global scale
// per segment, the GEMM's split-K partials, then (m <= kDecodeA16Rows) the fp16 operand
// form of the activation for the decode GEMM; every piece 256-byte aligned.
// Without split_k the GEMM region is left out (the GEMM then runs its last round of
// tiles unsplit: the same function, fp32 summation order aside).
LinearWorkspace carve(void* base, int64_t m, int64_t k, int64_t n, int64_t segments = 1, bool split_k = true) {
  // offsets first, pointers only for a real base
  const size_t o_codes = 0;
  const size_t o_scales = align_up(o_codes + (size_t)m * (size_t)(k / 2));
  const size_t o_partials = align_up(o_scales + nvfp4_scale_bytes(m, k));
  const size_t o_gsf = align_up(o_partials + sizeof(float) * nvfp4::kMaxAmaxPartials);
  const size_t o_gemm = align_up(o_gsf + sizeof(float) * (size_t)segments);
  const size_t gemm_bytes = split_k ? nvfp4::gemm_workspace_bytes(m, k, n) : 0;
  const size_t o_a16 = align_up(o_gemm + gemm_bytes);
  const size_t a16_bytes = m <= nvfp4::kDecodeA16Rows && segments == 1 ? (size_t)m * (size_t)k * 2u : 0;
  LinearWorkspace w{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, gemm_bytes, align_up(o_a16 + a16_bytes)};
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.codes = p + o_codes;
    w.scales = p + o_scales;
    w.partials = reinterpret_cast<float*>(p + o_partials);
    w.gsf = reinterpret_cast<float*>(p + o_gsf);
    w.gemm = gemm_bytes ? p + o_gemm : nullptr;
    w.a16 = a16_bytes ? reinterpret_cast<uint16_t*>(p + o_a16) : nullptr;
  }
  return w;
}

// Rows form `segments` consecutive blocks of m / segments rows; with a dynamic scale
// each block gets its own global scale (gsf_out[segment]).
// With `up` not NULL the input is the SwiGLU product of x (gate) and up.  A static
// scale forms it inside the single quantize pass; a dynamic one forms it once in the
// amax pass, which stores it in xbuf ([m][k] bf16) for the quantize pass to read.
int quantize_impl(const char* fn, const void* x, int64_t m, int64_t k, const float* gsf_static, int group,
                  uint8_t* codes, uint8_t* scales, float* gsf_out, float* partials, hipStream_t s,
                  int64_t segments = 1, const void* up = nullptr, void* xbuf = nullptr, uint16_t* a16 = nullptr) {
  int n_partials = 0;
  const float c = inv_sqrt(group);
  const int64_t seg_rows = m / segments;
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* upp = static_cast<const uint16_t*>(up);
  if (gsf_static == nullptr && segments == 1 && up == nullptr &&
      nvfp4::quantize_small_supported(m, k)) {   // small input: both passes in one launch
    Range stage("nvfp4.amax+quantize");
    return hip_status(nvfp4::launch_quantize_small(xp, m, k, group, c, codes, scales, gsf_out, s, a16), fn);
  }
  if (gsf_static == nullptr) {
    Range stage("nvfp4.amax");
    uint16_t* xout = upp != nullptr ? static_cast<uint16_t*>(xbuf) : nullptr;
    int rc = hip_status(nvfp4::launch_amax_partials(xp, upp, xout, seg_rows, k, (int)segments, group, c, partials,
                                                    &n_partials, s), fn);
    if (rc) return rc;
    if (xout != nullptr) {
      xp = xout;
      upp = nullptr;
    }
  }
  Range stage("nvfp4.quantize");
  return hip_status(nvfp4::launch_quantize(xp, upp, m, k, group, c, gsf_static, partials, n_partials, seg_rows,
                                           (int)segments, codes, scales, gsf_out, s, a16), fn);
}

size_t product_bytes(int64_t m, int64_t k) { return align_up((size_t)m * (size_t)k * 2u); }

int check_segments(const char* fn, int64_t segments, int64_t seg_rows) {
  if (segments < 1 || segments > nvfp4::kMaxSegments)
    return fail(NVFP4_ERR_ARG, "%s: segments must be in [1, %d], got %lld", fn, nvfp4::kMaxSegments,
                (long long)segments);
  if (seg_rows < 0 || (double)segments * (double)seg_rows >= (double)kMaxDim)
    return fail(NVFP4_ERR_SHAPE, "%s: segments * seg_rows must be in [0, 2^31), got %lld * %lld", fn,
                (long long)segments, (long long)seg_rows);
  return NVFP4_OK;
}

// nvfp4_linear over `segments` row blocks of seg_rows rows (1 for a plain call).
int linear_impl(const char* fn, const void* x, int64_t segments, int64_t seg_rows, int64_t k, const uint8_t* packed,
                const uint8_t* inv_scale, const float* global_sf_w, const void* bias, int64_t out_features,
                const float* global_sf_x, int rotation_group, void* out, float* gsf_out, void* workspace,
                size_t workspace_bytes, hipStream_t s, const void* up = nullptr, bool split_k = true) {
  // a dynamic scale over a SwiGLU product keeps the product after the linear workspace
  Range call(fn);
  const bool keep_product = up != nullptr && global_sf_x == nullptr;
  const int64_t m = segments * seg_rows;
  if (int rc = check_rows_k(fn, m, k, true)) return rc;
  if (int rc = check_group(fn, rotation_group, k, true)) return rc;
  if (out_features <= 0 || out_features >= kMaxDim)
    return fail(NVFP4_ERR_SHAPE, "%s: out_features must be in [1, 2^31), got %lld", fn, (long long)out_features);
  if (m == 0) return NVFP4_OK;
  if (!x || !packed || !inv_scale || !global_sf_w || !out) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (int rc = check_aligned(fn, "x", x)) return rc;
  if (int rc = check_nvfp4_operand(fn, "packed", packed, "inv_scale", inv_scale)) return rc;
  if (int rc = check_epilogue(fn, out, bias, global_sf_x, global_sf_w)) return rc;
  if (int rc = check_align(fn, "gsf_out", gsf_out, 4)) return rc;
  const size_t base = carve(nullptr, m, k, out_features, segments, split_k).bytes;
  const size_t need = base + (keep_product ? product_bytes(m, k) : 0);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN))
    return fail(NVFP4_ERR_WORKSPACE, "%s: need a %d-byte aligned workspace of %zu bytes, got %zu", fn,
                NVFP4_WORKSPACE_ALIGN, need, workspace_bytes);
  const LinearWorkspace ws = carve(workspace, m, k, out_features, segments, split_k);
  float* gsf = gsf_out != nullptr ? gsf_out : ws.gsf;   // the GEMM reads the scales where they were written
#ifndef NVFP4_FUSED_ONE_ROW
#define NVFP4_FUSED_ONE_ROW 1
#endif
  if (NVFP4_FUSED_ONE_ROW && rotation_group == 0 && up == nullptr && segments == 1 &&
      nvfp4::linear_decode_fused_supported(m, k, out_features, global_sf_x == nullptr, x, packed, inv_scale,
                                           ws.gemm_bytes, nvfp4::compute_units())) {
    // one row: quantized (and with a dynamic scale, its abs-max taken) by the decode
    // GEMM's blocks themselves, one launch
    Range stage(global_sf_x != nullptr ? "nvfp4.quantize+gemm" : "nvfp4.amax+quantize+gemm");
    return hip_status(nvfp4::launch_linear_decode_fused(static_cast<const uint16_t*>(x), k, packed, inv_scale,
                                                        out_features, global_sf_x,
                                                        global_sf_x != nullptr ? gsf_out : gsf, global_sf_w,
                                                        static_cast<const uint16_t*>(bias),
                                                        static_cast<uint16_t*>(out), ws.gemm, ws.gemm_bytes,
                                                        nvfp4::compute_units(), s),
                      fn);
  }
  const bool per_segment = global_sf_x == nullptr && segments > 1;
  void* xbuf = keep_product ? static_cast<uint8_t*>(workspace) + base : nullptr;
  // a few rows: the quantize pass also writes the fp16 operand form, and the decode GEMM
  // then expands only the weight
  const bool a16 = ws.a16 != nullptr && !per_segment &&
                   nvfp4::gemm_decode_a16_supported(m, k, ws.a16, packed, inv_scale);
  if (int rc = quantize_impl(fn, x, m, k, global_sf_x, rotation_group, ws.codes, ws.scales, gsf, ws.partials, s,
                             per_segment ? segments : 1, up, xbuf, a16 ? ws.a16 : nullptr))
    return rc;
  Range stage("nvfp4.gemm");
  if (a16)
    return hip_status(nvfp4::launch_gemm_decode_a16(ws.a16, m, k, packed, inv_scale, out_features, gsf, global_sf_w,
                                                    static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(out),
                                                    ws.gemm, ws.gemm_bytes, nvfp4::compute_units(), s),
                      fn);
  return hip_status(nvfp4::launch_gemm(ws.codes, ws.scales, m, k, packed, inv_scale, out_features, gsf, global_sf_w,
                                       per_segment ? seg_rows : 0, static_cast<const uint16_t*>(bias),
                                       static_cast<uint16_t*>(out), ws.gemm, ws.gemm_bytes, s),
                    fn);
}

// Fixed device scratch of nvfp4_linear_noalloc, for callers that cannot allocate.
// Each device the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: its device
// address is resolved once per device with hipGetSymbolAddress and only that address
// is handed to kernels.
static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's scratch address, resolved on the first call on that device.
int scratch_of_current_device(const char* fn, void** ptr) {
  int dev = -1;
  if (int rc = hip_status(hipGetDevice(&dev), fn)) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(NVFP4_ERR_HIP, "%s: device %d beyond the %d supported", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (int rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), fn)) return rc;
    if (p == nullptr || (uintptr_t)p % NVFP4_WORKSPACE_ALIGN)
      return fail(NVFP4_ERR_HIP, "%s: scratch of device %d resolved to an unusable address", fn, dev);
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" {

size_t nvfp4_scale_bytes(int64_t rows, int64_t k) {
  if (rows <= 0 || k <= 0) return 0;
  const int64_t kt = (k + NVFP4_SCALE_TILE_K - 1) / NVFP4_SCALE_TILE_K;
  return (size_t)kt * (size_t)rows * 8u;
}

size_t nvfp4_quantize_workspace_bytes(void) { return align_up(sizeof(float) * nvfp4::kMaxAmaxPartials); }

size_t nvfp4_linear_workspace_bytes(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k <= 0 || n <= 0) return 0;
  return carve(nullptr, m, k, n).bytes;
}

size_t nvfp4_linear_segmented_workspace_bytes(int64_t segments, int64_t seg_rows, int64_t k, int64_t n) {
  if (segments < 1 || segments > nvfp4::kMaxSegments || seg_rows < 0 || k <= 0 || n <= 0) return 0;
  return carve(nullptr, segments * seg_rows, k, n, segments).bytes;
}

size_t nvfp4_quantize_swiglu_workspace_bytes(int64_t m, int64_t k) {
  if (m < 0 || k <= 0) return 0;
  return nvfp4_quantize_workspace_bytes() + product_bytes(m, k);
}

size_t nvfp4_linear_swiglu_workspace_bytes(int64_t m, int64_t k, int64_t n) {
  if (m < 0 || k <= 0 || n <= 0) return 0;
  return carve(nullptr, m, k, n).bytes + product_bytes(m, k);
}

size_t nvfp4_gemm_workspace_bytes(int64_t m, int64_t k, int64_t n) {
  if (m <= 0 || k <= 0 || n <= 0) return 0;
  return nvfp4::gemm_workspace_bytes(m, k, n);
}

const char* nvfp4_last_error(void) { return g_err; }

int rotate_activation(const void* x, int x_dtype, void* y, int y_dtype, int64_t rows, int64_t k, int group_size,
                      void* stream) {
  const char* fn = "rotate_activation";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, rows, k, true)) return rc;
  if (int rc = check_group(fn, group_size, k, false)) return rc;
  if ((x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32) ||
      (y_dtype != NVFP4_DTYPE_BF16 && y_dtype != NVFP4_DTYPE_F32))
    return fail(NVFP4_ERR_ARG, "%s: dtype must be NVFP4_DTYPE_BF16 or NVFP4_DTYPE_F32", fn);
  if (rows == 0) return NVFP4_OK;
  if (x == nullptr || y == nullptr) return fail(NVFP4_ERR_ARG, "%s: x and y must not be NULL", fn);
  if (int rc = check_aligned(fn, "x", x)) return rc;
  if (int rc = check_aligned(fn, "y", y)) return rc;
  if (x == y && x_dtype != y_dtype) return fail(NVFP4_ERR_ARG, "%s: in-place rotation needs equal dtypes", fn);
  return hip_status(nvfp4::launch_rotate(x, x_dtype == NVFP4_DTYPE_BF16, y, y_dtype == NVFP4_DTYPE_BF16, rows, k,
                                         group_size, inv_sqrt(group_size), static_cast<hipStream_t>(stream)),
                    fn);
}

int nvfp4_quantize_weight(const void* w, int64_t n, int64_t k, uint8_t* packed, uint8_t* inv_scale,
                          float* global_sf_w, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_quantize_weight";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, n, k, false)) return rc;
  if (!w || !packed || !inv_scale || !global_sf_w) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (int rc = check_aligned(fn, "w", w)) return rc;
  if (int rc = check_nvfp4_operand(fn, "packed", packed, "inv_scale", inv_scale)) return rc;
  if (int rc = check_align(fn, "global_sf_w", global_sf_w, 4)) return rc;
  if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes() ||
      ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN))
    return fail(NVFP4_ERR_WORKSPACE, "%s: need a %d-byte aligned workspace of %zu bytes, got %zu", fn,
                NVFP4_WORKSPACE_ALIGN, nvfp4_quantize_workspace_bytes(), workspace_bytes);
  return quantize_impl(fn, w, n, k, nullptr, 0, packed, inv_scale, global_sf_w, static_cast<float*>(workspace),
                       static_cast<hipStream_t>(stream));
}

int nvfp4_quantize_activation(const void* x, int64_t m, int64_t k, const float* global_sf_x, int rotation_group,
                              uint8_t* codes, uint8_t* scales, float* gsf_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_quantize_activation";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, m, k, true)) return rc;
  if (int rc = check_group(fn, rotation_group, k, true)) return rc;
  if (m == 0) return NVFP4_OK;
  if (!x || !codes || !scales) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (int rc = check_aligned(fn, "x", x)) return rc;
  if (int rc = check_nvfp4_operand(fn, "codes", codes, "scales", scales)) return rc;
  if (int rc = check_align(fn, "global_sf_x", global_sf_x, 4)) return rc;
  if (int rc = check_align(fn, "gsf_out", gsf_out, 4)) return rc;
  if (global_sf_x == nullptr &&
      (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes() ||
       ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN)))
    return fail(NVFP4_ERR_WORKSPACE, "%s: the dynamic scale needs a %d-byte aligned workspace of %zu bytes", fn,
                NVFP4_WORKSPACE_ALIGN, nvfp4_quantize_workspace_bytes());
  return quantize_impl(fn, x, m, k, global_sf_x, rotation_group, codes, scales, gsf_out,
                       static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
}

int nvfp4_amax(const void* x, int64_t rows, int64_t k, int rotation_group, float* amax, int accumulate,
               void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_amax";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, rows, k, true)) return rc;
  if (int rc = check_group(fn, rotation_group, k, true)) return rc;
  if (!amax) return fail(NVFP4_ERR_ARG, "%s: amax must not be NULL", fn);
  if (int rc = check_align(fn, "amax", amax, 4)) return rc;
  if (rows > 0 && !x) return fail(NVFP4_ERR_ARG, "%s: x must not be NULL", fn);
  if (rows > 0)
    if (int rc = check_aligned(fn, "x", x)) return rc;
  if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes() ||
      ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN))
    return fail(NVFP4_ERR_WORKSPACE, "%s: need a %d-byte aligned workspace of %zu bytes", fn, NVFP4_WORKSPACE_ALIGN,
                nvfp4_quantize_workspace_bytes());
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partials = static_cast<float*>(workspace);
  int n_partials = 0;
  if (rows > 0) {
    int rc = hip_status(nvfp4::launch_amax_partials(static_cast<const uint16_t*>(x), nullptr, nullptr, rows, k, 1,
                                                    rotation_group,
                                                    inv_sqrt(rotation_group), partials, &n_partials, s), fn);
    if (rc) return rc;
  }
  return hip_status(nvfp4::launch_amax_finalize(partials, n_partials, amax, accumulate != 0, s), fn);
}

int nvfp4_swiglu(const void* gate, const void* up, int64_t rows, int64_t k, void* x, void* stream) {
  const char* fn = "nvfp4_swiglu";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, rows, k, true)) return rc;
  if (rows == 0) return NVFP4_OK;
  if (!gate || !up || !x) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (((uintptr_t)gate | (uintptr_t)up | (uintptr_t)x) % 16)
    return fail(NVFP4_ERR_ARG, "%s: tensors must be 16-byte aligned", fn);
  return hip_status(nvfp4::launch_swiglu(static_cast<const uint16_t*>(gate), static_cast<const uint16_t*>(up),
                                         static_cast<uint16_t*>(x), rows, k, static_cast<hipStream_t>(stream)),
                    fn);
}

int nvfp4_quantize_swiglu(const void* gate, const void* up, int64_t m, int64_t k, const float* global_sf_x,
                          uint8_t* codes, uint8_t* scales, float* gsf_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const char* fn = "nvfp4_quantize_swiglu";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, m, k, true)) return rc;
  if (m == 0) return NVFP4_OK;
  if (!gate || !up || !codes || !scales) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (((uintptr_t)gate | (uintptr_t)up) % 16) return fail(NVFP4_ERR_ARG, "%s: gate and up must be 16-byte aligned", fn);
  if (int rc = check_nvfp4_operand(fn, "codes", codes, "scales", scales)) return rc;
  if (int rc = check_align(fn, "global_sf_x", global_sf_x, 4)) return rc;
  if (int rc = check_align(fn, "gsf_out", gsf_out, 4)) return rc;
  const size_t need = nvfp4_quantize_swiglu_workspace_bytes(m, k);
  if (global_sf_x == nullptr &&
      (!workspace || workspace_bytes < need || ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN)))
    return fail(NVFP4_ERR_WORKSPACE, "%s: the dynamic scale needs a %d-byte aligned workspace of %zu bytes", fn,
                NVFP4_WORKSPACE_ALIGN, need);
  void* xbuf = global_sf_x == nullptr ? static_cast<uint8_t*>(workspace) + nvfp4_quantize_workspace_bytes() : nullptr;
  return quantize_impl(fn, gate, m, k, global_sf_x, 0, codes, scales, gsf_out, static_cast<float*>(workspace),
                       static_cast<hipStream_t>(stream), 1, up, xbuf);
}

int nvfp4_linear_swiglu(const void* gate, const void* up, int64_t m, int64_t k, const uint8_t* packed,
                        const uint8_t* inv_scale, const float* global_sf_w, const void* bias, int64_t out_features,
                        const float* global_sf_x, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_linear_swiglu";
  g_err[0] = 0;
  if (m > 0 && !up) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (((uintptr_t)gate | (uintptr_t)up) % 16) return fail(NVFP4_ERR_ARG, "%s: gate and up must be 16-byte aligned", fn);
  return linear_impl(fn, gate, 1, m, k, packed, inv_scale, global_sf_w, bias, out_features, global_sf_x, 0, out,
                     nullptr, workspace, workspace_bytes, static_cast<hipStream_t>(stream), up);
}

int nvfp4_dequantize(const uint8_t* packed, const uint8_t* scales, int64_t rows, int64_t k, const float* global_sf,
                     void* out, int out_dtype, void* stream) {
  const char* fn = "nvfp4_dequantize";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, rows, k, true)) return rc;
  if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_F32)
    return fail(NVFP4_ERR_ARG, "%s: out_dtype must be NVFP4_DTYPE_BF16 or NVFP4_DTYPE_F32", fn);
  if (rows == 0) return NVFP4_OK;
  if (!packed || !scales || !global_sf || !out) return fail(NVFP4_ERR_ARG, "%s: NULL argument", fn);
  if (((uintptr_t)packed % 8) || ((uintptr_t)out % 16))
    return fail(NVFP4_ERR_ARG, "%s: packed must be 8-byte and out 16-byte aligned", fn);
  if (int rc = check_align(fn, "global_sf", global_sf, 4)) return rc;
  return hip_status(nvfp4::launch_dequant(packed, scales, rows, k, global_sf, out, out_dtype == NVFP4_DTYPE_BF16,
                                          static_cast<hipStream_t>(stream)),
                    fn);
}

int nvfp4_static_global_scale(const float* amax, float margin, float* gsf, void* stream) {
  const char* fn = "nvfp4_static_global_scale";
  Range call(fn);
  g_err[0] = 0;
  if (!amax || !gsf) return fail(NVFP4_ERR_ARG, "%s: NULL argument", fn);
  if (int rc = check_align(fn, "amax", amax, 4)) return rc;
  if (int rc = check_align(fn, "gsf", gsf, 4)) return rc;
  if (!(margin > 0.0f) || margin != margin || margin > 3.0e38f)
    return fail(NVFP4_ERR_ARG, "%s: margin must be a positive finite number", fn);
  return hip_status(nvfp4::launch_static_scale(amax, margin, gsf, static_cast<hipStream_t>(stream)), fn);
}

int nvfp4_quantize_activation_segmented(const void* x, int64_t segments, int64_t seg_rows, int64_t k,
                                        int rotation_group, uint8_t* codes, uint8_t* scales, float* gsf_out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_quantize_activation_segmented";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_segments(fn, segments, seg_rows)) return rc;
  const int64_t m = segments * seg_rows;
  if (int rc = check_rows_k(fn, m, k, true)) return rc;
  if (int rc = check_group(fn, rotation_group, k, true)) return rc;
  if (m == 0) return NVFP4_OK;
  if (!x || !codes || !scales || !gsf_out) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (int rc = check_aligned(fn, "x", x)) return rc;
  if (int rc = check_nvfp4_operand(fn, "codes", codes, "scales", scales)) return rc;
  if (int rc = check_align(fn, "gsf_out", gsf_out, 4)) return rc;
  if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes() ||
      ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN))
    return fail(NVFP4_ERR_WORKSPACE, "%s: need a %d-byte aligned workspace of %zu bytes", fn, NVFP4_WORKSPACE_ALIGN,
                nvfp4_quantize_workspace_bytes());
  return quantize_impl(fn, x, m, k, nullptr, rotation_group, codes, scales, gsf_out, static_cast<float*>(workspace),
                       static_cast<hipStream_t>(stream), segments);
}

int nvfp4_gemm(const uint8_t* x_codes, const uint8_t* x_scale, int64_t m, int64_t k, const uint8_t* packed,
               const uint8_t* inv_scale, int64_t n, const float* gsf_x, const float* gsf_w, const void* bias,
               void* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "nvfp4_gemm";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, m, k, true)) return rc;
  if (n <= 0 || n >= kMaxDim) return fail(NVFP4_ERR_SHAPE, "%s: out_features must be in [1, 2^31), got %lld", fn, (long long)n);
  if (m == 0) return NVFP4_OK;
  if (!x_codes || !x_scale || !packed || !inv_scale || !gsf_x || !gsf_w || !out)
    return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  if (int rc = check_nvfp4_operand(fn, "x_codes", x_codes, "x_scale", x_scale)) return rc;
  if (int rc = check_nvfp4_operand(fn, "packed", packed, "inv_scale", inv_scale)) return rc;
  if (int rc = check_epilogue(fn, out, bias, gsf_x, gsf_w)) return rc;
  if (workspace != nullptr && ((uintptr_t)workspace % NVFP4_WORKSPACE_ALIGN))
    return fail(NVFP4_ERR_WORKSPACE, "%s: workspace must be %d-byte aligned", fn, NVFP4_WORKSPACE_ALIGN);
  return hip_status(nvfp4::launch_gemm(x_codes, x_scale, m, k, packed, inv_scale, n, gsf_x, gsf_w, 0,
                                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(out), workspace,
                                       workspace != nullptr ? workspace_bytes : 0, static_cast<hipStream_t>(stream)),
                    fn);
}

int nvfp4_linear(const void* x, int64_t m, int64_t k, const uint8_t* packed, const uint8_t* inv_scale,
                 const float* global_sf_w, const void* bias, int64_t out_features, const float* global_sf_x,
                 int rotation_group, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  return linear_impl("nvfp4_linear", x, 1, m, k, packed, inv_scale, global_sf_w, bias, out_features, global_sf_x,
                     rotation_group, out, nullptr, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int nvfp4_linear_noalloc(const void* x, int64_t m, int64_t k, const uint8_t* packed, const uint8_t* inv_scale,
                         const float* global_sf_w, const void* bias, int64_t out_features, const float* global_sf_x,
                         int rotation_group, void* out, void* stream) {
  const char* fn = "nvfp4_linear_noalloc";
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, m, k, true)) return rc;
  if (out_features <= 0 || out_features >= kMaxDim)
    return fail(NVFP4_ERR_SHAPE, "%s: out_features must be in [1, 2^31), got %lld", fn, (long long)out_features);
  if (m == 0) return NVFP4_OK;
  // the whole nvfp4_linear workspace when it fits, else the one without split-K partials
  const bool split_k = carve(nullptr, m, k, out_features).bytes <= NVFP4_NOALLOC_SCRATCH_BYTES;
  const size_t need = carve(nullptr, m, k, out_features, 1, split_k).bytes;
  if (need > NVFP4_NOALLOC_SCRATCH_BYTES)
    return fail(NVFP4_ERR_WORKSPACE,
                "%s: an [%lld, %lld] input needs %zu bytes of scratch, more than the fixed %zu; call nvfp4_linear "
                "with a workspace instead",
                fn, (long long)m, (long long)k, need, (size_t)NVFP4_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = scratch_of_current_device(fn, &ws)) return rc;
  return linear_impl(fn, x, 1, m, k, packed, inv_scale, global_sf_w, bias, out_features, global_sf_x, rotation_group,
                     out, nullptr, ws, NVFP4_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream), nullptr,
                     split_k);
}

int nvfp4_linear_segmented(const void* x, int64_t segments, int64_t seg_rows, int64_t k, const uint8_t* packed,
                           const uint8_t* inv_scale, const float* global_sf_w, const void* bias, int64_t out_features,
                           int rotation_group, void* out, float* gsf_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const char* fn = "nvfp4_linear_segmented";
  g_err[0] = 0;
  if (int rc = check_segments(fn, segments, seg_rows)) return rc;
  return linear_impl(fn, x, segments, seg_rows, k, packed, inv_scale, global_sf_w, bias, out_features, nullptr,
                     rotation_group, out, gsf_out, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int nvfp4_scale_to_canonical(const uint8_t* layout, uint8_t* canonical, int64_t rows, int64_t k, void* stream) {
  const char* fn = "nvfp4_scale_to_canonical";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, rows, k, true)) return rc;
  if (rows == 0) return NVFP4_OK;
  if (!layout || !canonical) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  return hip_status(nvfp4::launch_scale_layout(layout, canonical, rows, k, true, static_cast<hipStream_t>(stream)), fn);
}

int nvfp4_scale_from_canonical(const uint8_t* canonical, uint8_t* layout, int64_t rows, int64_t k, void* stream) {
  const char* fn = "nvfp4_scale_from_canonical";
  Range call(fn);
  g_err[0] = 0;
  if (int rc = check_rows_k(fn, rows, k, true)) return rc;
  if (rows == 0) return NVFP4_OK;
  if (!layout || !canonical) return fail(NVFP4_ERR_ARG, "%s: NULL tensor argument", fn);
  return hip_status(nvfp4::launch_scale_layout(canonical, layout, rows, k, false, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
