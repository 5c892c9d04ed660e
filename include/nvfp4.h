/*
 * nvfp4.h - C ABI of libnvfp4.so, the NVFP4 W4A4 linear on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute follows the pages on FastVideo's NVFP4 path, cited by title:
 *   [DEC]  "minimax_h3_nvfp4_decoder" (API reference of
 *          fastvideo.models.vaes.minimax_h3_nvfp4_decoder): rotate_activation,
 *          nvfp4_linear_inference, NVFP4DecoderLinear.
 *   [CONV] "convert_minimax_h3_text_encoder_nvfp4.py": quantize_language_linear,
 *          probe_relative_error, main.
 *   [BLOG] "FastH3-QAD-v2 and NVFP4 VAE Decoders: Better Quality, Faster Decoding,
 *          and Community LoRAs", section "The whole stack in NVFP4".
 *
 * Number formats.  FP4 is E2M1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 is the
 * sign).  Two codes per byte, the even K index in the low nibble, row-major
 * [rows][K/2] ([DEC] NVFP4DecoderLinear.from_packed).  One FP8 E4M3 (bias 7,
 * finite max 448) scale per 16 consecutive K values of a row ([BLOG]).  One fp32
 * global scale per tensor, gsf = 2688 / max(amax, 1e-12) with 2688 = 6 * 448
 * ([DEC] NVFP4DecoderLinear._activation_global_sf).  A value v quantizes to
 *     s    = E4M3_nearest_even_saturating((gsf * bmax) / 6)   (bmax: block max |v|)
 *     code = E2M1_nearest_even_saturating(v * (gsf / s))      (all codes 0 if s == 0)
 * every operation in IEEE fp32 round-to-nearest.
 *
 * Scale layout.  Block scales are stored k-tile-major: byte (row r, block b) sits at
 *     ((b / 8) * rows + r) * 8 + (b % 8)
 * i.e. [ceil(K/128)][rows][8]; a 128-wide K tile of every row is one contiguous run.
 * Bytes for blocks past K/16 (when K % 128 != 0) are padding and are written as 0.
 * nvfp4_scale_bytes() gives the size; nvfp4_scale_to_canonical /
 * nvfp4_scale_from_canonical convert to and from row-major [rows][K/16].
 *
 * Memory and streams.  Every pointer named *_dev is device memory owned by the
 * caller; the library never allocates or frees.  Global scales are fp32 device
 * scalars, so the dynamic path never waits on the host.  Every call is
 * asynchronous on `stream` (a hipStream_t; NULL is the default stream); it returns
 * once its kernels are queued.
 *
 * Errors.  Calls return NVFP4_OK (0) or a negative code before anything is queued;
 * nvfp4_last_error() then gives a message (per calling thread).  Argument checks
 * mirror the ValueErrors of [DEC] NVFP4DecoderLinear.__init__ and .from_packed.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  NVFP4_OK = 0,
  NVFP4_ERR_SHAPE = -1,      /* K not a multiple of 16, non-positive sizes, size overflow */
  NVFP4_ERR_ARG = -2,        /* bad rotation group, dtype, or a required NULL pointer */
  NVFP4_ERR_WORKSPACE = -3,  /* workspace too small or misaligned */
  NVFP4_ERR_HIP = -4         /* the HIP runtime refused a launch */
};

enum { NVFP4_DTYPE_BF16 = 0, NVFP4_DTYPE_F32 = 1 };

#define NVFP4_BLOCK_SIZE 16
#define NVFP4_SCALE_TILE_K 128
#define NVFP4_MAX_ROTATION_GROUP 128
#define NVFP4_WORKSPACE_ALIGN 256
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)   /* nvfp4_linear_noalloc's fixed device scratch */

/* Alignment.  Every call checks its pointers and returns NVFP4_ERR_ARG for a misaligned
 * one, before anything is queued:
 *   - bf16 / fp32 inputs (x, w, gate, up, rotate_activation's x and y, nvfp4_swiglu's
 *     x, nvfp4_dequantize's out): 16 bytes;
 *   - packed codes and block-scale arrays (packed, inv_scale, codes, scales, x_codes,
 *     x_scale): 8 bytes (nvfp4_dequantize reads its scales byte by byte: any address);
 *   - bf16 outputs and biases of the linear and GEMM calls (out, bias): 2 bytes (the
 *     kernels take wide stores and loads only where the address allows them);
 *   - fp32 scalars (global scales, gsf_out, amax): 4 bytes;
 *   - workspaces: NVFP4_WORKSPACE_ALIGN.
 * The scale-layout converters access bytes and need no alignment. */

/* Bytes of a block-scale array for a [rows, k] tensor in the layout above. */
size_t nvfp4_scale_bytes(int64_t rows, int64_t k);

/* Workspace nvfp4_quantize_activation / nvfp4_quantize_weight need (amax partials). */
size_t nvfp4_quantize_workspace_bytes(void);

/* Workspace nvfp4_linear needs for an [m, k] input and n outputs: activation codes
 * [m][k/2], their scales, amax partials, the activation global scale, the GEMM's
 * split-K partial sums (nvfp4_gemm_workspace_bytes) and, for m <= 4, the quantized
 * activation in fp16 [m][k] (the decode GEMM then expands only the weight), each
 * 256-byte aligned.  Depends on the compute-unit count of the current device. */
size_t nvfp4_linear_workspace_bytes(int64_t m, int64_t k, int64_t n);

/* Workspace nvfp4_linear_segmented needs for `segments` row blocks of seg_rows rows:
 * the nvfp4_linear workspace of the whole [segments * seg_rows, k] input with one
 * global-scale slot per segment.  0 for segments outside [1, 1024]. */
size_t nvfp4_linear_segmented_workspace_bytes(int64_t segments, int64_t seg_rows, int64_t k, int64_t n);

/* Workspace nvfp4_gemm can use for an [m, k] x [n, k] product (fp32 partial sums of
 * output tiles split along K to fill the GPU); 0 when the product would not split.
 * Depends on the compute-unit count of the current device. */
size_t nvfp4_gemm_workspace_bytes(int64_t m, int64_t k, int64_t n);

/*
 * rotate_activation ([DEC] rotate_activation(x, group_size); module docstring).
 * y[r, j*g:(j+1)*g] = x[r, j*g:(j+1)*g] @ (H_g / sqrt(g)), H_g the natural-order
 * Sylvester Hadamard matrix, computed in fp32 (butterfly strides 1, 2, ..., g/2, then
 * one multiply by fp32(1/sqrt(g))) and rounded to y_dtype (bf16: nearest even).
 * x_dev, y_dev: row-major [rows][k] of x_dtype / y_dtype (NVFP4_DTYPE_*); may alias
 * only if identical and of equal dtype.  group_size: a power of two, 2..128,
 * dividing k.  bf16 -> bf16 is the activation path; f32 -> bf16 is the weight fold of
 * [DEC] NVFP4DecoderLinear.from_linear followed by the cast of _packed_weight.
 */
int rotate_activation(const void* x_dev, int x_dtype, void* y_dev, int y_dtype,
                      int64_t rows, int64_t k, int group_size, void* stream);

/*
 * nvfp4_quantize_weight ([DEC] NVFP4DecoderLinear._packed_weight; [CONV]
 * quantize_language_linear).  w_dev: bf16 [n][k].  Writes packed_dev [n][k/2],
 * inv_scale_dev (nvfp4_scale_bytes(n, k), layout above) and *global_sf_w_dev =
 * 2688 / max(amax(w), 1e-12).  workspace: >= nvfp4_quantize_workspace_bytes().
 */
int nvfp4_quantize_weight(const void* w_dev, int64_t n, int64_t k,
                          uint8_t* packed_dev, uint8_t* inv_scale_dev, float* global_sf_w_dev,
                          void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_quantize_activation: steps 1-3 of [DEC] nvfp4_linear_inference on a bf16
 * [m][k] input.  rotation_group 0 = none, else x is first rotated as by
 * rotate_activation (the rotated values are never written).  global_sf_x_dev NULL =
 * dynamic scale from the amax of the (rotated) input; else the fp32 scale it points
 * to is used as is (static / unit scale).  Writes codes_dev [m][k/2], scale_dev
 * (nvfp4_scale_bytes(m, k)) and, if gsf_out_dev is not NULL, the scale used.
 */
int nvfp4_quantize_activation(const void* x_dev, int64_t m, int64_t k,
                              const float* global_sf_x_dev, int rotation_group,
                              uint8_t* codes_dev, uint8_t* scale_dev, float* gsf_out_dev,
                              void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_amax: the activation abs-max the calibration of static scales records ([DEC]
 * NVFP4DecoderLinear._activation_global_sf while calibrating, calibrate_static_scales):
 * max |v| over the bf16 [rows][k] input, after the optional rotation (rotation_group
 * 0 = none; the rotated values are never written).  accumulate 0: *amax_dev = that
 * maximum; else *amax_dev = max(*amax_dev, it), folding one batch into a running
 * record.  rows == 0 contributes 0.  workspace >= nvfp4_quantize_workspace_bytes().
 */
int nvfp4_amax(const void* x_dev, int64_t rows, int64_t k, int rotation_group, float* amax_dev, int accumulate,
               void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_static_global_scale: the static activation scale of [DEC]
 * _activation_global_sf from a calibrated abs-max, with calibrate_static_scales'
 * margin applied to the stored range first: *gsf_dev = fp32(2688 / max(fp32(*amax_dev
 * * margin), 1e-12)).  margin > 0 (1 = the recorded range as is).  The result is the
 * global_sf_x argument of nvfp4_linear / nvfp4_quantize_activation for a static scale.
 */
int nvfp4_static_global_scale(const float* amax_dev, float margin, float* gsf_dev, void* stream);

/*
 * nvfp4_quantize_activation_segmented: nvfp4_quantize_activation with a dynamic scale
 * applied separately to `segments` consecutive row blocks of seg_rows rows each, as
 * `segments` separate calls would ([TILES]: a dynamic-scale decoder takes one global
 * scale per tile).  x_dev bf16 [segments * seg_rows][k]; codes_dev / scale_dev as for
 * the whole input (scale layout with segments * seg_rows rows); gsf_out_dev receives
 * `segments` fp32 scales.  segments: 1..1024.
 */
int nvfp4_quantize_activation_segmented(const void* x_dev, int64_t segments, int64_t seg_rows, int64_t k,
                                        int rotation_group, uint8_t* codes_dev, uint8_t* scale_dev,
                                        float* gsf_out_dev, void* workspace_dev, size_t workspace_bytes,
                                        void* stream);

/*
 * nvfp4_gemm: step 4 of [DEC] nvfp4_linear_inference (the mm_fp4 call and the bias
 * add).  out[i, j] = bf16(alpha * sum_b sx[i,b] sw[j,b] sum_{k in b} qx[i,k] qw[j,k]),
 * alpha = 1 / (gsf_x * gsf_w) in fp32; then, if bias_dev is not NULL,
 * out = bf16(out + bias[j]).  Accumulation is fp32 (order unspecified).
 * x_codes_dev [m][k/2], x_scale_dev (layout above, m rows), packed_dev [n][k/2],
 * inv_scale_dev (n rows), gsf_x_dev / gsf_w_dev fp32 device scalars,
 * bias_dev bf16 [n] or NULL, out_dev bf16 [m][n].  workspace_dev: NULL, or 256-byte
 * aligned device memory; with nvfp4_gemm_workspace_bytes(m, k, n) bytes the tiles of
 * the last partial round are split along K (a deterministic, fixed-order sum), without
 * it they are not split.  The result is the same function either way (fp32
 * accumulation order differs).
 */
int nvfp4_gemm(const uint8_t* x_codes_dev, const uint8_t* x_scale_dev, int64_t m, int64_t k,
               const uint8_t* packed_dev, const uint8_t* inv_scale_dev, int64_t n,
               const float* gsf_x_dev, const float* gsf_w_dev, const void* bias_dev,
               void* out_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_linear ([DEC] nvfp4_linear_inference(x, packed, inv_scale, global_sf_w, bias,
 * out_features, global_sf_x), preceded by the optional rotation of
 * NVFP4DecoderLinear.forward).  x_dev: bf16 [m][k] (leading dimensions flattened by
 * the caller).  packed_dev [out_features][k/2] and inv_scale_dev from
 * nvfp4_quantize_weight; global_sf_w_dev its fp32 scale.  bias_dev bf16
 * [out_features] or NULL.  global_sf_x_dev NULL = dynamic activation scale.
 * rotation_group 0 = none; otherwise the result is bit-identical to
 * nvfp4_linear(rotate_activation(x, g), ..., 0).  out_dev bf16 [m][out_features].
 * workspace: >= nvfp4_linear_workspace_bytes(m, k, out_features), 256-byte aligned.
 */
int nvfp4_linear(const void* x_dev, int64_t m, int64_t k,
                 const uint8_t* packed_dev, const uint8_t* inv_scale_dev,
                 const float* global_sf_w_dev, const void* bias_dev, int64_t out_features,
                 const float* global_sf_x_dev, int rotation_group, void* out_dev,
                 void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_linear_noalloc: nvfp4_linear for callers that cannot allocate memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same result.  Instead of a caller workspace it
 * uses a fixed device array of NVFP4_NOALLOC_SCRATCH_BYTES that the library holds on
 * every device it runs on until the process ends; the call itself allocates nothing.
 *   - Size limit: the call succeeds when the nvfp4_linear workspace without its split-K
 *     region fits (activation codes m*k/2 and scales nvfp4_scale_bytes(m, k), plus
 *     64 KiB, plus 2*m*k bytes when m <= 4; about m*k <= 119 M values).  When
 *     nvfp4_linear_workspace_bytes(m, k, out_features) itself fits, the output is
 *     bit-identical to nvfp4_linear's; otherwise the GEMM's last round of tiles runs
 *     unsplit (the same function, fp32 summation order aside).  Larger inputs return
 *     NVFP4_ERR_WORKSPACE before anything is queued.
 *   - Every call on a device shares that device's array, and nothing in it needs to
 *     start at zero (each call writes what it reads).  Calls that overlap on one device
 *     (other streams, other threads) race on it: serialise them.
 *   - The first call on a device looks the array's address up (no allocation); make it
 *     outside graph capture.
 */
int nvfp4_linear_noalloc(const void* x_dev, int64_t m, int64_t k,
                         const uint8_t* packed_dev, const uint8_t* inv_scale_dev,
                         const float* global_sf_w_dev, const void* bias_dev, int64_t out_features,
                         const float* global_sf_x_dev, int rotation_group, void* out_dev, void* stream);

/*
 * nvfp4_linear_segmented: `segments` tiles of seg_rows rows through one linear in one
 * pass, each tile with its own dynamic activation scale ([TILES]: batching the 8
 * decoder tiles of a dynamic-scale NVFP4 decoder, which otherwise must decode one tile
 * per call because a shared amax would change every tile's codes).  Row block s of
 * out_dev equals nvfp4_linear on row block s of x_dev alone: the same codes, scales and
 * global scale, the product up to fp32 summation order.  x_dev bf16
 * [segments * seg_rows][k], out_dev bf16 [segments * seg_rows][out_features];
 * gsf_out_dev: NULL or `segments` fp32 (the per-tile scales).  Other arguments as for
 * nvfp4_linear; workspace >= nvfp4_linear_segmented_workspace_bytes.  segments: 1..1024.
 */
int nvfp4_linear_segmented(const void* x_dev, int64_t segments, int64_t seg_rows, int64_t k,
                           const uint8_t* packed_dev, const uint8_t* inv_scale_dev,
                           const float* global_sf_w_dev, const void* bias_dev, int64_t out_features,
                           int rotation_group, void* out_dev, float* gsf_out_dev,
                           void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_swiglu: the SwiGLU product that feeds down_proj ([CONV] module docstring: it
 * carries the widest activation outliers of the layer; --keep-bf16 mlp.down_proj).
 * x[r][i] = bf16(fp32(fp32(g / fp32(1 + exp(-g))) * u)) for g = gate[r][i], u =
 * up[r][i], with exp evaluated in fp32 by Cody-Waite reduction (15-bit ln2 head),
 * a degree-6 Taylor polynomial and an exact 2^n scaling, on an argument clamped to
 * [-80, 80] (within 3 ulps of exp; the steps fix the result bit for bit).
 * gate_dev, up_dev, x_dev: bf16 [rows][k], 16-byte aligned.
 */
int nvfp4_swiglu(const void* gate_dev, const void* up_dev, int64_t rows, int64_t k, void* x_dev, void* stream);

/* Workspaces of nvfp4_quantize_swiglu and nvfp4_linear_swiglu with a dynamic scale:
 * the plain ones plus room for the [m][k] bf16 product, which the amax pass forms once
 * and the quantize pass reads (a static scale needs no room: its single pass forms
 * the product in registers). */
size_t nvfp4_quantize_swiglu_workspace_bytes(int64_t m, int64_t k);
size_t nvfp4_linear_swiglu_workspace_bytes(int64_t m, int64_t k, int64_t n);

/*
 * nvfp4_quantize_swiglu: nvfp4_quantize_activation (no rotation) of
 * nvfp4_swiglu(gate, up) in fewer passes: the same codes, scales and global scale.
 * A static scale (global_sf_x_dev not NULL) quantizes in one pass that forms the
 * product in registers and writes only codes and scales; a dynamic one forms the
 * product in the amax pass (into the workspace) and quantizes it from there, saving
 * the separate SwiGLU pass.  workspace: >= nvfp4_quantize_swiglu_workspace_bytes.
 */
int nvfp4_quantize_swiglu(const void* gate_dev, const void* up_dev, int64_t m, int64_t k,
                          const float* global_sf_x_dev, uint8_t* codes_dev, uint8_t* scale_dev, float* gsf_out_dev,
                          void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_linear_swiglu: down_proj fed by its SwiGLU product, formed inside the
 * quantizer as in nvfp4_quantize_swiglu: bit-identical to
 * nvfp4_linear(nvfp4_swiglu(gate, up), m, k, ..., rotation_group 0).
 * workspace: >= nvfp4_linear_swiglu_workspace_bytes(m, k, out_features) for a
 * dynamic scale, nvfp4_linear_workspace_bytes for a static one.
 */
int nvfp4_linear_swiglu(const void* gate_dev, const void* up_dev, int64_t m, int64_t k,
                        const uint8_t* packed_dev, const uint8_t* inv_scale_dev, const float* global_sf_w_dev,
                        const void* bias_dev, int64_t out_features, const float* global_sf_x_dev, void* out_dev,
                        void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * nvfp4_dequantize: NVFP4 back to real values, the expansion the fused-dequant
 * fallback performs on GPUs that run the linear as a 16-bit GEMM ([TILES] the
 * encoder's fused dequantization flag).  out[r][i] = fp32(code * scale) / global_sf
 * (IEEE fp32), stored as bf16 (nearest even) or fp32 per out_dtype (NVFP4_DTYPE_*).
 * packed_dev [rows][k/2] (8-byte aligned), scale_dev (layout above), global_sf_dev
 * the tensor's fp32 scale, out_dev [rows][k] (16-byte aligned).
 */
int nvfp4_dequantize(const uint8_t* packed_dev, const uint8_t* scale_dev, int64_t rows, int64_t k,
                     const float* global_sf_dev, void* out_dev, int out_dtype, void* stream);

/* Scale-layout conversion: layout above <-> row-major [rows][k/16] bytes. */
int nvfp4_scale_to_canonical(const uint8_t* layout_dev, uint8_t* canonical_dev,
                             int64_t rows, int64_t k, void* stream);
int nvfp4_scale_from_canonical(const uint8_t* canonical_dev, uint8_t* layout_dev,
                               int64_t rows, int64_t k, void* stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
