/*
 * nvfp4.h -- C ABI of the NVFP4 W4A4 linear-layer library for AMD Instinct MI355X (gfx950).
 *
 * The library implements the three steps of an NVFP4 W4A4 linear layer as described in
 * "Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid
 * 27B LLM" (arXiv 2609.04098), ai.info AI-summary page:
 *
 *   1. encoding a tensor to NVFP4 -- 4-bit E2M1 values with one FP8 E4M3 scale per 16-element
 *      block, the block's largest value fixing that scale ("Methodology in Plain English"), under
 *      one FP32 global scale per tensor or calibrated module ("Main Findings");
 *   2. the W4A4 product of two NVFP4 operands with FP32 accumulation;
 *   3. fused modules: several calibrated modules concatenated along the output dimension and served
 *      as one product, each output segment divided by its own module's global scale.  Applying the
 *      largest of the modules' global scales to every segment instead is the serving defect that
 *      "Main Findings" reports (paired scales 1.82x and 2.75x apart); passing a table filled with
 *      that maximum reproduces it.
 *
 * Number format (the pages name the formats; the encoding rules the pages leave open are fixed
 * here and implemented identically by the CPU oracle used in the tests):
 *   - E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code = sign << 3 | magnitude index.
 *   - E4M3 is OCP e4m3fn (bias 7, max 448, no infinities); 0x7F is never produced.
 *   - g: FP32 global scale, encode direction (value ~= V * sd / g).  Dynamic g = 2688 / amax(x)
 *     (2688 = 6 * 448), or 1 when the tensor is all zeros.
 *   - per block of 16 consecutive elements of a row: s = fl(amax_block * fl(g / 6)), rounded to
 *     E4M3 (nearest, ties to even code, >= 448 saturates to 0x7E, subnormals kept); sd = its
 *     value; each element y = fl(|x| * fl(g / sd)) rounded to E2M1 (nearest, ties to even code,
 *     saturating at 6); sd == 0 gives magnitude 0; the sign bit is always copied (so -0.0 -> 0x8).
 *   - layout: codes [rows, cols/2] bytes, element 2j in the low nibble of byte j; scales
 *     [rows, cols/16] E4M3 bytes, row-major, no swizzle.  Blocks run along the row (for the
 *     product: along the contraction dimension K of both operands).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, except the segment-offset arrays of
 *     fused_nvfp4_gemm and nvfp4_harmonize_segments, which are HOST arrays.  The caller owns every buffer; the library
 *     allocates nothing, keeps no mutable global state, is thread-safe, and enqueues its work
 *     asynchronously on `stream` (a hipStream_t; NULL = the null stream).  Nothing synchronises
 *     with the host.
 *   - Every argument check happens on the host before any HIP call: a non-OK status other than
 *     NVFP4_EDEVICE means nothing was enqueued.  NVFP4_EDEVICE reports a HIP launch error.
 *   - Sizes are element counts; leading dimensions (ld*) are in elements of that tensor.
 *   - Empty problems (rows, M or N equal to 0) are valid and enqueue nothing, except that a
 *     dynamic global scale is still written (1, the scale of an all-zero tensor).  The data
 *     pointers of an empty problem may be NULL (an empty tensor may have no storage); global-scale
 *     pointers may not.
 *   - NaN and infinite inputs are unsupported: their codes are unspecified (no error is raised).
 *   - Results are deterministic: identical inputs give identical bits on every call.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_EINVAL = 1,  /* NULL pointer, unknown dtype, nseg out of range, bad flag value         */
  NVFP4_ESHAPE = 2,  /* negative size, cols/K not a multiple of 16, ld < row length, segment
                        offsets not rising strictly from 0 to N, problem too large             */
  NVFP4_EALIGN = 3,  /* a pointer or a row pitch is not aligned as the entry point requires  */
  NVFP4_EDEVICE = 4  /* the HIP runtime reported an error when the work was enqueued         */
} nvfp4_status;

typedef enum nvfp4_dtype {
  NVFP4_F32 = 0,
  NVFP4_BF16 = 1,
  NVFP4_F16 = 2
} nvfp4_dtype;

/* Largest number of segments (calibrated modules) in one fused product. */
#define NVFP4_MAX_SEGMENTS 16

/*
 * nvfp4_quantize -- encode x[rows, cols] (row pitch ldx elements) to NVFP4.
 *
 * Source: ai.info summary, "Methodology in Plain English" (E2M1 values, E4M3 scale per 16-element
 * block, the block's largest value fixes the scale) and "Main Findings" (one FP32 global scale per
 * module); activations are encoded on every call, weights once offline with the same routine.
 *
 *   x            device, dtype x_dtype (F32, BF16 or F16); 16-byte aligned; ldx * sizeof(elem) a
 *                multiple of 16 bytes; ldx >= cols.
 *   rows, cols   rows >= 0; cols >= 0 and a multiple of 16.
 *   global_scale device, one float.  dynamic == 0: read (static, e.g. calibrated, scale; must be
 *                positive and finite -- not checked, it lives on the device).  dynamic == 1: the
 *                dynamic scale 2688/amax(x) is computed and WRITTEN here (stream-ordered).
 *   codes        device, rows * cols/2 bytes, row pitch cols/2; 8-byte aligned.
 *   scales       device, rows * cols/16 bytes, row pitch cols/16.
 *   stream       hipStream_t.
 * Codes and scales are bit-exact with the rules in the file header.
 */
nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                            int64_t ldx, float* global_scale, int dynamic, uint8_t* codes,
                            uint8_t* scales, void* stream);

/*
 * nvfp4_silu_mul_quantize -- encode the gated MLP activation a = SiLU(gate) * up to NVFP4 in one
 * pass, without writing a: the input of the MLP's down projection.
 *
 * Source: ai.info summary, "Methodology in Plain English" (all linear layers quantized, 192 of
 * them MLP projections, so the down projection's input is encoded on the fly like every other
 * activation).  The pages name no activation function; this entry point takes the reading
 * SiLU(x) = x / (1 + e^-x) and a bfloat16 activation (the model's type):
 *
 *   a = bf16(SiLU(gate) * up)   rounded once, to nearest-even, from the exact real value
 *   codes, scales = the NVFP4 encoding of a, exactly as nvfp4_quantize encodes a BF16 tensor
 *
 * The value is formed in binary32 and, whenever that cannot decide the bfloat16 rounding for
 * certain (within 64 binary32 ulps of a bfloat16 midpoint, |gate| > 16, zero, subnormal or
 * non-finite results), in binary64; the result equals the rounding of the exact value except when
 * the exact value lies within binary64 rounding error of a bfloat16 midpoint.
 *
 *   gate, up     device, [rows, cols] of dtype (F32, BF16 or F16), row pitches ld_gate, ld_up
 *                (elements; >= cols; pitch in bytes a multiple of 16); 16-byte aligned.
 *   rows, cols   rows >= 0; cols >= 0 and a multiple of 16.
 *   global_scale, dynamic, codes, scales, stream: as nvfp4_quantize (the dynamic scale is
 *                2688 / max|a|).
 * Errors as nvfp4_quantize.
 */
nvfp4_status nvfp4_silu_mul_quantize(const void* gate, const void* up, nvfp4_dtype dtype,
                                     int64_t rows, int64_t cols, int64_t ld_gate, int64_t ld_up,
                                     float* global_scale, int dynamic, uint8_t* codes,
                                     uint8_t* scales, void* stream);

/*
 * nvfp4_gemm -- C[m, n] = sum_k a[m,k] * w[n,k] / (gA * gW) for NVFP4 operands; equivalent to
 * fused_nvfp4_gemm with one segment.
 *
 * Source: ai.info summary, "Main Findings" and "Methodology in Plain English" (W4A4: weights and
 * activations both NVFP4); the sum is accumulated in FP32 from exactly decoded products.
 *
 *   a_codes, a_scales   device, activations [M, K] encoded by nvfp4_quantize (pitches K/2, K/16).
 *   a_gscale            device, one float: gA.
 *   w_codes, w_scales   device, weights [N, K] (nn.Linear layout) encoded along K.
 *   w_gscale            device, one float: gW.
 *   M, N, K             M, N >= 0; K > 0 and a multiple of 16; K < 2^24; each operand's codes
 *                       below 2 GiB (M*K/2 and N*K/2 < 2^31).
 *   c                   device, [M, N] with row pitch ldc >= N, dtype c_dtype (F32 or BF16); the
 *                       product is rounded once from FP32 to BF16 when c_dtype is BF16.
 *   Alignment: every code/scale pointer 16-byte aligned and c 16-byte aligned.  K a multiple of 64
 *   selects the tiled kernels; other multiples of 16 take a slower general kernel.
 * Accuracy: |C - exact| <= 1e-4 * sum_k |a*w| / (gA*gW) per element (FP32 accumulation order is
 * unspecified), deterministic across calls.
 */
nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                        int64_t M, int64_t N, int64_t K, void* c, nvfp4_dtype c_dtype, int64_t ldc,
                        void* stream);

/*
 * fused_nvfp4_gemm -- product with a fused weight made of nseg calibrated modules concatenated
 * along N: columns [seg_offsets[j], seg_offsets[j+1]) come from module j, whose weights were
 * encoded with global scale seg_gscale[j]; those columns are divided by gA * seg_gscale[j].
 *
 * Source: ai.info summary, "Main Findings" (one FP32 global scale per module from calibration;
 * in_proj_qkv + z and in_proj_b + a served fused) and "Methodology in Plain English" (the repair of
 * the fused global scales).  Filling seg_gscale with max_j gW[j] reproduces the defect.
 *
 *   seg_gscale   device, nseg floats.
 *   seg_offsets  HOST, nseg + 1 int64: 0 = o_0 < o_1 < ... < o_nseg = N.  Read during the call
 *                only; may be freed on return.
 *   nseg         1 .. NVFP4_MAX_SEGMENTS.
 *   other arguments as nvfp4_gemm.  With N == 0 the offsets must be {0, 0} and nseg == 1.
 * The result equals, bit for bit, the concatenation of one nvfp4_gemm per segment.
 */
nvfp4_status fused_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* seg_gscale,
                              const int64_t* seg_offsets, int nseg, int64_t M, int64_t N,
                              int64_t K, void* c, nvfp4_dtype c_dtype, int64_t ldc, void* stream);

/*
 * nvfp4_linear -- the whole linear layer on a raw activation: encode x [M, K] to NVFP4 with the
 * static (calibrated) global scale *a_gscale, exactly as nvfp4_quantize(..., dynamic = 0) does,
 * writing its codes and scales to a_codes / a_scales, then form the fused product of those codes
 * with the fused weight, exactly as fused_nvfp4_gemm does.
 *
 * Source: ai.info summary, "Methodology in Plain English" (activations quantized on the fly with
 * calibrated scales; W4A4 on every linear layer) and "Main Findings" (decode is weight-bandwidth-
 * bound; fused modules keep their own global scales).  For decode shapes with at most 6 rows (K a
 * multiple of 1024 up to 8192, M * K / 1024 <= 32, at most 32 output columns per compute unit; K
 * up to 5120 for an F32 x) both steps run in one launch: every workgroup encodes the few activation
 * rows itself while its weight bytes stream in, and one of them writes the codes out.  Other
 * shapes, decode shapes with 7 to 16 rows included (where that redundant encode costs more than a
 * launch), run the encoder and the product as two launches.
 *
 *   x, x_dtype, ldx      device activation [M, K] (F32, BF16 or F16), as nvfp4_quantize's x.
 *   a_gscale             device, one float: the static activation scale gA (read only).
 *   a_codes, a_scales    device, [M, K/2] and [M, K/16] (pitches K/2, K/16): receive the codes and
 *                        scales nvfp4_quantize would write; 16-byte aligned.
 *   w_codes .. stream    as fused_nvfp4_gemm.
 * Results: a_codes / a_scales bit-identical to nvfp4_quantize's; C bit-identical to
 * fused_nvfp4_gemm on those codes.  Errors as nvfp4_quantize and fused_nvfp4_gemm; the checks of
 * both run before any launch.
 */
nvfp4_status nvfp4_linear(const void* x, nvfp4_dtype x_dtype, int64_t ldx, const float* a_gscale,
                          uint8_t* a_codes, uint8_t* a_scales, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* seg_gscale,
                          const int64_t* seg_offsets, int nseg, int64_t M, int64_t N, int64_t K,
                          void* c, nvfp4_dtype c_dtype, int64_t ldc, void* stream);

/*
 * nvfp4_fake_quantize -- out = dequantize(quantize(x)): the NVFP4 rounding error injected into a
 * high-precision tensor, without storing codes.
 *
 * Source: ai.info summary, "Methodology in Plain English" (fake quantization: quantize, dequantize,
 * continue in high precision).  Reading: each element is encoded exactly as nvfp4_quantize
 * encodes it and decoded as
 *   out = fl(V * sd / g)     (V * sd is exact; one correctly rounded binary32 division by g;
 *                             the sign bit is copied, so code 0x8 gives -0.0)
 * rounded once more to BF16 (nearest-even) when out_dtype is BF16.
 *
 *   x, x_dtype, rows, cols, ldx, global_scale, dynamic   as nvfp4_quantize.
 *   out          device, [rows, cols] of out_dtype (F32 or BF16), row pitch ldo (elements; >= cols;
 *                a multiple of 16 bytes); 16-byte aligned.  May not overlap x.
 * Errors as nvfp4_quantize.  Bit-exact.
 */
nvfp4_status nvfp4_fake_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                                 int64_t ldx, float* global_scale, int dynamic, void* out,
                                 nvfp4_dtype out_dtype, int64_t ldo, void* stream);

/*
 * nvfp4_quant_error_stats -- per-row statistics of the NVFP4 quantization error of x, the
 * quantities the pages report at NVFP4 granularity.
 *
 * Source: ai.info summary, "Main Findings" (per-token activation error 7.5-9.2 %, weight error
 * 10.5-11.9 %, 10-32 % of 16-element blocks dominated by a single value).  Readings:
 *   err2[r]      = sum_k (xh[r,k] - x[r,k])^2, xh = nvfp4_fake_quantize(x) in binary32, summed in
 *                  binary64 (per-token relative error: sqrt(err2 / norm2); a tensor's error:
 *                  sqrt(sum err2 / sum norm2));
 *   norm2[r]     = sum_k x[r,k]^2 in binary64;
 *   dominated[r] = number of 16-element blocks of row r whose largest magnitude a satisfies
 *                  2 a^2 > (sum of the block's 16 squares), in binary64 with the squares summed in
 *                  element order (all-zero blocks are not dominated).
 * The binary64 sums are deterministic; their summation order is unspecified (relative error below
 * cols * 2^-53).  dominated is exact.
 *
 *   x, x_dtype, rows, cols, ldx, global_scale, dynamic   as nvfp4_quantize.
 *   err2, norm2  device, rows doubles each, 8-byte aligned.
 *   dominated    device, rows int32, 4-byte aligned.
 * Errors as nvfp4_quantize.
 */
nvfp4_status nvfp4_quant_error_stats(const void* x, nvfp4_dtype x_dtype, int64_t rows,
                                     int64_t cols, int64_t ldx, float* global_scale, int dynamic,
                                     double* err2, double* norm2, int32_t* dominated,
                                     void* stream);

/*
 * nvfp4_requantize -- re-encode an NVFP4 tensor from global scale *g_in to *g_out:
 * codes_out, scales_out = quantize(fake-dequantized values of (codes, scales) under g_in, g_out),
 * the dequantized values formed as in nvfp4_fake_quantize.
 *
 * Source: ai.info summary, "Methodology in Plain English" (harmonizing fused global scales on the
 * checkpoint side); the single-module building block of nvfp4_harmonize_segments.
 *
 *   codes, scales        device, [rows, cols/2] and [rows, cols/16], contiguous rows; codes 8-byte
 *                        aligned.
 *   g_in, g_out          device, one float each.
 *   codes_out, scales_out  device, same shapes; may be the input buffers themselves (in place),
 *                        but must not overlap them otherwise.  codes_out 8-byte aligned.
 *   rows >= 0; cols >= 0, a multiple of 16; rows * cols/16 < 2^31.
 * Bit-exact.  Errors: EINVAL (NULL), ESHAPE, EALIGN as above; an empty tensor enqueues nothing.
 */
nvfp4_status nvfp4_requantize(const uint8_t* codes, const uint8_t* scales, const float* g_in,
                              const float* g_out, int64_t rows, int64_t cols, uint8_t* codes_out,
                              uint8_t* scales_out, void* stream);

/*
 * nvfp4_harmonize_segments -- checkpoint-side repair of a fused weight: every module j (rows
 * [seg_offsets[j], seg_offsets[j+1]) of the [N, K] weight, encoded under seg_gscale[j]) is
 * re-encoded as nvfp4_requantize does under the shared scale g* = min_j seg_gscale[j], which is
 * written to *shared_gscale.  The fused product may then use g* for every segment (a
 * fused_nvfp4_gemm table filled with g*, or nvfp4_gemm with g*).
 *
 * Source: ai.info summary, "Methodology in Plain English" (harmonizing fused global scales on the
 * checkpoint side) and "Main Findings" (one calibrated global scale per module; fused serving).
 * Reading: the smallest encode-direction scale belongs to the module with the widest calibrated
 * range, so no block scale of any module saturates when re-encoded under it; the module that owns
 * g* keeps its bytes.
 *
 *   codes, scales, codes_out, scales_out   as nvfp4_requantize, rows = N, cols = K.
 *   seg_gscale   device, nseg floats.
 *   seg_offsets  HOST, nseg + 1 int64 rising strictly from 0 to N (read during the call only).
 *   nseg         1 .. NVFP4_MAX_SEGMENTS.
 *   shared_gscale  device, one float, not one of seg_gscale[0 .. nseg).  Not written when N or K
 *                is 0 (nothing is enqueued).
 * Bit-exact.  Errors as fused_nvfp4_gemm for the segment table; EINVAL when shared_gscale lies
 * inside the seg_gscale table.
 */
nvfp4_status nvfp4_harmonize_segments(const uint8_t* codes, const uint8_t* scales,
                                      const float* seg_gscale, const int64_t* seg_offsets,
                                      int nseg, int64_t N, int64_t K, float* shared_gscale,
                                      uint8_t* codes_out, uint8_t* scales_out, void* stream);

/*
 * nvfp4_kv_fp8_store -- encode new tokens' keys (and values) to FP8 E4M3 under one static scale per
 * tensor and write each token's row into its cache slot.
 *
 * Source: ai.info summary, "Key Contributions" (an FP8 KV cache with calibrated per-layer scales
 * that cost nothing at serving time) and "Main Findings" (static per-tensor FP8 scales: one for the
 * K and one for the V tensor of each of the 16 attention layers).  The pages fix the format and the
 * granularity; the rules below are this library's reading:
 *   - the scale is decode-direction: code c stands for E4M3(c) * scale; an uncalibrated FP8 cache
 *     is scale 1, a calibrated one amax / 448 of calibration data;
 *   - code = sign(y) << 7 | E4M3(|y|), y = fl(x * fl(1 / scale)) in binary32; E4M3 nearest with
 *     ties to the even code, |y| >= 448 saturates to 0x7E, subnormal codes kept; the sign bit is
 *     copied, so -0.0 and negatives that round to zero give 0x80.  Codes are bit-exact.
 *
 *   key, value    device, [tokens, width] of dtype (F32, BF16 or F16), row pitches ld_key,
 *                 ld_value (elements, >= width, a multiple of 16 bytes); 16-byte aligned.  value
 *                 may be absent (keys only): value_scale NULL, and then value and value_cache
 *                 NULL as well.
 *   tokens, width tokens >= 0; width >= 0, a multiple of 16, at most 2^24.
 *   key_scale, value_scale  device, one float each, positive and finite (not checked).
 *   slot_mapping  device, tokens int64 (8-byte aligned), or NULL for slot t = token t.  Token t's
 *                 row goes to cache row slot_mapping[t]; a slot outside [0, num_slots) -- e.g. -1
 *                 for a padding token -- is skipped.  Two tokens with one slot race.
 *   key_cache, value_cache  device, [num_slots, width] bytes with row pitch cache_ld (bytes,
 *                 >= width, a multiple of 16); 16-byte aligned.  A paged cache
 *                 [blocks, block_size, heads, head_dim] is this table with width = heads*head_dim
 *                 and slot = block * block_size + position in block.
 * Errors as nvfp4_quantize; EINVAL also when value_scale is NULL but value or value_cache is not,
 * or value_scale is given for a non-empty problem without value or value_cache.  The cache
 * pointers may be NULL when num_slots is 0 (nothing is stored).
 */
nvfp4_status nvfp4_kv_fp8_store(const void* key, const void* value, nvfp4_dtype dtype,
                                int64_t tokens, int64_t width, int64_t ld_key, int64_t ld_value,
                                const float* key_scale, const float* value_scale,
                                const int64_t* slot_mapping, uint8_t* key_cache,
                                uint8_t* value_cache, int64_t num_slots, int64_t cache_ld,
                                void* stream);

/*
 * nvfp4_kv_fp8_load -- gather cache rows and decode them: out[t, i] = fl(E4M3(cache[slot_t, i]) *
 * scale) in binary32, rounded once to BF16 (nearest-even) when out_dtype is BF16.  The inverse of
 * nvfp4_kv_fp8_store for one tensor (the FP8 cache as attention reads it).
 *
 * Source: as nvfp4_kv_fp8_store.
 *
 *   cache         device, [num_slots, width] bytes, row pitch cache_ld (bytes, a multiple of 16).
 *   scale         device, one float (the tensor's decode-direction scale).
 *   slot_mapping  device int64[tokens] or NULL (slot t); a slot outside [0, num_slots) gives a
 *                 row of zeros.
 *   out           device, [tokens, width] of out_dtype (F32 or BF16), row pitch ld_out (elements,
 *                 a multiple of 16 bytes); 16-byte aligned.
 * Errors as nvfp4_kv_fp8_store.
 */
nvfp4_status nvfp4_kv_fp8_load(const uint8_t* cache, int64_t num_slots, int64_t cache_ld,
                               int64_t width, const float* scale, const int64_t* slot_mapping,
                               int64_t tokens, void* out, nvfp4_dtype out_dtype, int64_t ld_out,
                               void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* nvfp4_status_string(nvfp4_status s);

/* Library version as major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
