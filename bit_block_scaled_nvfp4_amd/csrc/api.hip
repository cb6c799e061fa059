// Host layer of libnvfp4: argument validation (before any HIP call), kernel selection, launch.
// The entry points and their contracts are declared in include/nvfp4.h.
#include <stdint.h>

#include "nvfp4_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t dtype_bytes(nvfp4_dtype d) { return d == NVFP4_F32 ? 4 : 2; }

bool valid_in_dtype(int d) { return d == NVFP4_F32 || d == NVFP4_BF16 || d == NVFP4_F16; }

bool valid_out_dtype(int d) { return d == NVFP4_F32 || d == NVFP4_BF16; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

// Largest extent (elements) a tensor may span from its base pointer, and the widest KV row.
constexpr int64_t kMaxSpan = int64_t(1) << 40;
constexpr int64_t kMaxKvWidth = int64_t(1) << 24;

nvfp4_status device_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_EDEVICE; }

// Validation shared by nvfp4_gemm and fused_nvfp4_gemm.
nvfp4_status check_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* seg_gscale,
                        const int64_t* seg_offsets, int nseg, int64_t M, int64_t N, int64_t K,
                        const void* c, int c_dtype, int64_t ldc) {
  if (!a_gscale || !seg_gscale || !seg_offsets) return NVFP4_EINVAL;
  // operands of an empty product may have no storage
  if (M != 0 && (!a_codes || !a_scales)) return NVFP4_EINVAL;
  if (N != 0 && (!w_codes || !w_scales)) return NVFP4_EINVAL;
  if (M != 0 && N != 0 && !c) return NVFP4_EINVAL;
  if (!valid_out_dtype(c_dtype)) return NVFP4_EINVAL;
  if (nseg < 1 || nseg > NVFP4_MAX_SEGMENTS) return NVFP4_EINVAL;
  if (M < 0 || N < 0 || K <= 0 || K % 16 != 0) return NVFP4_ESHAPE;
  if (M > kMaxDim || N > kMaxDim || K >= (int64_t(1) << 24)) return NVFP4_ESHAPE;
  // each operand's codes must stay below 2 GiB (32-bit row offsets inside the kernels)
  if (M * (K / 2) >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (ldc < N || ldc < 1) return NVFP4_ESHAPE;
  if (M * ldc > (int64_t(1) << 40)) return NVFP4_ESHAPE;
  if (seg_offsets[0] != 0 || seg_offsets[nseg] != N) return NVFP4_ESHAPE;
  for (int j = 0; j < nseg; ++j) {
    const bool empty_problem = (N == 0 && nseg == 1);
    if (!(seg_offsets[j + 1] > seg_offsets[j]) && !empty_problem) return NVFP4_ESHAPE;
  }
  if (!aligned(a_codes, 16) || !aligned(a_scales, 16) || !aligned(w_codes, 16) ||
      !aligned(w_scales, 16) || !aligned(c, 16) || !aligned(a_gscale, 4) ||
      !aligned(seg_gscale, 4))
    return NVFP4_EALIGN;
  return NVFP4_OK;
}

nvfp4::GemmArgs gemm_args(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                          const uint8_t* w_codes, const uint8_t* w_scales, const float* seg_gscale,
                          const int64_t* seg_offsets, int nseg, int64_t M, int64_t N, int64_t K,
                          void* c, nvfp4_dtype c_dtype, int64_t ldc) {
  nvfp4::GemmArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.a_g = a_gscale;
  a.w_codes = w_codes;
  a.w_scales = w_scales;
  a.seg_g = seg_gscale;
  a.M = (int32_t)M;
  a.N = (int32_t)N;
  a.K = (int32_t)K;
  a.k_pitch = (int32_t)K;
  a.c = c;
  a.c_bf16 = c_dtype == NVFP4_BF16 ? 1 : 0;
  a.c_accumulate = 0;
  a.ldc = ldc;
  a.seg.nseg = nseg;
  for (int j = 0; j <= nseg; ++j) a.seg.off[j] = (int32_t)seg_offsets[j];
  for (int j = nseg + 1; j <= NVFP4_MAX_SEGMENTS; ++j) a.seg.off[j] = (int32_t)N;
  return a;
}

nvfp4_status run_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                      const uint8_t* w_codes, const uint8_t* w_scales, const float* seg_gscale,
                      const int64_t* seg_offsets, int nseg, int64_t M, int64_t N, int64_t K,
                      void* c, nvfp4_dtype c_dtype, int64_t ldc, void* stream) {
  const nvfp4::GemmArgs a = gemm_args(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale,
                                      seg_offsets, nseg, M, N, K, c, c_dtype, ldc);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  switch (nvfp4::choose_gemm_path(M, K, a.c_bf16 != 0)) {
    case nvfp4::GemmPath::General:
      e = nvfp4::launch_gemm_general(a, s);
      break;
    case nvfp4::GemmPath::Tiled:
      e = nvfp4::launch_gemm_tiled(a, s);
      break;
    case nvfp4::GemmPath::Skinny:
      e = nvfp4::launch_gemm_skinny(a, s);
      break;
  }
  return device_status(e);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                            int64_t ldx, float* global_scale, int dynamic, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  if (!global_scale) return NVFP4_EINVAL;
  if (!(rows == 0 || cols == 0) && (!x || !codes || !scales)) return NVFP4_EINVAL;
  if (!valid_in_dtype(x_dtype)) return NVFP4_EINVAL;
  if (dynamic != 0 && dynamic != 1) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ESHAPE;
  if (ldx < cols || ldx < 1) return NVFP4_ESHAPE;
  if (rows * (cols / 16) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (rows > 0 && (rows - 1) * ldx + cols > (int64_t(1) << 40)) return NVFP4_ESHAPE;
  if (!aligned(x, 16) || (ldx * dtype_bytes(x_dtype)) % 16 != 0) return NVFP4_EALIGN;
  if (!aligned(codes, 8) || !aligned(global_scale, 4)) return NVFP4_EALIGN;
  if ((rows == 0 || cols == 0) && !dynamic) return NVFP4_OK;
  hipError_t e = nvfp4::launch_quantize(x, x_dtype, rows, cols, ldx, global_scale, dynamic, codes,
                                        scales, reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_silu_mul_quantize(const void* gate, const void* up, nvfp4_dtype dtype,
                                     int64_t rows, int64_t cols, int64_t ld_gate, int64_t ld_up,
                                     float* global_scale, int dynamic, uint8_t* codes,
                                     uint8_t* scales, void* stream) {
  if (!global_scale) return NVFP4_EINVAL;
  if (!(rows == 0 || cols == 0) && (!gate || !up || !codes || !scales)) return NVFP4_EINVAL;
  if (!valid_in_dtype(dtype)) return NVFP4_EINVAL;
  if (dynamic != 0 && dynamic != 1) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ESHAPE;
  if (ld_gate < cols || ld_gate < 1 || ld_up < cols || ld_up < 1) return NVFP4_ESHAPE;
  if (rows * (cols / 16) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (rows > 0 && ((rows - 1) * ld_gate + cols > (int64_t(1) << 40) ||
                   (rows - 1) * ld_up + cols > (int64_t(1) << 40)))
    return NVFP4_ESHAPE;
  if (!aligned(gate, 16) || !aligned(up, 16) || (ld_gate * dtype_bytes(dtype)) % 16 != 0 ||
      (ld_up * dtype_bytes(dtype)) % 16 != 0)
    return NVFP4_EALIGN;
  if (!aligned(codes, 8) || !aligned(global_scale, 4)) return NVFP4_EALIGN;
  if ((rows == 0 || cols == 0) && !dynamic) return NVFP4_OK;
  hipError_t e = nvfp4::launch_silu_mul_quantize(gate, up, dtype, rows, cols, ld_gate, ld_up,
                                                 global_scale, dynamic, codes, scales,
                                                 reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_fake_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                                 int64_t ldx, float* global_scale, int dynamic, void* out,
                                 nvfp4_dtype out_dtype, int64_t ldo, void* stream) {
  if (!global_scale) return NVFP4_EINVAL;
  if (!(rows == 0 || cols == 0) && (!x || !out)) return NVFP4_EINVAL;
  if (!valid_in_dtype(x_dtype) || !valid_out_dtype(out_dtype)) return NVFP4_EINVAL;
  if (dynamic != 0 && dynamic != 1) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ESHAPE;
  if (ldx < cols || ldx < 1 || ldo < cols || ldo < 1) return NVFP4_ESHAPE;
  if (rows * (cols / 16) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (rows > 0 && ((rows - 1) * ldx + cols > kMaxSpan || (rows - 1) * ldo + cols > kMaxSpan))
    return NVFP4_ESHAPE;
  if (!aligned(x, 16) || (ldx * dtype_bytes(x_dtype)) % 16 != 0) return NVFP4_EALIGN;
  if (!aligned(out, 16) || (ldo * dtype_bytes(out_dtype)) % 16 != 0) return NVFP4_EALIGN;
  if (!aligned(global_scale, 4)) return NVFP4_EALIGN;
  if ((rows == 0 || cols == 0) && !dynamic) return NVFP4_OK;
  hipError_t e = nvfp4::launch_fake_quantize(x, x_dtype, rows, cols, ldx, global_scale, dynamic,
                                             out, out_dtype, ldo,
                                             reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_quant_error_stats(const void* x, nvfp4_dtype x_dtype, int64_t rows,
                                     int64_t cols, int64_t ldx, float* global_scale, int dynamic,
                                     double* err2, double* norm2, int32_t* dominated,
                                     void* stream) {
  if (!global_scale) return NVFP4_EINVAL;
  if (rows != 0 && (!err2 || !norm2 || !dominated)) return NVFP4_EINVAL;
  if (!(rows == 0 || cols == 0) && !x) return NVFP4_EINVAL;
  if (!valid_in_dtype(x_dtype)) return NVFP4_EINVAL;
  if (dynamic != 0 && dynamic != 1) return NVFP4_EINVAL;
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ESHAPE;
  if (ldx < cols || ldx < 1) return NVFP4_ESHAPE;
  if (rows * (cols / 16) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (rows > 0 && (rows - 1) * ldx + cols > kMaxSpan) return NVFP4_ESHAPE;
  if (!aligned(x, 16) || (ldx * dtype_bytes(x_dtype)) % 16 != 0) return NVFP4_EALIGN;
  if (!aligned(err2, 8) || !aligned(norm2, 8) || !aligned(dominated, 4) ||
      !aligned(global_scale, 4))
    return NVFP4_EALIGN;
  if (rows == 0 && !dynamic) return NVFP4_OK;
  hipError_t e = nvfp4::launch_quant_error_stats(x, x_dtype, rows, cols, ldx, global_scale,
                                                 dynamic, err2, norm2, dominated,
                                                 reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_requantize(const uint8_t* codes, const uint8_t* scales, const float* g_in,
                              const float* g_out, int64_t rows, int64_t cols, uint8_t* codes_out,
                              uint8_t* scales_out, void* stream) {
  if (!g_in || !g_out) return NVFP4_EINVAL;
  if (rows != 0 && cols != 0 && (!codes || !scales || !codes_out || !scales_out))
    return NVFP4_EINVAL;
  if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ESHAPE;
  if (rows > kMaxDim || rows * (cols / 16) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (!aligned(codes, 8) || !aligned(codes_out, 8) || !aligned(g_in, 4) || !aligned(g_out, 4))
    return NVFP4_EALIGN;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  nvfp4::SegTable seg{};
  seg.nseg = 1;
  seg.off[0] = 0;
  for (int j = 1; j <= NVFP4_MAX_SEGMENTS; ++j) seg.off[j] = (int32_t)rows;
  hipError_t e = nvfp4::launch_requantize(codes, scales, rows, cols, seg, g_in, g_out, nullptr,
                                          codes_out, scales_out,
                                          reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_harmonize_segments(const uint8_t* codes, const uint8_t* scales,
                                      const float* seg_gscale, const int64_t* seg_offsets,
                                      int nseg, int64_t N, int64_t K, float* shared_gscale,
                                      uint8_t* codes_out, uint8_t* scales_out, void* stream) {
  if (!seg_gscale || !seg_offsets || !shared_gscale) return NVFP4_EINVAL;
  if (N != 0 && K != 0 && (!codes || !scales || !codes_out || !scales_out)) return NVFP4_EINVAL;
  if (nseg < 1 || nseg > NVFP4_MAX_SEGMENTS) return NVFP4_EINVAL;
  // the shared scale is written while the kernel reads the segment scales
  if (shared_gscale >= seg_gscale && shared_gscale < seg_gscale + nseg) return NVFP4_EINVAL;
  if (N < 0 || K < 0 || K % 16 != 0) return NVFP4_ESHAPE;
  if (N > kMaxDim || N * (K / 16) >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  if (seg_offsets[0] != 0 || seg_offsets[nseg] != N) return NVFP4_ESHAPE;
  for (int j = 0; j < nseg; ++j) {
    const bool empty_problem = (N == 0 && nseg == 1);
    if (!(seg_offsets[j + 1] > seg_offsets[j]) && !empty_problem) return NVFP4_ESHAPE;
  }
  if (!aligned(codes, 8) || !aligned(codes_out, 8) || !aligned(seg_gscale, 4) ||
      !aligned(shared_gscale, 4))
    return NVFP4_EALIGN;
  if (N == 0 || K == 0) return NVFP4_OK;
  nvfp4::SegTable seg{};
  seg.nseg = nseg;
  for (int j = 0; j <= nseg; ++j) seg.off[j] = (int32_t)seg_offsets[j];
  for (int j = nseg + 1; j <= NVFP4_MAX_SEGMENTS; ++j) seg.off[j] = (int32_t)N;
  hipError_t e = nvfp4::launch_requantize(codes, scales, N, K, seg, seg_gscale, nullptr,
                                          shared_gscale, codes_out, scales_out,
                                          reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_kv_fp8_store(const void* key, const void* value, nvfp4_dtype dtype,
                                int64_t tokens, int64_t width, int64_t ld_key, int64_t ld_value,
                                const float* key_scale, const float* value_scale,
                                const int64_t* slot_mapping, uint8_t* key_cache,
                                uint8_t* value_cache, int64_t num_slots, int64_t cache_ld,
                                void* stream) {
  if (!key_scale) return NVFP4_EINVAL;
  // the value tensor is optional: value_scale says whether it is there; then value and
  // value_cache are required (unless the problem is empty), else all three are absent
  const bool has_value = value_scale != nullptr;
  const bool empty = tokens == 0 || width == 0;
  if (!empty && (!key || (!key_cache && num_slots > 0))) return NVFP4_EINVAL;
  if (has_value && !empty && (!value || (!value_cache && num_slots > 0))) return NVFP4_EINVAL;
  if (!has_value && (value || value_cache)) return NVFP4_EINVAL;
  if (!valid_in_dtype(dtype)) return NVFP4_EINVAL;
  if (tokens < 0 || width < 0 || width % 16 != 0 || num_slots < 0) return NVFP4_ESHAPE;
  if (tokens > kMaxDim || width > kMaxKvWidth) return NVFP4_ESHAPE;
  if (ld_key < width || ld_key < 1 || cache_ld < width || cache_ld < 1) return NVFP4_ESHAPE;
  if (has_value && (ld_value < width || ld_value < 1)) return NVFP4_ESHAPE;
  if (tokens > 0 && ((tokens - 1) * ld_key + width > kMaxSpan ||
                     (has_value && (tokens - 1) * ld_value + width > kMaxSpan)))
    return NVFP4_ESHAPE;
  if (num_slots > 0 && (num_slots - 1) * cache_ld + width > kMaxSpan) return NVFP4_ESHAPE;
  const int64_t eb = dtype_bytes(dtype);
  if (!aligned(key, 16) || (ld_key * eb) % 16 != 0 || !aligned(key_cache, 16) ||
      cache_ld % 16 != 0 || !aligned(key_scale, 4))
    return NVFP4_EALIGN;
  if (has_value && (!aligned(value, 16) || (ld_value * eb) % 16 != 0 ||
                    !aligned(value_cache, 16) || !aligned(value_scale, 4)))
    return NVFP4_EALIGN;
  if (slot_mapping && !aligned(slot_mapping, 8)) return NVFP4_EALIGN;
  if (empty) return NVFP4_OK;
  hipError_t e = nvfp4::launch_kv_store(key, value, dtype, tokens, width, ld_key, ld_value,
                                        key_scale, value_scale, slot_mapping, key_cache,
                                        value_cache, num_slots, cache_ld,
                                        reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_kv_fp8_load(const uint8_t* cache, int64_t num_slots, int64_t cache_ld,
                               int64_t width, const float* scale, const int64_t* slot_mapping,
                               int64_t tokens, void* out, nvfp4_dtype out_dtype, int64_t ld_out,
                               void* stream) {
  if (!scale) return NVFP4_EINVAL;
  if (tokens != 0 && width != 0 && (!out || (!cache && num_slots > 0))) return NVFP4_EINVAL;
  if (!valid_out_dtype(out_dtype)) return NVFP4_EINVAL;
  if (tokens < 0 || width < 0 || width % 16 != 0 || num_slots < 0) return NVFP4_ESHAPE;
  if (tokens > kMaxDim || width > kMaxKvWidth) return NVFP4_ESHAPE;
  if (cache_ld < width || cache_ld < 1 || ld_out < width || ld_out < 1) return NVFP4_ESHAPE;
  if (tokens > 0 && (tokens - 1) * ld_out + width > kMaxSpan) return NVFP4_ESHAPE;
  if (num_slots > 0 && (num_slots - 1) * cache_ld + width > kMaxSpan) return NVFP4_ESHAPE;
  if (!aligned(cache, 16) || cache_ld % 16 != 0 || !aligned(out, 16) ||
      (ld_out * dtype_bytes(out_dtype)) % 16 != 0 || !aligned(scale, 4))
    return NVFP4_EALIGN;
  if (slot_mapping && !aligned(slot_mapping, 8)) return NVFP4_EALIGN;
  if (tokens == 0 || width == 0) return NVFP4_OK;
  hipError_t e = nvfp4::launch_kv_load(cache, num_slots, cache_ld, width, scale, slot_mapping,
                                       tokens, out, out_dtype, ld_out,
                                       reinterpret_cast<hipStream_t>(stream));
  return device_status(e);
}

nvfp4_status nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gscale,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gscale,
                        int64_t M, int64_t N, int64_t K, void* c, nvfp4_dtype c_dtype, int64_t ldc,
                        void* stream) {
  const int64_t off[2] = {0, N};
  nvfp4_status st = check_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, off, 1, M,
                               N, K, c, c_dtype, ldc);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  return run_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, off, 1, M, N, K, c,
                  c_dtype, ldc, stream);
}

nvfp4_status fused_nvfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_gscale, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* seg_gscale,
                              const int64_t* seg_offsets, int nseg, int64_t M, int64_t N,
                              int64_t K, void* c, nvfp4_dtype c_dtype, int64_t ldc, void* stream) {
  nvfp4_status st = check_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale,
                               seg_offsets, nseg, M, N, K, c, c_dtype, ldc);
  if (st != NVFP4_OK) return st;
  if (M == 0 || N == 0) return NVFP4_OK;
  return run_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, seg_offsets, nseg, M,
                  N, K, c, c_dtype, ldc, stream);
}

nvfp4_status nvfp4_linear(const void* x, nvfp4_dtype x_dtype, int64_t ldx, const float* a_gscale,
                          uint8_t* a_codes, uint8_t* a_scales, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* seg_gscale,
                          const int64_t* seg_offsets, int nseg, int64_t M, int64_t N, int64_t K,
                          void* c, nvfp4_dtype c_dtype, int64_t ldc, void* stream) {
  nvfp4_status st = check_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale,
                               seg_offsets, nseg, M, N, K, c, c_dtype, ldc);
  if (st != NVFP4_OK) return st;
  if (M != 0 && !x) return NVFP4_EINVAL;
  if (!valid_in_dtype(x_dtype)) return NVFP4_EINVAL;
  if (ldx < K || ldx < 1) return NVFP4_ESHAPE;
  if (M > 0 && (M - 1) * ldx + K > kMaxSpan) return NVFP4_ESHAPE;
  if (!aligned(x, 16) || (ldx * dtype_bytes(x_dtype)) % 16 != 0) return NVFP4_EALIGN;
  if (M == 0) return NVFP4_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (N > 0 && nvfp4::choose_gemm_path(M, K, c_dtype == NVFP4_BF16) == nvfp4::GemmPath::Skinny &&
      nvfp4::skinny_one_pass(M, N, K, x_dtype)) {
    nvfp4::GemmArgs a = gemm_args(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale,
                                  seg_offsets, nseg, M, N, K, c, c_dtype, ldc);
    return device_status(
        nvfp4::launch_gemm_skinny_encode(a, x, x_dtype, ldx, a_codes, a_scales, s));
  }
  hipError_t e = nvfp4::launch_quantize(x, x_dtype, M, K, ldx, const_cast<float*>(a_gscale), 0,
                                        a_codes, a_scales, s);
  if (e != hipSuccess) return NVFP4_EDEVICE;
  if (N == 0) return NVFP4_OK;
  return run_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, seg_offsets, nseg, M,
                  N, K, c, c_dtype, ldc, stream);
}

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK:
      return "NVFP4_OK: success";
    case NVFP4_EINVAL:
      return "NVFP4_EINVAL: null pointer, unknown dtype, bad flag or segment count";
    case NVFP4_ESHAPE:
      return "NVFP4_ESHAPE: bad size, leading dimension, K not a multiple of 16, or segment offsets";
    case NVFP4_EALIGN:
      return "NVFP4_EALIGN: pointer or row pitch not aligned as required";
    case NVFP4_EDEVICE:
      return "NVFP4_EDEVICE: the HIP runtime reported an error";
  }
  return "NVFP4: unknown status";
}

int nvfp4_version(void) { return 200; }

}  // extern "C"
