// Internal declarations shared by the host layer and the kernels of libnvfp4 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// Per-launch segment table, passed by value in the kernel arguments.  Column n belongs to the
// segment j with off[j] <= n < off[j+1]; its epilogue factor is 1 / (gA * seg_g[j]).
struct SegTable {
  int32_t nseg;
  int32_t off[NVFP4_MAX_SEGMENTS + 1];
};

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_g;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* seg_g;
  int32_t M, N, K;
  // elements per row of A and W (codes k_pitch / 2 bytes, scales k_pitch / 16): K, except in the
  // pieces into which the decode-shaped product splits a long K
  int32_t k_pitch;
  void* c;
  int32_t c_bf16;        // 0: f32 output, 1: bf16 output
  int32_t c_accumulate;  // decode-shaped product, f32 output only: 1 adds into C instead of writing
  int64_t ldc;
  SegTable seg;
};

// Kernel launchers (defined next to their kernels).  They return the launch status.
hipError_t launch_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                           float* g, int dynamic, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);
hipError_t launch_silu_mul_quantize(const void* gate, const void* up, nvfp4_dtype dt,
                                    int64_t rows, int64_t cols, int64_t ldg, int64_t ldu,
                                    float* g, int dynamic, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream);
// Dynamic global scale in three steps around an encoding kernel: launch_dynamic_amax clears *cell
// and leaves max|x| in it; the encoding kernel reads it as 2688 / amax (codec::read_global_scale);
// launch_finalize_dynamic then replaces it with that scale.
hipError_t launch_dynamic_amax(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                               int64_t ldx, float* cell, hipStream_t stream);
hipError_t launch_finalize_dynamic(float* cell, hipStream_t stream);
hipError_t launch_fake_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                int64_t ldx, float* g, int dynamic, void* out, nvfp4_dtype out_dt,
                                int64_t ldo, hipStream_t stream);
hipError_t launch_quant_error_stats(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                    int64_t ldx, float* g, int dynamic, double* err2,
                                    double* norm2, int32_t* dominated, hipStream_t stream);
// Re-encode rows [seg.off[j], seg.off[j+1]) from global scale g_in[j] to *g_out, or, when g_out is
// null, to min_j g_in[j] (written to *g_shared when it is not null).
hipError_t launch_requantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, const SegTable& seg, const float* g_in,
                             const float* g_out, float* g_shared, uint8_t* codes_out,
                             uint8_t* scales_out, hipStream_t stream);
hipError_t launch_kv_store(const void* key, const void* value, nvfp4_dtype dt, int64_t tokens,
                           int64_t width, int64_t ld_key, int64_t ld_value, const float* key_scale,
                           const float* value_scale, const int64_t* slots, uint8_t* key_cache,
                           uint8_t* value_cache, int64_t num_slots, int64_t cache_ld,
                           hipStream_t stream);
hipError_t launch_kv_load(const uint8_t* cache, int64_t num_slots, int64_t cache_ld,
                          int64_t width, const float* scale, const int64_t* slots, int64_t tokens,
                          void* out, nvfp4_dtype out_dt, int64_t ld_out, hipStream_t stream);
hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_general(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream);
// Whether the one-pass decode kernel's encoding form serves an M x N x K product on an activation
// of type x_dtype (M <= 16, K a multiple of 1024 up to kSkinnyMaxK -- 5120 for f32 --, at most 32
// columns per compute unit), and that kernel: the raw activation x [M, K] (row pitch ldx elements)
// is encoded with the static scale *a.a_g inside the launch; the codes and scales go to `codes` /
// `scales` (row pitch K/2, K/16).
bool skinny_one_pass(int64_t M, int64_t N, int64_t K, int x_dtype);
hipError_t launch_gemm_skinny_encode(const GemmArgs& a, const void* x, nvfp4_dtype x_dtype,
                                     int64_t ldx, uint8_t* codes, uint8_t* scales,
                                     hipStream_t stream);

// The skinny (decode-shape) kernel keeps a workgroup's 16 weight rows over all of K in LDS
// (9/16 byte per element), in phases of 1024: K up to this bound, a multiple of 1024.
constexpr int64_t kSkinnyMaxK = 8192;
// Largest K of the streaming decode kernel (its LDS holds the activation scales of all of K).
constexpr int64_t kStreamMaxK = 32768;

// Which kernel family serves a problem.  The choice depends on M and K only, never on N, so a
// fused product and its per-segment products run the same kernel with the same accumulation order.
enum class GemmPath { General, Tiled, Skinny };
GemmPath choose_gemm_path(int64_t M, int64_t K, bool c_bf16);
hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream);

}  // namespace nvfp4
