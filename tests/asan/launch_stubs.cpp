// Host-only stand-ins for the kernel launchers of libnvfp4, for a sanitizer build of the host layer
// (api.hip) on a machine without a GPU.  Every launcher does nothing and reports success, so a call
// that passes validation returns NVFP4_OK without touching a device; the sanitizers then watch the
// host layer's own reads of its arguments (segment offsets, tables) and its arithmetic.
#include "nvfp4_internal.h"

namespace nvfp4 {

hipError_t launch_quantize(const void*, nvfp4_dtype, int64_t, int64_t, int64_t, float*, int,
                           uint8_t*, uint8_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_silu_mul_quantize(const void*, const void*, nvfp4_dtype, int64_t, int64_t,
                                    int64_t, int64_t, float*, int, uint8_t*, uint8_t*,
                                    hipStream_t) {
  return hipSuccess;
}
hipError_t launch_dynamic_amax(const void*, nvfp4_dtype, int64_t, int64_t, int64_t, float*,
                               hipStream_t) {
  return hipSuccess;
}
hipError_t launch_finalize_dynamic(float*, hipStream_t) { return hipSuccess; }
hipError_t launch_fake_quantize(const void*, nvfp4_dtype, int64_t, int64_t, int64_t, float*, int,
                                void*, nvfp4_dtype, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_quant_error_stats(const void*, nvfp4_dtype, int64_t, int64_t, int64_t, float*,
                                    int, double*, double*, int32_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_requantize(const uint8_t*, const uint8_t*, int64_t, int64_t, const SegTable& seg,
                             const float*, const float*, float*, uint8_t*, uint8_t*,
                             hipStream_t) {
  // the table the host layer built must be well formed
  if (seg.nseg < 1 || seg.nseg > NVFP4_MAX_SEGMENTS) return hipErrorInvalidValue;
  return hipSuccess;
}
hipError_t launch_kv_store(const void*, const void*, nvfp4_dtype, int64_t, int64_t, int64_t,
                           int64_t, const float*, const float*, const int64_t*, uint8_t*,
                           uint8_t*, int64_t, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_kv_load(const uint8_t*, int64_t, int64_t, int64_t, const float*, const int64_t*,
                          int64_t, void*, nvfp4_dtype, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gemm_tiled(const GemmArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_general(const GemmArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_skinny(const GemmArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_gemm_stream(const GemmArgs&, hipStream_t) { return hipSuccess; }
bool skinny_one_pass(int64_t M, int64_t N, int64_t K, int) {
  return M >= 1 && M <= 16 && K % 1024 == 0 && K <= kSkinnyMaxK && N <= 32 * 256;
}
hipError_t launch_gemm_skinny_encode(const GemmArgs&, const void*, nvfp4_dtype, int64_t, uint8_t*,
                                     uint8_t*, hipStream_t) {
  return hipSuccess;
}
GemmPath choose_gemm_path(int64_t M, int64_t K, bool) {
  return M <= 16 ? GemmPath::Skinny : (K % 64 == 0 ? GemmPath::Tiled : GemmPath::General);
}

}  // namespace nvfp4
