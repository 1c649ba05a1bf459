// Host-only stand-ins for the kernel launchers of libsmlp, for the sanitizer build of the
// C ABI's host code (api.cpp, layout.cpp).  No GPU is involved: every launcher reports
// hipErrorNotReady, so a call that passes validation comes back as SMLP_ERR_HIP.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace smlp {

int launch_skinny_gate_up(const Plan&, const void*, const void*, void*, hipStream_t) { return (int)hipErrorNotReady; }
int launch_skinny_down(const Plan&, const void*, void*, void*, hipStream_t) { return (int)hipErrorNotReady; }
bool decode_layer_eligible(const Plan&) { return false; }
int launch_decode_layer(const Plan&, const void*, const void*, const void*, void*, void*, int, int, hipStream_t) {
  return (int)hipErrorNotReady;
}
int launch_finalize(bool, const float*, int, int, int, void*, int, int, int, hipStream_t) { return (int)hipErrorNotReady; }
int launch_skinny_linear(const SkinnyPlan&, const void*, const void*, void*, int, int, int, int, int, float*,
                         hipStream_t, int) {
  return (int)hipErrorNotReady;
}
int launch_gemm_linear(const GemmPlan&, const void*, const void*, void*, int, int, int, int, int, float*, hipStream_t) {
  return (int)hipErrorNotReady;
}
int launch_restore_logical(const void*, void*, int64_t, int64_t, const int64_t*, int, int, int, hipStream_t) {
  return (int)hipErrorNotReady;
}
int launch_gemm_gate_up(const Plan&, const void*, const void*, void*, hipStream_t) { return (int)hipErrorNotReady; }
int launch_gemm_down(const Plan&, const void*, void*, void*, hipStream_t) { return (int)hipErrorNotReady; }
int launch_fp32_gate_up(const Plan&, const float*, const float*, void*, hipStream_t) { return (int)hipErrorNotReady; }
int launch_fp32_down(const Plan&, const float*, float*, void*, hipStream_t) { return (int)hipErrorNotReady; }
int launch_fp32_layer(const Plan&, const float*, const float*, const float*, float*, hipStream_t) {
  return (int)hipErrorNotReady;
}
int launch_slice_rank(const void*, const void*, void*, void*, int64_t, int64_t, int, int, int, hipStream_t) {
  return (int)hipErrorNotReady;
}
int launch_rms_rescale(const float*, uint16_t*, int64_t, int64_t, hipStream_t) { return (int)hipErrorNotReady; }
int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return (int)hipErrorNotReady;
}

}  // namespace smlp
