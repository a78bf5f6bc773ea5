// sanitize_stubs.cpp -- kernel launchers for a CPU-only build of the library's
// host layer (mha_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The sanitized build checks argument
// validation, workspace arithmetic and error reporting; every launcher here
// reports that no device is present, so nothing reaches a GPU.
#include "mha_internal.h"

namespace mha {

hipError_t launch_attn_f32(const AttnArgs&, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorNoDevice; }
hipError_t launch_attn_mfma(const AttnArgs&, DType, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorNoDevice; }
hipError_t launch_gemm_mfma(const GemmBatch&, DType, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorNoDevice; }
hipError_t launch_gemm_ln(const GemmProblem&, DType, hipStream_t, hipEvent_t, hipEvent_t, hipEvent_t, hipEvent_t) {
  return hipErrorNoDevice;
}
hipError_t launch_proj_attn(const ProjAttnArgs&, DType, hipStream_t, hipEvent_t, hipEvent_t) {
  return hipErrorNoDevice;
}
hipError_t launch_bwd_mfma(const BwdArgs&, DType, hipStream_t, hipEvent_t const*) { return hipErrorNoDevice; }
hipError_t launch_bwd_f32(const BwdArgs&, int, int, hipStream_t, hipEvent_t const*) { return hipErrorNoDevice; }
hipError_t launch_decode_mfma(const DecodeArgs&, DType, hipStream_t, hipEvent_t, hipEvent_t, hipEvent_t, hipEvent_t) {
  return hipErrorNoDevice;
}

hipError_t decode_scratch(void**) { return hipErrorNoDevice; }

}  // namespace mha
