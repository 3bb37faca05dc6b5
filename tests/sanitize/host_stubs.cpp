// Stand-ins for the device side of libmxattn, so that the host code (host.cpp: checks,
// plan builder, status and error text) runs under AddressSanitizer and UBSan on a
// machine without a GPU.  The launchers record that they were reached and launch
// nothing; the one HIP copy the host code makes (the plan) becomes a host memcpy into
// the harness's own buffer.  Built by tests/test_sanitizers.py with g++.
#include <hip/hip_runtime.h>
#include <string.h>

#include "kernels.h"

int g_launches = 0;

extern "C" {
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  memcpy(dst, src, n);
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stand-in HIP error"; }
}

namespace mxattn {
static unsigned char g_scratch[64];
hipError_t launch_quant_qk(const QuantArgs&, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t launch_quant_v(const QuantArgs&, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t launch_quant_vkey(const QuantArgs&, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t launch_copy_bf16(const void*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, void*, hipStream_t) {
  return g_launches++, hipSuccess;
}
hipError_t launch_channel_mean(const QuantArgs&, float*, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t launch_quant_qk_pre(const QuantArgs&, const float*, int, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t launch_center_comp(const CompArgs&, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t launch_decode(int, const DecArgs&, hipStream_t) { return g_launches++, hipSuccess; }
hipError_t decode_scratch(void** ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}
hipError_t launch_fwd(int, int, int, int, int, const FwdArgs& a, hipStream_t) {
  // the plan a document forward would read: its header must be the one built for it
  if (a.plan != nullptr && (a.plan->magic != PLAN_MAGIC || a.plan->ndocs != a.ndocs || a.plan->n_tokens != a.N))
    return hipErrorInvalidValue;
  return g_launches++, hipSuccess;
}
}  // namespace mxattn
