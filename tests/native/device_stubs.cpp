// Host-only stand-ins for the library's device-side functions (kernel
// launchers, device queries), so that the C-ABI layer and the host
// preparation code can be built and run under the address and
// undefined-behaviour sanitizers without a GPU.  Every launcher reports a
// failure: the sanitizer driver only reaches them through paths it expects to
// fail, and a call it did not expect shows up as a failed check.
#include "internal.h"

namespace svdq {

namespace {
constexpr int kNoDevice = 100;  // hipErrorNoDevice
}

const char* hip_error_name(int) { return "no device (host-only build)"; }
int device_cus() { return kMaxCUs; }
int scratch_buffer(void**) { return kNoDevice; }
int launch_calibrate(const uint16_t*, int, int, float*, int, void*) { return kNoDevice; }
int launch_act_quant_down(const uint16_t*, int, int, int, const float*, const uint16_t*, uint8_t*, uint16_t*, float*,
                          const ActPlan&, int, float, void*) {
  return kNoDevice;
}
int launch_z_reduce(const float*, int, int, int, float*, void*) { return kNoDevice; }
int launch_act8_quant(const uint16_t*, int, int, const float*, int8_t*, uint16_t*, void*) { return kNoDevice; }
int launch_add(void*, const void*, size_t, int, void*) { return kNoDevice; }
int launch_lowrank_up(const float*, const svdq_layer&, int, void*, int, void*) { return kNoDevice; }
int launch_gemm_up(const uint8_t*, const uint16_t*, const float*, const svdq_layer&, int, void*, int, void*, void*) {
  return kNoDevice;
}
int launch_gemm8_up(const int8_t*, const uint16_t*, const float*, const svdq_w8a8_layer&, int, void*, int, void*,
                    void*) {
  return kNoDevice;
}
int launch_gemm_fp4_up(const uint8_t*, const uint8_t*, const float*, const svdq_fp4_layer&, int, void*, int, void*,
                       void*) {
  return kNoDevice;
}

}  // namespace svdq
