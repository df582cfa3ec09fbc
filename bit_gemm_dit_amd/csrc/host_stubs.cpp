// Host-only stand-ins of the kernel launchers, linked only into the sanitizer build
// of the ABI layer (`python bit_gemm_dit_amd/build.py --sanitize`).
//
// That build instruments abi.cpp with AddressSanitizer and UndefinedBehaviorSanitizer
// on the CPU and runs the ABI's CPU tests against it: argument validation, pointer
// overlap arithmetic, size queries and status strings.  No kernel is compiled into
// it; every launcher here reports hipErrorNoDevice, which the ABI turns into
// DIT_EDEVICE like any launch failure.
#include "common.hpp"

namespace ditq {

hipError_t launch_quant_fp4(const uint16_t*, int, int, int, uint8_t*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_fp8(const uint16_t*, int, int, int, uint8_t*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_mx8(const uint16_t*, int, int, int, uint8_t*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_nv4(const uint16_t*, int, int, int, uint8_t*, uint8_t*, uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_nv4_static(const uint16_t*, int, int, int, uint8_t*, uint8_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_amax_bf16(const uint16_t*, int, int, int, uint32_t*, uint32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_pack(int, int, const uint16_t*, int, int, int, uint8_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gemm(int, const uint8_t*, const void*, const uint8_t*, int, int, int, int, const RmsArgs*,
                       const ResidualArgs*, uint16_t*, int, uint8_t*, uint8_t*, float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gated_silu(const uint16_t*, int, int, int, uint16_t*, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_mfma_probe(int, int, unsigned long long*, hipStream_t) { return hipErrorNoDevice; }

}  // namespace ditq
