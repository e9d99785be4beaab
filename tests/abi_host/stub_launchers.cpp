// Stand-ins for the kernel launchers, linked into a host-only build of the C
// ABI (fa_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.  The
// argument-validation tests pass only arguments that must be rejected before
// anything is launched, so reaching a launcher is itself a failure: each one
// reports which and aborts.
#include <cstdio>
#include <cstdlib>

#include "fa_kernels.h"

namespace fa {
namespace {
[[noreturn]] void reached(const char* what) {
  std::fprintf(stderr, "kernel launcher reached in a validation test: %s\n", what);
  std::abort();
}
}  // namespace

template <typename T>
hipError_t launch_fwd(const FwdArgs<T>&, int, bool, bool, hipStream_t) { reached("forward"); }
template <typename T>
hipError_t launch_bwd_stage(const BwdArgs<T>&, int, bool, BwdStage, hipStream_t) {
  reached("backward stage");
}
template <typename T>
hipError_t launch_bwd(const BwdArgs<T>&, int, bool, hipStream_t) { reached("backward"); }
template <typename T>
hipError_t launch_decode(const DecArgs<T>&, int, bool, int, hipStream_t) { reached("decode"); }
template <typename T>
hipError_t launch_fp8_quantize(const Fp8QuantArgs<T>&, int, hipStream_t) { reached("fp8"); }

hipError_t noalloc_scratch(hipStream_t, void**) { reached("scratch lookup"); }
template <typename T>
hipError_t launch_fwd_fp8(const Fp8FwdArgs<T>&, int, bool, hipStream_t) { reached("fp8 forward"); }
template hipError_t launch_fwd_fp8<bf16_t>(const Fp8FwdArgs<bf16_t>&, int, bool, hipStream_t);
template hipError_t launch_fwd_fp8<f16_t>(const Fp8FwdArgs<f16_t>&, int, bool, hipStream_t);

template hipError_t launch_fwd<bf16_t>(const FwdArgs<bf16_t>&, int, bool, bool, hipStream_t);
template hipError_t launch_fwd<f16_t>(const FwdArgs<f16_t>&, int, bool, bool, hipStream_t);
template hipError_t launch_fwd<float>(const FwdArgs<float>&, int, bool, bool, hipStream_t);
template hipError_t launch_bwd_stage<bf16_t>(const BwdArgs<bf16_t>&, int, bool, BwdStage,
                                             hipStream_t);
template hipError_t launch_bwd_stage<f16_t>(const BwdArgs<f16_t>&, int, bool, BwdStage,
                                            hipStream_t);
template hipError_t launch_bwd<bf16_t>(const BwdArgs<bf16_t>&, int, bool, hipStream_t);
template hipError_t launch_bwd<f16_t>(const BwdArgs<f16_t>&, int, bool, hipStream_t);
template hipError_t launch_decode<bf16_t>(const DecArgs<bf16_t>&, int, bool, int, hipStream_t);
template hipError_t launch_decode<f16_t>(const DecArgs<f16_t>&, int, bool, int, hipStream_t);
template hipError_t launch_fp8_quantize<bf16_t>(const Fp8QuantArgs<bf16_t>&, int, hipStream_t);
template hipError_t launch_fp8_quantize<f16_t>(const Fp8QuantArgs<f16_t>&, int, hipStream_t);

}  // namespace fa
