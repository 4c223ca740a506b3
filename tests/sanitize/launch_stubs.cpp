// Host-only stand-ins for the kernel launchers of libevoattn, so that the C
// ABI's argument checks (evo_attn_api.cpp) can be built and exercised on a
// machine without a GPU, under AddressSanitizer and UndefinedBehaviorSanitizer.
// Each launcher records that it was reached and returns success; none touches
// the pointers it is given.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include "evo_attn_launch.h"

namespace evo_stub {
long launches = 0;
}

namespace evo {

hipError_t launch_fwd_bf16(const FwdArgs&, hipStream_t) { return ++evo_stub::launches, hipSuccess; }
hipError_t launch_fwd_f16(const FwdArgs&, hipStream_t) { return ++evo_stub::launches, hipSuccess; }
hipError_t launch_fwd_f32(const FwdArgs&, hipStream_t) { return ++evo_stub::launches, hipSuccess; }
hipError_t launch_bwd(const BwdArgs&, int, hipStream_t) { return ++evo_stub::launches, hipSuccess; }
hipError_t launch_trimul(const void*, const void*, void*, int64_t, int64_t, int, int, hipStream_t) {
    return ++evo_stub::launches, hipSuccess;
}
// the matrix-core backward kernels take every call here (16-bit and fp32),
// so that the workspace arithmetic runs for all of them
bool bwd_mfma_eligible(const BwdArgs&, int dtype) { return dtype != 0; }
bool bwd_f32_mfma_eligible(const BwdArgs&) { return true; }
int64_t bwd_dpair_chunks(int64_t, int64_t N, int64_t, int64_t) { return N < 8 ? N : 8; }

}  // namespace evo
