// Internal launcher interface between the C ABI (evo_attn_api.cpp) and the
// kernels.  Not installed; callers use include/evo_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evo {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* mask;  // [B,N,1,1,L] or nullptr
    const void* pair;  // [B,1,H,L,L] or nullptr
    void* out;
    float* lse;        // [B,N,H,L] or nullptr
    int64_t B, N, L, H, D;
};

// bf16 inputs, D in {8, 16, 32}: MFMA kernel.  Returns the hipError_t of the launch.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);

// f16 inputs, D in {8, 16, 32}: the same MFMA kernel on binary16 operands.
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t stream);

// f32 inputs, D in {8, 16, 32, 64}: vector-ALU kernel.
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

}  // namespace evo
