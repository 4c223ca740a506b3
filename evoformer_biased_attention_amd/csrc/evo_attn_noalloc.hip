// evo_attn_bwd_noalloc: the backward pass with its pair-gradient workspace in
// a library-owned static device array instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array `scratch` lives in this file's code object: every GPU the library
// runs on holds its own copy of kScratchBytes until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is taken once per device with hipGetSymbolAddress (with that device
// current, on the entry point's first call there) and only that address is
// handed to the kernels.  Calls on one GPU share its array: calls that overlap
// in time on one GPU (two streams, two threads) race on it.  The pair
// gradient's partial sums are written in full before they are read, so the
// array needs no clearing between calls.  A shape whose recommended workspace
// is larger than the array gets as many whole chunks of partial sums as fit
// (the pass then splits N that many ways).
#include "../../include/evo_attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(40) << 20;  // 40 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, taken on first use; nullptr on a
// HIP error (its code kept for evo_attn_last_hip_error by the caller).
void* scratch_on(int dev, hipError_t* err) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_ptr[dev] = p;
    }
    *err = hipSuccess;
    return g_ptr[dev];
}

thread_local int g_noalloc_hip_error = 0;

}  // namespace

extern "C" size_t evo_attn_bwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int evo_attn_bwd_noalloc_last_hip_error(void) { return g_noalloc_hip_error; }

extern "C" evo_status_t evo_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* mask_bias,
                                             const void* pair_bias, const void* out, const float* lse,
                                             const void* dout, void* dq, void* dk, void* dv, void* dmask_bias,
                                             void* dpair_bias, float* delta, const evo_shape_t* shape,
                                             evo_dtype_t dtype, void* stream) {
    // host-only checks first: no HIP call before the arguments are accepted
    const evo_status_t st = evo_attn_bwd_check(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                               dmask_bias, dpair_bias, delta, nullptr, 0, shape, dtype);
    if (st != EVO_OK) return st;
    // as many of the recommended N-chunks as fit: a chunk is one fp32
    // [B,H,L,ceil4(L)] plane (it is at most `want`, which fits in size_t)
    const size_t want = dpair_bias ? evo_attn_bwd_workspace_size(shape, dtype) : 0;
    size_t need = want;
    if (want > kScratchBytes) {
        const size_t plane = static_cast<size_t>(shape->B) * static_cast<size_t>(shape->H) *
                             static_cast<size_t>(shape->L) * static_cast<size_t>((shape->L + 3) / 4 * 4) * 4u;
        if (plane > kScratchBytes / 2) return EVO_ERR_SCRATCH;
        need = kScratchBytes - kScratchBytes % plane;
    }
    void* ws = nullptr;
    if (need) {
        int dev = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess && (dev < 0 || dev >= kMaxDevices)) err = hipErrorInvalidDevice;
        if (err == hipSuccess) ws = scratch_on(dev, &err);
        if (err != hipSuccess) {
            g_noalloc_hip_error = static_cast<int>(err);
            return EVO_ERR_HIP;
        }
    }
    return evo_attn_bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, delta,
                        ws, need, shape, dtype, stream);
}
