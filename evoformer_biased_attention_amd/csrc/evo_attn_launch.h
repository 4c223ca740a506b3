// Internal launcher interface between the C ABI (evo_attn_api.cpp) and the
// kernels.  Not installed; callers use include/evo_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evo {

// Element strides of the attention tensors.  q, k, v, out: the b, n, l (row)
// and h axes; the d axis is contiguous.  Biases: keys contiguous.  The C ABI
// checks that the q, k, v and out strides are multiples of 16 bytes.  In the
// backward pass each gradient shares the strides of the tensor it belongs to
// (dout those of out, dq of q, dk of k, dv of v, dmask of the mask, dpair of
// the pair bias, delta the lse rows).
struct Strides {
    int64_t q[4], k[4], v[4], o[4];  // b, n, l, h
    int64_t mb, mn;                  // mask row of (b, n)
    int64_t pb, ph, pi;              // pair matrix of (b, h), its query rows
    int64_t lrow;                    // lse: elements between consecutive (b, n, h) rows, >= L
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* mask;  // [B,N,1,1,L] or nullptr
    const void* pair;  // [B,1,H,L,L] or nullptr
    void* out;
    float* lse;        // [B,N,H,L] (rows lrow apart) or nullptr
    int64_t B, N, L, H, D;
    Strides st;
};

// bf16 inputs, D in {8, 16, 32, 64}: MFMA kernel.  Returns the hipError_t of the launch.
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);

// f16 inputs, D in {8, 16, 32, 64}: the same MFMA kernel on binary16 operands.
hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t stream);

// f32 inputs, D in {8, 16, 32, 64}: the fp32 matrix-core kernel, or the
// vector-ALU one for layouts past its 32-bit offsets.
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* mask;   // [B,N,1,1,L] or nullptr
    const void* pair;   // [B,1,H,L,L] or nullptr
    const void* out;    // forward output [B,N,L,H,D]
    const float* lse;   // forward log-sum-exp [B,N,H,L] (rows lrow apart)
    const void* dout;   // incoming gradient [B,N,L,H,D]
    void* dq;
    void* dk;
    void* dv;
    void* dmask;        // [B,N,1,1,L] or nullptr (only with mask)
    void* dpair;        // [B,1,H,L,L] or nullptr (only with pair)
    float* delta;       // [B,N,H,L] (rows lrow apart), written
    float* ws;          // workspace for the pair gradient's partial sums, or nullptr
    int64_t ws_chunks;  // N-chunks the workspace holds ([ws_chunks][B][H][L][L] fp32)
    int64_t B, N, L, H, D;
    Strides st;         // element strides of every tensor and of its gradient
};

// Backward pass, dtype 0 = f32, 1 = bf16, 2 = f16, D in {8, 16, 32, 64}.
// Returns the hipError_t of the first failing launch.
hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t stream);

// The backward's three stages (each a kernel that owns its outputs).
constexpr unsigned kStageDq = 1;     // dq, and delta (read by the other two)
constexpr unsigned kStageDkDv = 2;   // dk, dv, dmask
constexpr unsigned kStageDpair = 4;  // dpair

// Matrix-core backward: the stages it implements, whether it accepts the
// arguments, and a launch of some of those stages in stage order.
extern const unsigned kBwdMfmaStages;
bool bwd_mfma_eligible(const BwdArgs& a, int dtype);
// The number of N-chunks whose pair-gradient partial sums the matrix-core
// path would like in its workspace (0: no workspace wanted).
int64_t bwd_dpair_chunks(int64_t B, int64_t N, int64_t L, int64_t H);
// Row length (fp32 elements) of those partial sums: L rounded up to a
// multiple of 4, so that every 4-key group of a row is one aligned 16-byte
// piece of its own row.  One chunk holds B * H * L rows.
__host__ __device__ inline int64_t bwd_ws_row(int64_t L) { return (L + 3) / 4 * 4; }
hipError_t launch_bwd_mfma(const BwdArgs& a, int dtype, unsigned stages, hipStream_t stream);

// Matrix-core backward for fp32 inputs (evo_attn_bwd_f32.hip): the stages it
// implements (dq + delta, dk/dv/dmask, dpair), whether it accepts the
// arguments, and a launch of some of those stages in stage order.  Its pair
// gradient uses the workspace as the 16-bit kernels do (ws_chunks ranges).
extern const unsigned kBwdF32MfmaStages;
bool bwd_f32_mfma_eligible(const BwdArgs& a);
hipError_t launch_bwd_f32_mfma(const BwdArgs& a, unsigned stages, hipStream_t stream);

// Triangle multiplication, 16-bit formats, [planes][L][L] operands.
hipError_t launch_trimul(const void* a, const void* w, void* x, int64_t planes, int64_t L, int incoming, int f16,
                         hipStream_t stream);

}  // namespace evo
