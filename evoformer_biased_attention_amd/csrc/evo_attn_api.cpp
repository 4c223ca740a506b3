// C ABI of libevoattn.so: argument validation and kernel selection.
//
// The checks carry over the input contract of the DS4Sci_EvoformerAttention
// Python front end described on the page "DeepSpeed DS4Sci_EvoformerAttention
// 内核实战指南" (hmyw.cn): fp16/bf16 inputs on the accelerator (section 5.1),
// at most two biases whose shapes are derived from Q's and checked strictly,
// a missing bias taking the same path as an all-zero one (sections 5.2 and
// 5.4).  Here the shapes are passed explicitly, so "strict shape checks"
// become size and overflow checks on evo_shape_t; the guide's L > 16 limit is
// not kept (any L >= 1 works).
#include "../../include/evo_attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "evo_attn_launch.h"

namespace {

constexpr int64_t kMaxBytes = int64_t(1) << 62;

// a * b without overflow past kMaxBytes; returns -1 on overflow.
int64_t mul_checked(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a != 0 && b > kMaxBytes / a) return -1;
    return a * b;
}

int64_t elem_size(evo_dtype_t dt) { return dt == EVO_DTYPE_F32 ? 4 : 2; }

struct Extent {
    uintptr_t lo = 0, hi = 0;  // [lo, hi), empty when lo == hi
    bool overlaps(const Extent& o) const { return lo < o.hi && o.lo < hi; }
};

Extent extent(const void* p, int64_t bytes) {
    Extent e;
    if (p) {
        e.lo = reinterpret_cast<uintptr_t>(p);
        e.hi = e.lo + static_cast<uintptr_t>(bytes);
    }
    return e;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

thread_local int g_last_hip_error = 0;

// The 16-bit (bf16, f16) kernel addresses one (b, n, h) slice and one pair
// matrix with 32-bit byte offsets.
constexpr int64_t kMaxOffset = int64_t(1) << 31;

bool supported(evo_dtype_t dt, int64_t L, int64_t H, int64_t D) {
    if (dt == EVO_DTYPE_BF16 || dt == EVO_DTYPE_F16)
        return (D == 8 || D == 16 || D == 32) && L * H * D * 2 < kMaxOffset && L * L * 2 < kMaxOffset;
    if (dt == EVO_DTYPE_F32) return D == 8 || D == 16 || D == 32 || D == 64;
    return false;
}

}  // namespace

extern "C" evo_status_t evo_attn_check(const void* q, const void* k, const void* v, const void* mask_bias,
                                       const void* pair_bias, const void* out, const float* lse,
                                       const evo_shape_t* shape, evo_dtype_t dtype) {
    if (!shape || !q || !k || !v || !out) return EVO_ERR_NULL_POINTER;
    const int64_t B = shape->B, N = shape->N, L = shape->L, H = shape->H, D = shape->D;
    if (B < 1 || N < 1 || L < 1 || H < 1 || D < 1) return EVO_ERR_BAD_SHAPE;
    if (dtype != EVO_DTYPE_F32 && dtype != EVO_DTYPE_BF16 && dtype != EVO_DTYPE_F16) return EVO_ERR_BAD_DTYPE;
    const int64_t es = elem_size(dtype);

    // Byte sizes of every tensor, each bounded by 2^62.
    int64_t qkv = es;
    for (int64_t s : {B, N, L, H, D}) qkv = mul_checked(qkv, s);
    int64_t msk = es;
    for (int64_t s : {B, N, L}) msk = mul_checked(msk, s);
    int64_t par = es;
    for (int64_t s : {B, H, L, L}) par = mul_checked(par, s);
    int64_t lsb = 4;
    for (int64_t s : {B, N, H, L}) lsb = mul_checked(lsb, s);
    if (qkv < 0 || msk < 0 || par < 0 || lsb < 0) return EVO_ERR_BAD_SHAPE;

    for (const void* p : {q, k, v, mask_bias, pair_bias, out, static_cast<const void*>(lse)})
        if (p && !aligned16(p)) return EVO_ERR_MISALIGNED;

    const Extent eo = extent(out, qkv), el = extent(lse, lsb);
    for (const Extent& in : {extent(q, qkv), extent(k, qkv), extent(v, qkv), extent(mask_bias, msk),
                             extent(pair_bias, par)})
        if (eo.overlaps(in) || el.overlaps(in)) return EVO_ERR_ALIASING;
    if (eo.overlaps(el)) return EVO_ERR_ALIASING;

    if (!supported(dtype, L, H, D)) return EVO_ERR_UNSUPPORTED;
    return EVO_OK;
}

extern "C" evo_status_t evo_attn_fwd(const void* q, const void* k, const void* v, const void* mask_bias,
                                     const void* pair_bias, void* out, float* lse, const evo_shape_t* shape,
                                     evo_dtype_t dtype, void* stream) {
    const evo_status_t st = evo_attn_check(q, k, v, mask_bias, pair_bias, out, lse, shape, dtype);
    if (st != EVO_OK) return st;
    evo::FwdArgs a{q, k, v, mask_bias, pair_bias, out, lse, shape->B, shape->N, shape->L, shape->H, shape->D};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = dtype == EVO_DTYPE_BF16  ? evo::launch_fwd_bf16(a, s)
                     : dtype == EVO_DTYPE_F16 ? evo::launch_fwd_f16(a, s)
                                              : evo::launch_fwd_f32(a, s);
    if (err == hipSuccess) return EVO_OK;
    g_last_hip_error = static_cast<int>(err);
    return EVO_ERR_HIP;
}

namespace {

// Gradient support: every dtype with D in {8, 16, 32, 64} (section 5.4 of the
// guide gives D <= 64 as the backward pass's limit).
bool bwd_supported(evo_dtype_t dt, int64_t D) {
    return (dt == EVO_DTYPE_F32 || dt == EVO_DTYPE_BF16 || dt == EVO_DTYPE_F16) &&
           (D == 8 || D == 16 || D == 32 || D == 64);
}

}  // namespace

extern "C" evo_status_t evo_attn_bwd_check(const void* q, const void* k, const void* v, const void* mask_bias,
                                           const void* pair_bias, const void* out, const float* lse,
                                           const void* dout, const void* dq, const void* dk, const void* dv,
                                           const void* dmask_bias, const void* dpair_bias, const float* delta,
                                           const void* workspace, size_t workspace_bytes, const evo_shape_t* shape,
                                           evo_dtype_t dtype) {
    if (!shape || !q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !delta)
        return EVO_ERR_NULL_POINTER;
    const int64_t B = shape->B, N = shape->N, L = shape->L, H = shape->H, D = shape->D;
    if (B < 1 || N < 1 || L < 1 || H < 1 || D < 1) return EVO_ERR_BAD_SHAPE;
    if (dtype != EVO_DTYPE_F32 && dtype != EVO_DTYPE_BF16 && dtype != EVO_DTYPE_F16) return EVO_ERR_BAD_DTYPE;
    if ((dmask_bias && !mask_bias) || (dpair_bias && !pair_bias)) return EVO_ERR_NO_BIAS;
    const int64_t es = elem_size(dtype);

    int64_t qkv = es;
    for (int64_t s : {B, N, L, H, D}) qkv = mul_checked(qkv, s);
    int64_t msk = es;
    for (int64_t s : {B, N, L}) msk = mul_checked(msk, s);
    int64_t par = es;
    for (int64_t s : {B, H, L, L}) par = mul_checked(par, s);
    int64_t row = 4;
    for (int64_t s : {B, N, H, L}) row = mul_checked(row, s);
    if (qkv < 0 || msk < 0 || par < 0 || row < 0) return EVO_ERR_BAD_SHAPE;

    if (workspace && workspace_bytes > static_cast<size_t>(kMaxBytes)) return EVO_ERR_BAD_SHAPE;
    for (const void* p : {q, k, v, mask_bias, pair_bias, out, static_cast<const void*>(lse), dout, dq, dk, dv,
                          dmask_bias, dpair_bias, static_cast<const void*>(delta), workspace})
        if (p && !aligned16(p)) return EVO_ERR_MISALIGNED;

    const Extent outs[] = {extent(dq, qkv),        extent(dk, qkv),   extent(dv, qkv),
                           extent(dmask_bias, msk), extent(dpair_bias, par), extent(delta, row),
                           extent(workspace, workspace ? static_cast<int64_t>(workspace_bytes) : 0)};
    const Extent ins[] = {extent(q, qkv),         extent(k, qkv),   extent(v, qkv), extent(mask_bias, msk),
                          extent(pair_bias, par), extent(out, qkv), extent(lse, row), extent(dout, qkv)};
    for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a) {
        for (const Extent& in : ins)
            if (outs[a].overlaps(in)) return EVO_ERR_ALIASING;
        for (size_t c = a + 1; c < sizeof(outs) / sizeof(outs[0]); ++c)
            if (outs[a].overlaps(outs[c])) return EVO_ERR_ALIASING;
    }
    if (!bwd_supported(dtype, D)) return EVO_ERR_UNSUPPORTED;
    return EVO_OK;
}

namespace {

// Workspace chunks the call can use: what the matrix-core path wants, capped
// by what the given workspace holds (0: none).
int64_t usable_chunks(const evo_shape_t* s, evo_dtype_t dtype, size_t workspace_bytes) {
    evo::BwdArgs probe{};
    probe.B = s->B, probe.N = s->N, probe.L = s->L, probe.H = s->H, probe.D = s->D;
    if (!evo::bwd_mfma_eligible(probe, static_cast<int>(dtype))) return 0;
    const int64_t want = evo::bwd_dpair_chunks(s->B, s->N, s->L, s->H);
    const int64_t per = s->B * s->H * s->L * s->L * 4;  // bytes of one chunk's partial sums
    const int64_t fit = static_cast<int64_t>(workspace_bytes / static_cast<size_t>(per));
    const int64_t c = want < fit ? want : fit;
    return c >= 2 ? c : 0;
}

}  // namespace

extern "C" size_t evo_attn_bwd_workspace_size(const evo_shape_t* shape, evo_dtype_t dtype) {
    if (!shape || shape->B < 1 || shape->N < 1 || shape->L < 1 || shape->H < 1 || shape->D < 1) return 0;
    int64_t par = 4;
    for (int64_t s : {shape->B, shape->H, shape->L, shape->L}) par = mul_checked(par, s);
    if (par < 0) return 0;
    const int64_t c = usable_chunks(shape, dtype, ~static_cast<size_t>(0) >> 2);
    const int64_t bytes = mul_checked(par, c);
    return bytes < 0 ? 0 : static_cast<size_t>(bytes);
}

extern "C" evo_status_t evo_attn_bwd(const void* q, const void* k, const void* v, const void* mask_bias,
                                     const void* pair_bias, const void* out, const float* lse, const void* dout,
                                     void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias,
                                     float* delta, void* workspace, size_t workspace_bytes, const evo_shape_t* shape,
                                     evo_dtype_t dtype, void* stream) {
    const evo_status_t st = evo_attn_bwd_check(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                               dmask_bias, dpair_bias, delta, workspace, workspace_bytes, shape,
                                               dtype);
    if (st != EVO_OK) return st;
    evo::BwdArgs a{q,  k,  v,  mask_bias,  pair_bias,  out,   lse,     dout,    dq,      dk,      dv,
                   dmask_bias, dpair_bias, delta, nullptr, 0, shape->B, shape->N, shape->L, shape->H, shape->D};
    if (workspace && dpair_bias) {
        a.ws_chunks = usable_chunks(shape, dtype, workspace_bytes);
        if (a.ws_chunks) a.ws = static_cast<float*>(workspace);
    }
    const hipError_t err = evo::launch_bwd(a, static_cast<int>(dtype), static_cast<hipStream_t>(stream));
    if (err == hipSuccess) return EVO_OK;
    g_last_hip_error = static_cast<int>(err);
    return EVO_ERR_HIP;
}

extern "C" int evo_attn_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char* evo_status_string(evo_status_t status) {
    switch (status) {
    case EVO_OK: return "ok";
    case EVO_ERR_NULL_POINTER: return "a required pointer (q, k, v, out or shape) is NULL";
    case EVO_ERR_BAD_SHAPE: return "a size is below 1 or a tensor exceeds 2^62 bytes";
    case EVO_ERR_BAD_DTYPE: return "dtype is not an evo_dtype_t value";
    case EVO_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
    case EVO_ERR_ALIASING: return "an output overlaps an input or another output";
    case EVO_ERR_UNSUPPORTED: return "dtype / head dimension combination not implemented";
    case EVO_ERR_HIP: return "the HIP runtime reported an error at launch";
    case EVO_ERR_NO_BIAS: return "a bias gradient was requested for a bias that was not given";
    }
    return "unknown status";
}
