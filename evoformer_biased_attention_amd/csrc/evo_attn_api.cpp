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

#include <algorithm>
#include <cstdint>
#include <initializer_list>
#include <utility>

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

// The 16-bit (bf16, f16) kernel addresses the rows of one (b, n, h) slice
// and of one pair matrix with 32-bit byte offsets, including rows up to 128
// past L (which must land beyond the range, not wrap).
constexpr int64_t kMaxOffset = int64_t(1) << 31;
constexpr int64_t kMaxOffset32 = int64_t(1) << 32;

// Whether rows of `row_elems` elements, es bytes each, keep every offset of
// the 16-bit kernel in 32 bits: the last row's end below 2^31 (the buffer
// range) and row L + 128 below 2^32.
bool rows_fit(int64_t L, int64_t row_elems, int64_t last_row_bytes) {
    const int64_t row = mul_checked(row_elems, 2);
    const int64_t lo = mul_checked(L - 1, row), hi = mul_checked(L + 128, row);
    return row >= 0 && lo >= 0 && lo + last_row_bytes < kMaxOffset && hi >= 0 && hi < kMaxOffset32;
}

bool dim_supported(evo_dtype_t dt, int64_t D) {
    if (dt == EVO_DTYPE_BF16 || dt == EVO_DTYPE_F16) return D == 8 || D == 16 || D == 32 || D == 64;
    return dt == EVO_DTYPE_F32 && (D == 8 || D == 16 || D == 32 || D == 64);
}

// The pair rows count only when a pair bias is given: without one the kernel
// forms no pair offset.
bool offsets_fit(evo_dtype_t dt, const evo_shape_t& s, const evo_layout_t& lay, bool pair) {
    if (dt == EVO_DTYPE_F32) return true;
    const int64_t L = s.L, D = s.D;
    return rows_fit(L, lay.q[2], D * 2) && rows_fit(L, lay.k[2], D * 2) && rows_fit(L, lay.v[2], D * 2) &&
           (!pair || rows_fit(L, lay.pair_i, L * 2));
}

// Largest element offset + 1 over axes {(size, stride)}, or -1 past 2^62.
int64_t span_elems(std::initializer_list<std::pair<int64_t, int64_t>> axes) {
    int64_t e = 1;
    for (const auto& a : axes) {
        const int64_t t = mul_checked(a.first - 1, a.second);
        if (t < 0 || e > kMaxBytes - t) return -1;
        e += t;
    }
    return e;
}

// Whether distinct indices of a tensor with axes {(stride, size)} and a
// contiguous innermost run of `inner` elements have distinct offsets: taken in
// increasing stride order, each axis of size > 1 must step past everything the
// faster axes cover.
bool disjoint_axes(std::pair<int64_t, int64_t>* ax, int count, int64_t inner) {
    std::sort(ax, ax + count);
    int64_t e = inner;
    for (int i = 0; i < count; ++i) {
        const auto& a = ax[i];
        if (a.second <= 1) continue;
        if (a.first < e) return false;
        const int64_t t = mul_checked(a.second - 1, a.first);
        if (t < 0 || e > kMaxBytes - t) return false;
        e += t;
    }
    return true;
}

// The same for a [B,N,L,H,D] tensor with strides st (b, n, l, h; d contiguous).
bool no_self_overlap(const int64_t* st, const evo_shape_t& s) {
    std::pair<int64_t, int64_t> ax[4] = {{st[0], s.B}, {st[1], s.N}, {st[2], s.L}, {st[3], s.H}};
    return disjoint_axes(ax, 4, s.D);
}

// evo_layout_t -> the kernels' stride set
evo::Strides strides_of(const evo_layout_t& lay) {
    evo::Strides st{};
    for (int i = 0; i < 4; ++i) {
        st.q[i] = lay.q[i];
        st.k[i] = lay.k[i];
        st.v[i] = lay.v[i];
        st.o[i] = lay.out[i];
    }
    st.mb = lay.mask_b, st.mn = lay.mask_n;
    st.pb = lay.pair_b, st.ph = lay.pair_h, st.pi = lay.pair_i;
    st.lrow = lay.lse_row;
    return st;
}

}  // namespace

extern "C" void evo_attn_dense_layout(const evo_shape_t* shape, evo_layout_t* layout) {
    if (!shape || !layout) return;
    // a stride that overflows becomes -1, which the checks reject
    const int64_t N = shape->N, L = shape->L, H = shape->H, D = shape->D;
    const int64_t hd = mul_checked(H, D), lhd = mul_checked(L, hd), ll = mul_checked(L, L);
    const int64_t dense[4] = {mul_checked(N, lhd), lhd, hd, D};
    for (int a = 0; a < 4; ++a) layout->q[a] = layout->k[a] = layout->v[a] = layout->out[a] = dense[a];
    layout->mask_b = mul_checked(N, L);
    layout->mask_n = L;
    layout->pair_b = mul_checked(H, ll);
    layout->pair_h = ll;
    layout->pair_i = L;
    layout->lse_row = L;
}

extern "C" evo_status_t evo_attn_check_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                               const void* pair_bias, const void* out, const float* lse,
                                               const evo_layout_t* layout, const evo_shape_t* shape,
                                               evo_dtype_t dtype) {
    if (!shape || !layout || !q || !k || !v || !out) return EVO_ERR_NULL_POINTER;
    const evo_shape_t& s = *shape;
    const evo_layout_t& lay = *layout;
    const int64_t B = s.B, N = s.N, L = s.L, H = s.H, D = s.D;
    if (B < 1 || N < 1 || L < 1 || H < 1 || D < 1) return EVO_ERR_BAD_SHAPE;
    if (dtype != EVO_DTYPE_F32 && dtype != EVO_DTYPE_BF16 && dtype != EVO_DTYPE_F16) return EVO_ERR_BAD_DTYPE;
    const int64_t es = elem_size(dtype);

    // strides: non-negative; pair rows and lse rows at least L apart
    const int64_t* qkvo[4] = {lay.q, lay.k, lay.v, lay.out};
    for (const int64_t* t : qkvo)
        for (int a = 0; a < 4; ++a)
            if (t[a] < 0) return EVO_ERR_BAD_SHAPE;
    if (lay.mask_b < 0 || lay.mask_n < 0 || lay.pair_b < 0 || lay.pair_h < 0) return EVO_ERR_BAD_SHAPE;
    if (pair_bias && lay.pair_i < L) return EVO_ERR_BAD_SHAPE;
    if (lse && lay.lse_row < L) return EVO_ERR_BAD_SHAPE;

    // byte extents, each below 2^62
    int64_t ext[4];
    for (int t = 0; t < 4; ++t) {
        const int64_t e = span_elems({{B, qkvo[t][0]}, {N, qkvo[t][1]}, {L, qkvo[t][2]}, {H, qkvo[t][3]}, {D, 1}});
        ext[t] = e < 0 ? -1 : mul_checked(e, es);
    }
    const int64_t me = span_elems({{B, lay.mask_b}, {N, lay.mask_n}, {L, 1}});
    const int64_t pe = span_elems({{B, lay.pair_b}, {H, lay.pair_h}, {L, lay.pair_i}, {L, 1}});
    const int64_t bnh = mul_checked(mul_checked(B, N), H);
    const int64_t le = bnh < 0 ? -1 : span_elems({{bnh, lay.lse_row}, {L, 1}});
    const int64_t msk = me < 0 ? -1 : mul_checked(me, es), par = pe < 0 ? -1 : mul_checked(pe, es);
    const int64_t lsb = le < 0 ? -1 : mul_checked(le, 4);
    for (int64_t x : {ext[0], ext[1], ext[2], ext[3], msk, par, lsb})
        if (x < 0) return EVO_ERR_BAD_SHAPE;

    for (const void* p : {q, k, v, mask_bias, pair_bias, out, static_cast<const void*>(lse)})
        if (p && !aligned16(p)) return EVO_ERR_MISALIGNED;

    // outputs: out's strides must not map two elements to one address, and
    // out and lse may overlap neither an input nor each other
    if (!no_self_overlap(lay.out, s)) return EVO_ERR_ALIASING;
    const Extent eo = extent(out, ext[3]), el = extent(lse, lsb);
    for (const Extent& in : {extent(q, ext[0]), extent(k, ext[1]), extent(v, ext[2]), extent(mask_bias, msk),
                             extent(pair_bias, par)})
        if (eo.overlaps(in) || el.overlaps(in)) return EVO_ERR_ALIASING;
    if (eo.overlaps(el)) return EVO_ERR_ALIASING;

    if (!dim_supported(dtype, D)) return EVO_ERR_UNSUPPORTED;
    // rows of q, k, v and out start 16-byte aligned (the kernels move rows in
    // 16-byte pieces); bias strides need no alignment (unaligned ones take the
    // exact path)
    for (const int64_t* t : qkvo)
        for (int a = 0; a < 4; ++a)
            if ((t[a] % 16) * es % 16) return EVO_ERR_MISALIGNED;  // t[a] >= 0; no overflow for any stride
    if (!offsets_fit(dtype, s, lay, pair_bias != nullptr)) return EVO_ERR_UNSUPPORTED;
    return EVO_OK;
}

extern "C" evo_status_t evo_attn_check(const void* q, const void* k, const void* v, const void* mask_bias,
                                       const void* pair_bias, const void* out, const float* lse,
                                       const evo_shape_t* shape, evo_dtype_t dtype) {
    if (!shape) return EVO_ERR_NULL_POINTER;
    evo_layout_t lay;
    evo_attn_dense_layout(shape, &lay);
    return evo_attn_check_strided(q, k, v, mask_bias, pair_bias, out, lse, &lay, shape, dtype);
}

extern "C" evo_status_t evo_attn_fwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                             const void* pair_bias, void* out, float* lse, const evo_layout_t* layout,
                                             const evo_shape_t* shape, evo_dtype_t dtype, void* stream) {
    const evo_status_t st = evo_attn_check_strided(q, k, v, mask_bias, pair_bias, out, lse, layout, shape, dtype);
    if (st != EVO_OK) return st;
    const evo::FwdArgs a{q,        k,        v,        mask_bias, pair_bias,          out, lse,
                         shape->B, shape->N, shape->L, shape->H,  shape->D, strides_of(*layout)};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = dtype == EVO_DTYPE_BF16  ? evo::launch_fwd_bf16(a, s)
                           : dtype == EVO_DTYPE_F16 ? evo::launch_fwd_f16(a, s)
                                                    : evo::launch_fwd_f32(a, s);
    if (err == hipSuccess) return EVO_OK;
    g_last_hip_error = static_cast<int>(err);
    return EVO_ERR_HIP;
}

extern "C" evo_status_t evo_attn_fwd(const void* q, const void* k, const void* v, const void* mask_bias,
                                     const void* pair_bias, void* out, float* lse, const evo_shape_t* shape,
                                     evo_dtype_t dtype, void* stream) {
    const evo_status_t st = evo_attn_check(q, k, v, mask_bias, pair_bias, out, lse, shape, dtype);
    if (st != EVO_OK) return st;
    evo_layout_t lay;
    evo_attn_dense_layout(shape, &lay);
    return evo_attn_fwd_strided(q, k, v, mask_bias, pair_bias, out, lse, &lay, shape, dtype, stream);
}

namespace {

// Gradient support: every dtype with D in {8, 16, 32, 64} (section 5.4 of the
// guide gives D <= 64 as the backward pass's limit).
bool bwd_supported(evo_dtype_t dt, int64_t D) {
    return (dt == EVO_DTYPE_F32 || dt == EVO_DTYPE_BF16 || dt == EVO_DTYPE_F16) &&
           (D == 8 || D == 16 || D == 32 || D == 64);
}

}  // namespace

extern "C" evo_status_t evo_attn_bwd_check_strided(const void* q, const void* k, const void* v,
                                                   const void* mask_bias, const void* pair_bias, const void* out,
                                                   const float* lse, const void* dout, const void* dq, const void* dk,
                                                   const void* dv, const void* dmask_bias, const void* dpair_bias,
                                                   const float* delta, const void* workspace,
                                                   size_t workspace_bytes, const evo_layout_t* layout,
                                                   const evo_shape_t* shape, evo_dtype_t dtype) {
    if (!shape || !layout || !q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !delta)
        return EVO_ERR_NULL_POINTER;
    const evo_shape_t& s = *shape;
    const evo_layout_t& lay = *layout;
    const int64_t B = s.B, N = s.N, L = s.L, H = s.H, D = s.D;
    if (B < 1 || N < 1 || L < 1 || H < 1 || D < 1) return EVO_ERR_BAD_SHAPE;
    if (dtype != EVO_DTYPE_F32 && dtype != EVO_DTYPE_BF16 && dtype != EVO_DTYPE_F16) return EVO_ERR_BAD_DTYPE;
    if ((dmask_bias && !mask_bias) || (dpair_bias && !pair_bias)) return EVO_ERR_NO_BIAS;
    const int64_t es = elem_size(dtype);

    // strides: non-negative; pair rows and lse / delta rows at least L apart
    const int64_t* qkvo[4] = {lay.q, lay.k, lay.v, lay.out};
    for (const int64_t* t : qkvo)
        for (int a = 0; a < 4; ++a)
            if (t[a] < 0) return EVO_ERR_BAD_SHAPE;
    if (lay.mask_b < 0 || lay.mask_n < 0 || lay.pair_b < 0 || lay.pair_h < 0) return EVO_ERR_BAD_SHAPE;
    if (pair_bias && lay.pair_i < L) return EVO_ERR_BAD_SHAPE;
    if (lay.lse_row < L) return EVO_ERR_BAD_SHAPE;

    // byte extents, each below 2^62; a gradient spans what its tensor spans
    int64_t ext[4];
    for (int t = 0; t < 4; ++t) {
        const int64_t e = span_elems({{B, qkvo[t][0]}, {N, qkvo[t][1]}, {L, qkvo[t][2]}, {H, qkvo[t][3]}, {D, 1}});
        ext[t] = e < 0 ? -1 : mul_checked(e, es);
    }
    const int64_t me = span_elems({{B, lay.mask_b}, {N, lay.mask_n}, {L, 1}});
    const int64_t pe = span_elems({{B, lay.pair_b}, {H, lay.pair_h}, {L, lay.pair_i}, {L, 1}});
    const int64_t bnh = mul_checked(mul_checked(B, N), H);
    const int64_t le = bnh < 0 ? -1 : span_elems({{bnh, lay.lse_row}, {L, 1}});
    const int64_t msk = me < 0 ? -1 : mul_checked(me, es), par = pe < 0 ? -1 : mul_checked(pe, es);
    const int64_t row = le < 0 ? -1 : mul_checked(le, 4);
    for (int64_t x : {ext[0], ext[1], ext[2], ext[3], msk, par, row})
        if (x < 0) return EVO_ERR_BAD_SHAPE;

    if (workspace && workspace_bytes > static_cast<size_t>(kMaxBytes)) return EVO_ERR_BAD_SHAPE;
    for (const void* p : {q, k, v, mask_bias, pair_bias, out, static_cast<const void*>(lse), dout, dq, dk, dv,
                          dmask_bias, dpair_bias, static_cast<const void*>(delta), workspace})
        if (p && !aligned16(p)) return EVO_ERR_MISALIGNED;

    // outputs: no two elements of one gradient at one address, and no output
    // overlapping an input or another output
    if (!no_self_overlap(lay.q, s) || !no_self_overlap(lay.k, s) || !no_self_overlap(lay.v, s))
        return EVO_ERR_ALIASING;
    if (dmask_bias) {
        std::pair<int64_t, int64_t> ax[2] = {{lay.mask_b, B}, {lay.mask_n, N}};
        if (!disjoint_axes(ax, 2, L)) return EVO_ERR_ALIASING;
    }
    if (dpair_bias) {
        std::pair<int64_t, int64_t> ax[3] = {{lay.pair_b, B}, {lay.pair_h, H}, {lay.pair_i, L}};
        if (!disjoint_axes(ax, 3, L)) return EVO_ERR_ALIASING;
    }
    const Extent outs[] = {extent(dq, ext[0]),     extent(dk, ext[1]),          extent(dv, ext[2]),
                           extent(dmask_bias, msk), extent(dpair_bias, par),     extent(delta, row),
                           extent(workspace, workspace ? static_cast<int64_t>(workspace_bytes) : 0)};
    const Extent ins[] = {extent(q, ext[0]),         extent(k, ext[1]),   extent(v, ext[2]),
                          extent(mask_bias, msk),    extent(pair_bias, par), extent(out, ext[3]),
                          extent(lse, row),          extent(dout, ext[3])};
    for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a) {
        for (const Extent& in : ins)
            if (outs[a].overlaps(in)) return EVO_ERR_ALIASING;
        for (size_t c = a + 1; c < sizeof(outs) / sizeof(outs[0]); ++c)
            if (outs[a].overlaps(outs[c])) return EVO_ERR_ALIASING;
    }
    if (!bwd_supported(dtype, D)) return EVO_ERR_UNSUPPORTED;
    // rows of q, k, v and out (and so of their gradients) start 16-byte aligned
    for (const int64_t* t : qkvo)
        for (int a = 0; a < 4; ++a)
            if ((t[a] % 16) * es % 16) return EVO_ERR_MISALIGNED;  // t[a] >= 0; no overflow for any stride
    return EVO_OK;
}

extern "C" evo_status_t evo_attn_bwd_check(const void* q, const void* k, const void* v, const void* mask_bias,
                                           const void* pair_bias, const void* out, const float* lse,
                                           const void* dout, const void* dq, const void* dk, const void* dv,
                                           const void* dmask_bias, const void* dpair_bias, const float* delta,
                                           const void* workspace, size_t workspace_bytes, const evo_shape_t* shape,
                                           evo_dtype_t dtype) {
    if (!shape) return EVO_ERR_NULL_POINTER;
    evo_layout_t lay;
    evo_attn_dense_layout(shape, &lay);
    return evo_attn_bwd_check_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias,
                                      dpair_bias, delta, workspace, workspace_bytes, &lay, shape, dtype);
}

namespace {

// Workspace chunks a call can use: what the matrix-core path wants, capped by
// what the given workspace holds (0: none).  `a` carries the shape, the
// biases present and the strides.
int64_t usable_chunks(const evo::BwdArgs& a, evo_dtype_t dtype, size_t workspace_bytes) {
    const bool mfma = dtype == EVO_DTYPE_F32 ? evo::bwd_f32_mfma_eligible(a)
                                            : evo::bwd_mfma_eligible(a, static_cast<int>(dtype));
    if (!mfma) return 0;
    const int64_t want = evo::bwd_dpair_chunks(a.B, a.N, a.L, a.H);
    int64_t per = 4;  // bytes of one chunk's partial sums
    for (int64_t s : {a.B, a.H, a.L, evo::bwd_ws_row(a.L)}) per = mul_checked(per, s);
    if (per <= 0) return 0;
    const int64_t fit = static_cast<int64_t>(workspace_bytes / static_cast<size_t>(per));
    const int64_t c = want < fit ? want : fit;
    return c >= 2 ? c : 0;
}

}  // namespace

extern "C" size_t evo_attn_bwd_workspace_size(const evo_shape_t* shape, evo_dtype_t dtype) {
    if (!shape || shape->B < 1 || shape->N < 1 || shape->L < 1 || shape->H < 1 || shape->D < 1) return 0;
    int64_t par = 4;
    for (int64_t s : {shape->B, shape->H, shape->L}) par = mul_checked(par, s);
    if (par < 0) return 0;  // beyond 2^62 bytes; L is now below 2^62, so its rounded row length fits
    par = mul_checked(par, evo::bwd_ws_row(shape->L));
    if (par < 0) return 0;
    evo_layout_t lay;
    evo_attn_dense_layout(shape, &lay);
    // the workspace serves the pair gradient only: probe with a pair bias present
    static const char kPresent = 0;
    evo::BwdArgs probe{};
    probe.B = shape->B, probe.N = shape->N, probe.L = shape->L, probe.H = shape->H, probe.D = shape->D;
    probe.pair = &kPresent;
    probe.st = strides_of(lay);
    const int64_t c = usable_chunks(probe, dtype, ~static_cast<size_t>(0) >> 2);
    const int64_t bytes = mul_checked(par, c);
    return bytes < 0 ? 0 : static_cast<size_t>(bytes);
}

extern "C" evo_status_t evo_attn_bwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                             const void* pair_bias, const void* out, const float* lse,
                                             const void* dout, void* dq, void* dk, void* dv, void* dmask_bias,
                                             void* dpair_bias, float* delta, void* workspace, size_t workspace_bytes,
                                             const evo_layout_t* layout, const evo_shape_t* shape, evo_dtype_t dtype,
                                             void* stream) {
    const evo_status_t st = evo_attn_bwd_check_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                                       dmask_bias, dpair_bias, delta, workspace, workspace_bytes,
                                                       layout, shape, dtype);
    if (st != EVO_OK) return st;
    evo::BwdArgs a{q,  k,  v,  mask_bias,  pair_bias,  out,   lse,     dout,    dq,      dk,      dv,
                   dmask_bias, dpair_bias, delta, nullptr, 0, shape->B, shape->N, shape->L, shape->H, shape->D,
                   strides_of(*layout)};
    if (workspace && dpair_bias) {
        a.ws_chunks = usable_chunks(a, dtype, workspace_bytes);
        if (a.ws_chunks) a.ws = static_cast<float*>(workspace);
    }
    const hipError_t err = evo::launch_bwd(a, static_cast<int>(dtype), static_cast<hipStream_t>(stream));
    if (err == hipSuccess) return EVO_OK;
    g_last_hip_error = static_cast<int>(err);
    return EVO_ERR_HIP;
}

extern "C" evo_status_t evo_attn_bwd(const void* q, const void* k, const void* v, const void* mask_bias,
                                     const void* pair_bias, const void* out, const float* lse, const void* dout,
                                     void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias,
                                     float* delta, void* workspace, size_t workspace_bytes, const evo_shape_t* shape,
                                     evo_dtype_t dtype, void* stream) {
    if (!shape) return EVO_ERR_NULL_POINTER;
    evo_layout_t lay;
    evo_attn_dense_layout(shape, &lay);
    return evo_attn_bwd_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias,
                                delta, workspace, workspace_bytes, &lay, shape, dtype, stream);
}

extern "C" evo_status_t evo_trimul_check(const void* a, const void* w, const void* x,
                                         const evo_trimul_shape_t* shape, evo_trimul_direction_t direction,
                                         evo_dtype_t dtype) {
    if (!shape || !a || !w || !x) return EVO_ERR_NULL_POINTER;
    if (shape->B < 1 || shape->C < 1 || shape->L < 1) return EVO_ERR_BAD_SHAPE;
    if (direction != EVO_TRIMUL_OUTGOING && direction != EVO_TRIMUL_INCOMING) return EVO_ERR_BAD_SHAPE;
    if (dtype != EVO_DTYPE_F32 && dtype != EVO_DTYPE_BF16 && dtype != EVO_DTYPE_F16) return EVO_ERR_BAD_DTYPE;
    int64_t bytes = elem_size(dtype);
    for (int64_t s : {shape->B, shape->C, shape->L, shape->L}) bytes = mul_checked(bytes, s);
    if (bytes < 0) return EVO_ERR_BAD_SHAPE;
    for (const void* p : {a, w, x})
        if (!aligned16(p)) return EVO_ERR_MISALIGNED;
    const Extent ex = extent(x, bytes);
    if (ex.overlaps(extent(a, bytes)) || ex.overlaps(extent(w, bytes))) return EVO_ERR_ALIASING;
    // matrix-core kernel: 16-bit formats, one plane's rows (up to L + 128 of
    // them) addressed with 32-bit byte offsets
    const int64_t L = shape->L;
    if (dtype == EVO_DTYPE_F32 || L * L * 2 >= kMaxOffset || (L + 128) * L * 2 >= kMaxOffset32)
        return EVO_ERR_UNSUPPORTED;
    return EVO_OK;
}

extern "C" evo_status_t evo_trimul(const void* a, const void* w, void* x, const evo_trimul_shape_t* shape,
                                   evo_trimul_direction_t direction, evo_dtype_t dtype, void* stream) {
    const evo_status_t st = evo_trimul_check(a, w, x, shape, direction, dtype);
    if (st != EVO_OK) return st;
    const hipError_t err = evo::launch_trimul(a, w, x, shape->B * shape->C, shape->L,
                                              direction == EVO_TRIMUL_INCOMING, dtype == EVO_DTYPE_F16,
                                              static_cast<hipStream_t>(stream));
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
    case EVO_ERR_SCRATCH: return "the shape needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}
