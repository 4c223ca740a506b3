// Backward pass of Evoformer biased attention on the vector ALUs.
//
// The forward operation is out = softmax(q.K^T / sqrt(D) + mask + pair) . V
// (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南", hmyw.cn, sections 4
// and 5.2).  Section 5.4 of that page describes the backward pass the fused
// kernel pairs with: it keeps no [L, L] matrix, re-reads q, k, v, out and the
// per-row log-sum-exp, forms the row quantity delta, and produces bias
// gradients only when the caller asks for them.  The gradients follow from the
// definition by the chain rule; with P_ij = exp(s_ij - lse_i):
//
//   delta_i = dO_i . out_i
//   dS_ij   = P_ij (dO_i . v_j - delta_i)
//   dq_i    = sum_j dS_ij k_j / sqrt(D)      dk_j = sum_i dS_ij q_i / sqrt(D)
//   dv_j    = sum_i P_ij dO_i
//   dmask[b,n,j]   = sum_{h,i} dS[b,n,h,i,j] (the mask broadcasts over h, i)
//   dpair[b,h,i,j] = sum_n dS[b,n,h,i,j]     (the pair bias broadcasts over n)
//
// Three kernels, each owning its outputs so that every sum is formed in one
// place in a fixed order (no atomics; results do not depend on scheduling):
//   bwd_dq_kernel    one lane per query row: delta (written out), dq
//   bwd_dkdv_kernel  one lane per key: dk, dv for every head, then dmask
//   bwd_dpair_kernel one lane per query row, a group of keys: dpair over n
// All arithmetic is fp32; stored values are widened on load and rounded to
// nearest-even on store.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "evo_attn_launch.h"

namespace evo {
namespace {

constexpr int kLanes = 64;  // one wavefront per workgroup; one row per lane
constexpr int kBlk = 64;    // rows of the other axis staged in LDS per step
constexpr int kJG = 16;     // keys per dpair workgroup
constexpr float kLog2e = 1.4426950408889634f;

// Storage formats: S is the stored element type.
struct TF32 {
    using S = float;
    static __device__ float ld(const S* p, int64_t i) { return p[i]; }
    static __device__ void st(S* p, int64_t i, float x) { p[i] = x; }
};
struct TBF16 {
    using S = uint16_t;
    static __device__ float ld(const S* p, int64_t i) { return __uint_as_float(uint32_t(p[i]) << 16); }
    // round to nearest, ties to even; NaN stays a (quiet) NaN
    static __device__ void st(S* p, int64_t i, float x) {
        uint32_t u = __float_as_uint(x);
        if ((u & 0x7fffffffu) > 0x7f800000u) {
            p[i] = uint16_t((u >> 16) | 0x40u);
            return;
        }
        u += 0x7fffu + ((u >> 16) & 1u);
        p[i] = uint16_t(u >> 16);
    }
};
struct TF16 {
    using S = _Float16;
    static __device__ float ld(const S* p, int64_t i) { return float(p[i]); }
    static __device__ void st(S* p, int64_t i, float x) { p[i] = _Float16(x); }  // v_cvt_f16_f32: RNE
};

template <class T>
struct Params {
    using S = typename T::S;
    const S *q, *k, *v, *mask, *pair, *out, *dout;
    const float* lse;
    S *dq, *dk, *dv, *dmask, *dpair;
    float* delta;
    int64_t B, N, L, H;
    int64_t blocks_l;  // ceil(L / 64)
    int64_t groups_j;  // ceil(L / kJG)
    float scale;       // 1 / sqrt(D)
    Strides st;        // element strides; each gradient shares its tensor's (dout: out's, delta: lse's)
};

// exp(s - lse) for a live row; rows whose lse is -inf have no softmax and
// give every key the weight 0.
__device__ inline float weight(float s, float lse_i) {
    return lse_i == -INFINITY ? 0.f : exp2f((s - lse_i) * kLog2e);
}

// ---------------------------------------------------------------------------
// dq and delta: one lane per query i of (b, n, h); keys in LDS blocks.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(kLanes) void bwd_dq_kernel(Params<T> p) {
    __shared__ float kt[kBlk][D + 1];
    __shared__ float vt[kBlk][D + 1];
    __shared__ float ms[kBlk];
    __shared__ float pt[kLanes][kBlk + 1];  // pair tile: [query in block][key in block]

    int64_t id = blockIdx.x;
    const int64_t qb = id % p.blocks_l;
    id /= p.blocks_l;
    const int64_t h = id % p.H;
    id /= p.H;
    const int64_t n = id % p.N;
    const int64_t b = id / p.N;
    const int64_t L = p.L;
    const Strides& st = p.st;
    const int lane = threadIdx.x;
    const int64_t i = qb * kLanes + lane;
    const bool active = i < L;
    const int64_t irow = active ? i : L - 1;
    // elements (b, n, 0, h, 0) of q, k, v and out / dout
    const int64_t qs = b * st.q[0] + n * st.q[1] + h * st.q[3], ks = b * st.k[0] + n * st.k[1] + h * st.k[3];
    const int64_t vs = b * st.v[0] + n * st.v[1] + h * st.v[3], os = b * st.o[0] + n * st.o[1] + h * st.o[3];

    float qr[D], dor[D], acc[D];
    float delta = 0.f;
    for (int d = 0; d < D; ++d) {
        qr[d] = T::ld(p.q, qs + irow * st.q[2] + d);
        dor[d] = T::ld(p.dout, os + irow * st.o[2] + d);
        delta = fmaf(dor[d], T::ld(p.out, os + irow * st.o[2] + d), delta);
        acc[d] = 0.f;
    }
    const int64_t row = ((b * p.N + n) * p.H + h) * st.lrow + irow;
    const float lse_i = p.lse[row];
    if (active) p.delta[row] = delta;
    const typename T::S* mrow = p.mask ? p.mask + b * st.mb + n * st.mn : nullptr;
    const typename T::S* pmat = p.pair ? p.pair + b * st.pb + h * st.ph : nullptr;

    for (int64_t k0 = 0; k0 < L; k0 += kBlk) {
        const int cnt = int(L - k0 < kBlk ? L - k0 : kBlk);
        __syncthreads();
        for (int e = lane; e < kBlk * D; e += kLanes) {
            const int j = e / D, d = e % D;
            const bool in = j < cnt;
            kt[j][d] = in ? T::ld(p.k, ks + (k0 + j) * st.k[2] + d) : 0.f;
            vt[j][d] = in ? T::ld(p.v, vs + (k0 + j) * st.v[2] + d) : 0.f;
        }
        ms[lane] = (mrow && lane < cnt) ? T::ld(mrow, k0 + lane) : 0.f;
        if (pmat)
            for (int e = lane; e < kLanes * kBlk; e += kLanes) {
                const int r = e / kBlk, c = e % kBlk;
                const int64_t gi = qb * kLanes + r;
                pt[r][c] = (gi < L && c < cnt) ? T::ld(pmat, gi * st.pi + k0 + c) : 0.f;
            }
        __syncthreads();
        for (int j = 0; j < cnt; ++j) {
            float dot = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
                dot = fmaf(qr[d], kt[j][d], dot);
                dp = fmaf(dor[d], vt[j][d], dp);
            }
            float s = dot * p.scale + ms[j];
            if (pmat) s += pt[lane][j];
            const float ds = weight(s, lse_i) * (dp - delta);
            for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, kt[j][d], acc[d]);
        }
    }
    if (!active) return;
    for (int d = 0; d < D; ++d) T::st(p.dq, qs + i * st.q[2] + d, acc[d] * p.scale);
}

// ---------------------------------------------------------------------------
// dk, dv (every head) and dmask: one lane per key j of (b, n); queries in LDS
// blocks.  The workgroup visits the heads in order, so the mask gradient, a
// sum over heads and queries, is complete when it ends.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(kLanes) void bwd_dkdv_kernel(Params<T> p) {
    __shared__ float qt[kBlk][D + 1];
    __shared__ float dos[kBlk][D + 1];
    __shared__ float ls[kBlk];
    __shared__ float dl[kBlk];
    __shared__ float pt[kBlk][kLanes + 1];  // pair tile: [query in block][key in block]

    int64_t id = blockIdx.x;
    const int64_t kb = id % p.blocks_l;
    id /= p.blocks_l;
    const int64_t n = id % p.N;
    const int64_t b = id / p.N;
    const int64_t L = p.L, H = p.H;
    const Strides& st = p.st;
    const int lane = threadIdx.x;
    const int64_t j = kb * kLanes + lane;
    const bool active = j < L;
    const int64_t jrow = active ? j : L - 1;
    const int64_t mrow = b * st.mb + n * st.mn;
    const float mask_j = p.mask ? T::ld(p.mask, mrow + jrow) : 0.f;
    float dmask = 0.f;

    for (int64_t h = 0; h < H; ++h) {
        const int64_t qs = b * st.q[0] + n * st.q[1] + h * st.q[3], ks = b * st.k[0] + n * st.k[1] + h * st.k[3];
        const int64_t vs = b * st.v[0] + n * st.v[1] + h * st.v[3], os = b * st.o[0] + n * st.o[1] + h * st.o[3];
        const float* lrow = p.lse + ((b * p.N + n) * H + h) * st.lrow;
        const float* drow = p.delta + ((b * p.N + n) * H + h) * st.lrow;
        const typename T::S* pmat = p.pair ? p.pair + b * st.pb + h * st.ph : nullptr;
        float kr[D], vr[D], dk[D], dv[D];
        for (int d = 0; d < D; ++d) {
            kr[d] = T::ld(p.k, ks + jrow * st.k[2] + d);
            vr[d] = T::ld(p.v, vs + jrow * st.v[2] + d);
            dk[d] = 0.f;
            dv[d] = 0.f;
        }
        for (int64_t i0 = 0; i0 < L; i0 += kBlk) {
            const int cnt = int(L - i0 < kBlk ? L - i0 : kBlk);
            __syncthreads();
            for (int e = lane; e < kBlk * D; e += kLanes) {
                const int r = e / D, d = e % D;
                const bool in = r < cnt;
                qt[r][d] = in ? T::ld(p.q, qs + (i0 + r) * st.q[2] + d) : 0.f;
                dos[r][d] = in ? T::ld(p.dout, os + (i0 + r) * st.o[2] + d) : 0.f;
            }
            ls[lane] = lane < cnt ? lrow[i0 + lane] : -INFINITY;
            dl[lane] = lane < cnt ? drow[i0 + lane] : 0.f;
            if (pmat)
                for (int e = lane; e < kBlk * kLanes; e += kLanes) {
                    const int r = e / kLanes, c = e % kLanes;
                    const int64_t gj = kb * kLanes + c;
                    pt[r][c] = (r < cnt && gj < L) ? T::ld(pmat, (i0 + r) * st.pi + gj) : 0.f;
                }
            __syncthreads();
            for (int r = 0; r < cnt; ++r) {
                const float lse_i = ls[r];
                if (lse_i == -INFINITY) continue;  // a row without softmax: no gradient flows
                float dot = 0.f, dp = 0.f;
                for (int d = 0; d < D; ++d) {
                    dot = fmaf(qt[r][d], kr[d], dot);
                    dp = fmaf(dos[r][d], vr[d], dp);
                }
                float s = dot * p.scale + mask_j;
                if (pmat) s += pt[r][lane];
                const float w = exp2f((s - lse_i) * kLog2e);
                const float ds = w * (dp - dl[r]);
                for (int d = 0; d < D; ++d) {
                    dv[d] = fmaf(w, dos[r][d], dv[d]);
                    dk[d] = fmaf(ds, qt[r][d], dk[d]);
                }
                dmask += ds;
            }
        }
        if (active)
            for (int d = 0; d < D; ++d) {
                T::st(p.dk, ks + j * st.k[2] + d, dk[d] * p.scale);
                T::st(p.dv, vs + j * st.v[2] + d, dv[d]);
            }
    }
    if (active && p.dmask) T::st(p.dmask, mrow + j, dmask);
}

// ---------------------------------------------------------------------------
// dpair: one lane per query i, kJG keys per workgroup, the sum over n formed
// in order in registers.  The pair values of the tile do not depend on n and
// are loaded once.
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ __launch_bounds__(kLanes) void bwd_dpair_kernel(Params<T> p) {
    __shared__ float kt[kJG][D + 1];
    __shared__ float vt[kJG][D + 1];
    __shared__ float ms[kJG];

    int64_t id = blockIdx.x;
    const int64_t jg = id % p.groups_j;
    id /= p.groups_j;
    const int64_t ib = id % p.blocks_l;
    id /= p.blocks_l;
    const int64_t h = id % p.H;
    const int64_t b = id / p.H;
    const int64_t L = p.L, H = p.H;
    const Strides& st = p.st;
    const int lane = threadIdx.x;
    const int64_t i = ib * kLanes + lane;
    const bool active = i < L;
    const int64_t irow = active ? i : L - 1;
    const int64_t j0 = jg * kJG;
    const int jcnt = int(L - j0 < kJG ? L - j0 : kJG);
    const int64_t pmat = b * st.pb + h * st.ph;
    const typename T::S* prow = p.pair + pmat + irow * st.pi + j0;

    float pr[kJG], acc[kJG];
#pragma unroll
    for (int c = 0; c < kJG; ++c) {
        pr[c] = c < jcnt ? T::ld(prow, c) : 0.f;
        acc[c] = 0.f;
    }
    for (int64_t n = 0; n < p.N; ++n) {
        const int64_t qs = b * st.q[0] + n * st.q[1] + h * st.q[3], ks = b * st.k[0] + n * st.k[1] + h * st.k[3];
        const int64_t vs = b * st.v[0] + n * st.v[1] + h * st.v[3], os = b * st.o[0] + n * st.o[1] + h * st.o[3];
        float qr[D], dor[D];
        for (int d = 0; d < D; ++d) {
            qr[d] = T::ld(p.q, qs + irow * st.q[2] + d);
            dor[d] = T::ld(p.dout, os + irow * st.o[2] + d);
        }
        const int64_t row = ((b * p.N + n) * H + h) * st.lrow + irow;
        const float lse_i = p.lse[row];
        const float delta = p.delta[row];
        __syncthreads();
        for (int e = lane; e < kJG * D; e += kLanes) {
            const int c = e / D, d = e % D;
            const bool in = c < jcnt;
            kt[c][d] = in ? T::ld(p.k, ks + (j0 + c) * st.k[2] + d) : 0.f;
            vt[c][d] = in ? T::ld(p.v, vs + (j0 + c) * st.v[2] + d) : 0.f;
        }
        if (lane < kJG) ms[lane] = (p.mask && lane < jcnt) ? T::ld(p.mask, b * st.mb + n * st.mn + j0 + lane) : 0.f;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kJG; ++c) {
            float dot = 0.f, dp = 0.f;
            for (int d = 0; d < D; ++d) {
                dot = fmaf(qr[d], kt[c][d], dot);
                dp = fmaf(dor[d], vt[c][d], dp);
            }
            const float s = dot * p.scale + ms[c] + pr[c];
            acc[c] = fmaf(weight(s, lse_i), dp - delta, acc[c]);
        }
    }
    if (!active) return;
    typename T::S* out = p.dpair + pmat + i * st.pi + j0;
#pragma unroll
    for (int c = 0; c < kJG; ++c)
        if (c < jcnt) T::st(out, c, acc[c]);
}

// stages: a mask of kStageDq | kStageDkDv | kStageDpair, the kernels to run here
template <class T, int D>
hipError_t launch_all(const BwdArgs& a, unsigned stages, hipStream_t stream) {
    using S = typename T::S;
    Params<T> p;
    p.q = static_cast<const S*>(a.q);
    p.k = static_cast<const S*>(a.k);
    p.v = static_cast<const S*>(a.v);
    p.mask = static_cast<const S*>(a.mask);
    p.pair = static_cast<const S*>(a.pair);
    p.out = static_cast<const S*>(a.out);
    p.dout = static_cast<const S*>(a.dout);
    p.lse = a.lse;
    p.dq = static_cast<S*>(a.dq);
    p.dk = static_cast<S*>(a.dk);
    p.dv = static_cast<S*>(a.dv);
    p.dmask = static_cast<S*>(a.dmask);
    p.dpair = static_cast<S*>(a.dpair);
    p.delta = a.delta;
    p.B = a.B;
    p.N = a.N;
    p.L = a.L;
    p.H = a.H;
    p.blocks_l = (a.L + kLanes - 1) / kLanes;
    p.groups_j = (a.L + kJG - 1) / kJG;
    p.scale = float(1.0 / std::sqrt(double(D)));
    p.st = a.st;

    const int64_t g_dq = a.B * a.N * a.H * p.blocks_l;
    const int64_t g_kv = a.B * a.N * p.blocks_l;
    const int64_t g_pair = a.B * a.H * p.blocks_l * p.groups_j;
    if (g_dq > 0x7fffffff || g_kv > 0x7fffffff || g_pair > 0x7fffffff) return hipErrorInvalidConfiguration;

    // delta is written by the dq kernel and read by the other two, which
    // follow it on the same stream.
    void* args[] = {&p};
    hipError_t e = hipSuccess;
    if (stages & kStageDq)
        e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<T, D>), dim3(unsigned(g_dq)), dim3(kLanes),
                            args, 0, stream);
    if (e == hipSuccess && (stages & kStageDkDv))
        e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<T, D>), dim3(unsigned(g_kv)),
                            dim3(kLanes), args, 0, stream);
    if (e == hipSuccess && (stages & kStageDpair) && a.dpair)
        e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dpair_kernel<T, D>), dim3(unsigned(g_pair)),
                            dim3(kLanes), args, 0, stream);
    return e;
}

template <class T>
hipError_t launch_dim(const BwdArgs& a, unsigned stages, hipStream_t stream) {
    switch (a.D) {
    case 8: return launch_all<T, 8>(a, stages, stream);
    case 16: return launch_all<T, 16>(a, stages, stream);
    case 32: return launch_all<T, 32>(a, stages, stream);
    case 64: return launch_all<T, 64>(a, stages, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_valu(const BwdArgs& a, int dtype, unsigned stages, hipStream_t stream) {
    if (!stages) return hipSuccess;
    switch (dtype) {
    case 0: return launch_dim<TF32>(a, stages, stream);
    case 1: return launch_dim<TBF16>(a, stages, stream);
    case 2: return launch_dim<TF16>(a, stages, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The matrix-core kernels take the stages they implement for the shapes
// they accept (every dtype with D in {8, 16, 32, 64} and any L, on layouts
// whose rows span every head and fit 32-bit offsets); the vector-ALU kernels take
// the rest.  The dq stage goes first in either case: it writes delta.
hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t stream) {
    if (dtype == 0 && bwd_f32_mfma_eligible(a)) {
        hipError_t e = launch_bwd_f32_mfma(a, kBwdF32MfmaStages, stream);
        if (e != hipSuccess) return e;
        return launch_valu(a, dtype, (kStageDq | kStageDkDv | kStageDpair) & ~kBwdF32MfmaStages, stream);
    }
    const unsigned mfma = bwd_mfma_eligible(a, dtype) ? kBwdMfmaStages : 0u;
    hipError_t e = hipSuccess;
    if (mfma & kStageDq) e = launch_bwd_mfma(a, dtype, kStageDq, stream);
    else e = launch_valu(a, dtype, kStageDq, stream);
    if (e != hipSuccess) return e;
    if (mfma & ~kStageDq) e = launch_bwd_mfma(a, dtype, mfma & ~kStageDq, stream);
    if (e != hipSuccess) return e;
    return launch_valu(a, dtype, (kStageDkDv | kStageDpair) & ~mfma, stream);
}

}  // namespace evo
