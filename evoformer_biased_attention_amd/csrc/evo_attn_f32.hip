// fp32 forward kernel: full-precision path for small problems.
//
// Computes, per query row, softmax(q.K^T / sqrt(D) + mask + pair) . V and the
// natural-log LSE (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
// hmyw.cn, sections 4, 5.2 and 5.4) entirely in fp32 on the vector ALUs: this
// path exists for callers that need fp32 accuracy, not for throughput.
//
// One 64-lane wavefront per (b, n, h, block of 64 queries); each lane owns one
// query and keeps q, the output accumulator and its running max / sum in
// registers.  Keys are visited in blocks of 64 staged in LDS, and each key
// updates the lane's state with a one-pass (online) softmax.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "evo_attn_launch.h"

namespace evo {
namespace {

constexpr int kQ = 64;  // queries per workgroup (one wavefront)
constexpr int kK = 64;  // keys per LDS block

struct F32Params {
    const float *q, *k, *v, *mask, *pair;
    float *out, *lse;
    int64_t N, L, H, qblocks;
    Strides st;
    float scale;
};

template <int D>
__global__ __launch_bounds__(kQ) void fwd_f32_kernel(F32Params p) {
    const float* __restrict__ q = p.q;
    const float* __restrict__ k = p.k;
    const float* __restrict__ v = p.v;
    const int64_t N = p.N, L = p.L, H = p.H, qblocks = p.qblocks;
    const float scale = p.scale;
    const Strides& st = p.st;
    __shared__ float ks[kK][D + 1];
    __shared__ float vs[kK][D + 1];

    // workgroup -> (b, n, h, query block), query block fastest
    int64_t id = blockIdx.x;
    const int64_t qb = id % qblocks;
    id /= qblocks;
    const int64_t h = id % H;
    id /= H;
    const int64_t n = id % N;
    const int64_t b = id / N;

    const int lane = threadIdx.x;
    const int64_t i = qb * kQ + lane;
    const bool active = i < L;
    const int64_t qbase = b * st.q[0] + n * st.q[1] + h * st.q[3];
    const int64_t kbase = b * st.k[0] + n * st.k[1] + h * st.k[3];
    const int64_t vbase = b * st.v[0] + n * st.v[1] + h * st.v[3];

    float qr[D], acc[D];
    const int64_t irow = active ? i : L - 1;
    for (int d = 0; d < D; ++d) {
        qr[d] = q[qbase + irow * st.q[2] + d];
        acc[d] = 0.f;
    }
    const float* mrow = p.mask ? p.mask + b * st.mb + n * st.mn : nullptr;
    const float* prow = p.pair ? p.pair + b * st.pb + h * st.ph + irow * st.pi : nullptr;

    float m = -INFINITY, l = 0.f;
    for (int64_t k0 = 0; k0 < L; k0 += kK) {
        const int cnt = (int)((L - k0) < kK ? (L - k0) : kK);
        __syncthreads();
        for (int e = lane; e < kK * D; e += kQ) {
            const int j = e / D, d = e % D;
            float kv = 0.f, vv = 0.f;
            if (j < cnt) {
                kv = k[kbase + (k0 + j) * st.k[2] + d];
                vv = v[vbase + (k0 + j) * st.v[2] + d];
            }
            ks[j][d] = kv;
            vs[j][d] = vv;
        }
        __syncthreads();
        for (int j = 0; j < cnt; ++j) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[j][d], dot);
            float s = dot * scale;
            if (mrow) s += mrow[k0 + j];
            if (prow) s += prow[k0 + j];
            if (s == -INFINITY) continue;  // contributes nothing
            const float mn = fmaxf(m, s);
            const float alpha = expf(m - mn);  // 0 when m was -inf
            const float p = expf(s - mn);
            l = l * alpha + p;
            for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d] * alpha);
            m = mn;
        }
    }
    if (!active) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = p.out + b * st.o[0] + n * st.o[1] + h * st.o[3] + i * st.o[2];
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
    if (p.lse) p.lse[((b * N + n) * H + h) * st.lrow + i] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int64_t qblocks = (a.L + kQ - 1) / kQ;
    const int64_t blocks = a.B * a.N * a.H * qblocks;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    F32Params p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.mask = static_cast<const float*>(a.mask);
    p.pair = static_cast<const float*>(a.pair);
    p.out = static_cast<float*>(a.out);
    p.lse = a.lse;
    p.N = a.N, p.L = a.L, p.H = a.H, p.qblocks = qblocks;
    p.st = a.st;
    p.scale = (float)(1.0 / std::sqrt((double)D));
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_kernel<D>), dim3((unsigned)blocks), dim3(kQ),
                           args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
    switch (a.D) {
    case 8: return launch<8>(a, stream);
    case 16: return launch<16>(a, stream);
    case 32: return launch<32>(a, stream);
    case 64: return launch<64>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace evo
