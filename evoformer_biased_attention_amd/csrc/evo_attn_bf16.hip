// bf16 forward kernel for head dimension 32 on gfx950 (MI355X).
//
// Operation (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
// hmyw.cn, sections 4, 5.2 and 5.4): for each (b, n, h) slice and query i,
//   out_i = softmax_j(q_i.k_j / sqrt(D) + mask[b,n,j] + pair[b,h,i,j]) . V,
//   lse_i = ln sum_j exp(...),
// with the [L, L] score matrix never written to memory.
//
// Design (CDNA4, wave64):
//  * Both dense contractions run on v_mfma_f32_16x16x32_bf16 with fp32
//    accumulation.  Scores are formed transposed, S^T = K . Q^T, so that the
//    MFMA result layout puts one query per lane column: lane (c + 16 g) holds
//    query c and keys 4g..4g+3 of every 16-key tile.  Row statistics (max,
//    sum) are therefore lane-local up to a 4-way cross-lane reduction, and the
//    probabilities of a lane are exactly the B operand of the second MFMA,
//    O^T = V^T . P^T, whose result again has one query per lane column: the
//    online-softmax rescale of the output accumulator needs no data movement.
//  * V is the only operand that needs its contraction index (the key) made
//    contiguous per lane; each 64-key block of V is written transposed into
//    LDS once per workgroup and read as 8-byte rows by every wavefront.
//  * Q and K operands are read straight from global memory as 16-byte rows
//    (D = 32 bf16 = 64 contiguous bytes per row); the 4 wavefronts of a
//    workgroup share the K rows through the L1 cache.
//  * The softmax works in base 2: s2 = s * log2(e), exp2 on v_exp_f32.
//
// Workgroup = 4 wavefronts x 32 queries = 128 queries of one (b, n, h).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "evo_attn_launch.h"

namespace evo {
namespace {

// bf16 data is moved as integers; __bf16 vectors appear only as MFMA operands.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int D = 32;
constexpr int kWaves = 4;
constexpr int kQTiles = 2;                    // 16-query MFMA tiles per wavefront
constexpr int kWaveQ = 16 * kQTiles;          // 32 queries per wavefront
constexpr int kBlockQ = kWaves * kWaveQ;      // 128 queries per workgroup
constexpr int kKB = 64;                       // keys per iteration
constexpr int kKT = kKB / 16;                 // 16-key tiles per iteration
constexpr int kVtStride = kKB + 8;            // LDS row (one d) of transposed V, in bf16
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
    const u16* q;
    const u16* k;
    const u16* v;
    const u16* mask;  // nullable
    const u16* pair;  // nullable
    u16* out;
    float* lse;       // nullable
    int64_t N, L, H;
    int64_t qblocks;  // ceil(L / kBlockQ)
    int64_t total;    // number of workgroups
    float c1;         // log2(e) / sqrt(D)
};

__device__ inline float bf2f(u16 x) { return __builtin_bit_cast(float, (uint32_t)x << 16); }

// Two floats -> two bf16 (round to nearest even) packed in one dword, low half first.
__device__ inline uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ inline bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ inline uint4 load16(const u16* p) { return *reinterpret_cast<const uint4*>(p); }

// Workgroups are dealt round-robin over the 8 XCDs.  Renumber them so that
// each XCD receives one contiguous range of the logical order (b, h, n, query
// block): the query blocks of one (n, h) share K/V, and all sequences n of one
// head share the pair bias, within a single XCD's L2.
__device__ inline int64_t logical_block(int64_t hw, int64_t total) {
    const int64_t xcd = hw % 8, j = hw / 8;
    const int64_t per = total / 8, extra = total % 8;  // the first `extra` XCDs get one more
    return xcd < extra ? xcd * (per + 1) + j : extra * (per + 1) + (xcd - extra) * per + j;
}

__global__ __launch_bounds__(kWaves * 64) void fwd_bf16_d32_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) u16 vt[D * kVtStride];

    int64_t id = logical_block(blockIdx.x, p.total);
    const int64_t qb = id % p.qblocks;
    id /= p.qblocks;
    const int64_t n = id % p.N;
    id /= p.N;
    const int64_t h = id % p.H;
    const int64_t b = id / p.H;

    const int64_t L = p.L, HD = p.H * D;
    const int64_t slice = ((b * p.N + n) * L * p.H + h) * D;  // element (b, n, 0, h, 0)
    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64;
    const int c = lane % 16, g = lane / 16;  // MFMA column (query) and lane group
    const int64_t q0 = qb * kBlockQ + wave * kWaveQ;

    // Q operands: B[k = d][n = query] -> lane (c + 16g) holds q[query c][8g .. 8g+7].
    bf16x8 qop[kQTiles];
    for (int t = 0; t < kQTiles; ++t) {
        int64_t i = q0 + 16 * t + c;
        if (i >= L) i = L - 1;
        qop[t] = as_bf16x8(load16(p.q + slice + i * HD + 8 * g));
    }

    const u16* mrow = p.mask ? p.mask + (b * p.N + n) * L : nullptr;
    const u16* pbase = p.pair ? p.pair + (b * p.H + h) * L * L : nullptr;

    f32x4 oacc[kQTiles][2];
    float mrun[kQTiles], lrun[kQTiles];
    for (int t = 0; t < kQTiles; ++t) {
        oacc[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        oacc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        mrun[t] = -INFINITY;
        lrun[t] = 0.f;
    }

    for (int64_t k0 = 0; k0 < L; k0 += kKB) {
        // ---- stage V[k0 .. k0+63][0..31] transposed into LDS: vt[d][key] ----
        {
            const int key = tid / 4, dc = (tid % 4) * 8;
            const int64_t j = k0 + key;
            uint4 val = {0u, 0u, 0u, 0u};
            if (j < L) val = load16(p.v + slice + j * HD + dc);
            const uint32_t w[4] = {val.x, val.y, val.z, val.w};
            __syncthreads();  // previous iteration's readers are done
            for (int e = 0; e < 8; ++e) vt[(dc + e) * kVtStride + key] = (u16)(w[e / 2] >> (16 * (e % 2)));
        }

        // ---- S^T = K . Q^T for 4 key tiles x kQTiles query tiles ----
        f32x4 s[kQTiles][kKT];
        for (int kt = 0; kt < kKT; ++kt) {
            int64_t j = k0 + 16 * kt + c;  // A[m = key][k = d]: lane (c + 16g) holds k[key c][8g..]
            if (j >= L) j = L - 1;
            const bf16x8 kop = as_bf16x8(load16(p.k + slice + j * HD + 8 * g));
            for (int t = 0; t < kQTiles; ++t)
                s[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }

        // ---- scale, biases, masking of keys past L (base-2 units) ----
        for (int kt = 0; kt < kKT; ++kt) {
            const int64_t jb = k0 + 16 * kt + 4 * g;  // this lane's 4 keys: jb .. jb+3
            float mb[4] = {0.f, 0.f, 0.f, 0.f};
            if (mrow)
                for (int r = 0; r < 4; ++r) mb[r] = jb + r < L ? bf2f(mrow[jb + r]) : 0.f;
            for (int t = 0; t < kQTiles; ++t) {
                int64_t i = q0 + 16 * t + c;
                if (i >= L) i = L - 1;
                for (int r = 0; r < 4; ++r) {
                    const int64_t j = jb + r;
                    float bias = mb[r];
                    if (pbase && j < L) bias += bf2f(pbase[i * L + j]);
                    s[t][kt][r] = j < L ? fmaf(s[t][kt][r], p.c1, bias * kLog2e) : -INFINITY;
                }
            }
        }

        // ---- online softmax per query tile ----
        bf16x8 pop[kQTiles][2];
        for (int t = 0; t < kQTiles; ++t) {
            float mx = -INFINITY;
            for (int kt = 0; kt < kKT; ++kt)
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[t][kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(mrun[t], mx);
            const float msub = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrun[t] - msub);
            float sum = 0.f;
            for (int kt = 0; kt < kKT; ++kt)
                for (int r = 0; r < 4; ++r) {
                    const float pv = __builtin_amdgcn_exp2f(s[t][kt][r] - msub);
                    s[t][kt][r] = pv;
                    sum += pv;
                }
            lrun[t] = lrun[t] * alpha + sum;  // per-lane partial sum over this lane's keys
            mrun[t] = mnew;
            for (int dh = 0; dh < 2; ++dh) oacc[t][dh] *= alpha;
            // B operand of O^T = V^T P^T: element e of 32-key chunk cc is key 32cc + 16(e/4) + 4g + e%4
            for (int cc = 0; cc < 2; ++cc) {
                const f32x4 a = s[t][2 * cc], b = s[t][2 * cc + 1];
                pop[t][cc] = as_bf16x8(uint4{pack2(a[0], a[1]), pack2(a[2], a[3]), pack2(b[0], b[1]), pack2(b[2], b[3])});
            }
        }

        __syncthreads();  // transposed V visible

        // ---- O^T += V^T . P^T ----
        for (int cc = 0; cc < 2; ++cc)
            for (int dh = 0; dh < 2; ++dh) {
                // A[m = d][k]: lane (c + 16g) holds V[key(g, e)][16dh + c]
                const u16* row = vt + (16 * dh + c) * kVtStride + 32 * cc + 4 * g;
                const uint2 lo = *reinterpret_cast<const uint2*>(row);
                const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
                const bf16x8 vop = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
                for (int t = 0; t < kQTiles; ++t)
                    oacc[t][dh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[t][cc], oacc[t][dh], 0, 0, 0);
            }
    }

    // ---- epilogue: normalise, write O (bf16) and LSE (fp32, natural log) ----
    for (int t = 0; t < kQTiles; ++t) {
        float l = lrun[t];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int64_t i = q0 + 16 * t + c;
        if (i >= L) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        for (int dh = 0; dh < 2; ++dh) {
            // lane (c + 16g) holds O^T[d = 16dh + 4g + r][query c], r = 0..3
            u16* dst = p.out + slice + i * HD + 16 * dh + 4 * g;
            const f32x4 o = oacc[t][dh] * inv;
            *reinterpret_cast<uint2*>(dst) = uint2{pack2(o[0], o[1]), pack2(o[2], o[3])};
        }
        if (p.lse && g == 0)
            p.lse[((b * p.N + n) * p.H + h) * L + i] = l > 0.f ? (mrun[t] + __log2f(l)) * kLn2 : -INFINITY;
    }
}

}  // namespace

hipError_t launch_fwd_bf16_d32(const FwdArgs& a, hipStream_t stream) {
    Params p;
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.mask = static_cast<const u16*>(a.mask);
    p.pair = static_cast<const u16*>(a.pair);
    p.out = static_cast<u16*>(a.out);
    p.lse = a.lse;
    p.N = a.N;
    p.L = a.L;
    p.H = a.H;
    p.qblocks = (a.L + kBlockQ - 1) / kBlockQ;
    p.total = a.B * a.N * a.H * p.qblocks;
    p.c1 = (float)(1.4426950408889634 / std::sqrt((double)D));
    if (p.total > 0x7fffffff) return hipErrorInvalidConfiguration;
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_d32_kernel), dim3((unsigned)p.total),
                           dim3(kWaves * 64), args, 0, stream);
}

}  // namespace evo
