// Microbenchmarks of the gfx950 (MI355X) units the attention kernels lean on:
// the bf16 matrix cores, the transcendental and plain vector ALU, their
// overlap, LDS reads, global -> LDS copies and HBM streaming.  Each result is
// the sustained rate of one instruction kind with enough independent work in
// flight to hide its latency, timed with HIP events over the whole grid (and
// with the shader clock inside each wave, which gives cycles per instruction).
//
// Usage: micro [test ...]   tests: mfma exp fma cvt mix coissue lds dma dmaissue hbm
// (no argument: all).  One JSON object per line on stdout.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#define CHECK(x)                                                                              \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(1);                                                                          \
        }                                                                                     \
    } while (0)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kChains = 8;  // independent dependency chains per wave

__device__ inline bf16x8 bf16_operand(int lane, int salt) {
    bf16x8 v;
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)(0.001f * (float)((lane * 7 + e * 3 + salt) % 17));
    return v;
}

// `iters` x kChains independent v_mfma_f32_16x16x32_bf16 per wave.
__global__ void k_mfma(float* out, int iters, long long* clk) {
    const int lane = threadIdx.x & 63;
    const bf16x8 a = bf16_operand(lane, 1), b = bf16_operand(lane, 2);
    f32x4 acc[kChains];
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
    const long long t0 = clock64();
#pragma unroll 4
    for (int i = 0; i < iters; ++i)
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    const long long t1 = clock64();
    float s = 0.f;
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + threadIdx.x) / 64] = t1 - t0;
}

// `iters` x kChains independent v_exp_f32 per wave (the negation is an input modifier).
__global__ void k_exp(float* out, int iters, long long* clk) {
    const int lane = threadIdx.x & 63;
    float x[kChains];
    for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
    const long long t0 = clock64();
#pragma unroll 4
    for (int i = 0; i < iters; ++i)
        for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
    const long long t1 = clock64();
    float s = 0.f;
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + threadIdx.x) / 64] = t1 - t0;
}

// `iters` x kChains independent v_fma_f32 per wave.
__global__ void k_fma(float* out, int iters, long long* clk, float a, float b) {
    const int lane = threadIdx.x & 63;
    float x[kChains];
    for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
    const long long t0 = clock64();
#pragma unroll 4
    for (int i = 0; i < iters; ++i)
        for (int c = 0; c < kChains; ++c) x[c] = fmaf(x[c], a, b);
    const long long t1 = clock64();
    float s = 0.f;
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + threadIdx.x) / 64] = t1 - t0;
}

// `iters` x kChains v_cvt_pk_bf16_f32 per wave (each result feeds the next input).
__global__ void k_cvt(float* out, int iters, long long* clk) {
    const int lane = threadIdx.x & 63;
    float x[kChains];
    for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
    const long long t0 = clock64();
#pragma unroll 4
    for (int i = 0; i < iters; ++i)
        for (int c = 0; c < kChains; ++c) {
            const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[c], x[c]}, bf16x2));
            x[c] = __builtin_bit_cast(float, w);
        }
    const long long t1 = clock64();
    float s = 0.f;
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + threadIdx.x) / 64] = t1 - t0;
}

// Per iteration: one MFMA (four rotating accumulators) and E independent
// exponentials (FMA: fma instead) in the same wave: does the wave issue the
// vector instructions while the matrix core works?
template <int E, bool FMA = false>
__global__ void k_mix(float* out, int iters, long long* clk) {
    const int lane = threadIdx.x & 63;
    const bf16x8 a = bf16_operand(lane, 1), b = bf16_operand(lane, 2);
    f32x4 acc[4];
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
    float x[kChains];
    for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
    const long long t0 = clock64();
    for (int i = 0; i < iters; i += 4)
        for (int c = 0; c < 4; ++c) {
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
            for (int e = 0; e < E; ++e) {
                float& y = x[(c * E + e) % kChains];
                y = FMA ? fmaf(y, 0.999f, 0.001f) : __builtin_amdgcn_exp2f(-y);
            }
        }
    const long long t1 = clock64();
    float s = 0.f;
    for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    for (int c = 0; c < kChains; ++c) s += x[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + threadIdx.x) / 64] = t1 - t0;
}

// Two kinds of waves in one workgroup of 8: waves 0-3 run MFMAs, waves 4-7
// vector work (wave w runs on SIMD w % 4, so each SIMD holds one of each).
// KIND of the vector work: 0 exponentials, 1 fma, 2 the softmax mix (per 8
// values: 8 fma, 8 exponentials, 4 bf16 conversions).
template <int KIND>
__global__ void k_coissue(float* out, int iters_mfma, int iters_exp, long long* clk) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float s = 0.f;
    long long t0 = clock64();
    if (wave < 4) {
        const bf16x8 a = bf16_operand(lane, 1), b = bf16_operand(lane, 2);
        f32x4 acc[kChains];
        for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, (float)c};
        for (int i = 0; i < iters_mfma; ++i)
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
        for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3];
    } else {
        float x[kChains];
        for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
        for (int i = 0; i < iters_exp; ++i) {
            if (KIND == 0)
                for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
            else if (KIND == 1)
                for (int c = 0; c < kChains; ++c) x[c] = fmaf(x[c], 0.999f, 0.001f);
            else {
                for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(fmaf(x[c], -0.9f, 0.01f));
                for (int c = 0; c < kChains; c += 2) {
                    const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[c], x[c + 1]}, bf16x2));
                    x[c] = __builtin_bit_cast(float, w & 0xffff0000u);
                }
            }
        }
        for (int c = 0; c < kChains; ++c) s += x[c];
    }
    const long long t1 = clock64();
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + threadIdx.x) / 64] = t1 - t0;
}

// LDS reads: every wave reads 16 bytes per lane per instruction from
// consecutive 1 KB rows (no bank conflicts), `iters` x 8 reads.
__global__ void k_lds(float* out, int iters, long long* clk) {
    __shared__ uint4 buf[4096];  // 64 KB
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 4096; i += blockDim.x) buf[i] = uint4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    uint32_t acc = 0;
    const long long t0 = clock64();
    for (int i = 0; i < iters; ++i) {
        uint4 r[8];
        for (int u = 0; u < 8; ++u) r[u] = buf[((i * 8 + u + wave * 5) & 63) * 64 + lane];
        for (int u = 0; u < 8; ++u) acc += r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
    }
    const long long t1 = clock64();
    out[blockIdx.x * blockDim.x + tid] = (float)acc;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + tid) / 64] = t1 - t0;
}

// Global -> LDS copies (buffer loads with the LDS destination bit, 16 bytes
// per lane, each wave request a whole 1 KB) from a buffer of `bytes` bytes
// that stays in L2; 8 copies in flight per wave, `iters` rounds.
__global__ void k_dma(const uint4* src, uint32_t bytes, float* out, int iters, long long* clk) {
    __shared__ uint4 buf[8][1024];  // 8 slots of 16 KB: one 1 KB segment per wave and slot
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(src), (short)0, (int)bytes, 0x00020000);
    const uint32_t seg = bytes / 1024;
    const long long t0 = clock64();
    for (int i = 0; i < iters; ++i) {
        for (int u = 0; u < 8; ++u) {
            const uint32_t off = (((uint32_t)(blockIdx.x * 131 + i * 8 + u) * 64 + wave) % seg) * 1024 + 16 * lane;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&buf[u][64 * wave],
                                                     16, (int)off, 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    const long long t1 = clock64();
    __syncthreads();
    out[blockIdx.x * blockDim.x + tid] = (float)buf[tid & 7][tid].x;
    if (lane == 0) clk[(blockIdx.x * blockDim.x + tid) / 64] = t1 - t0;
}

// Issue cost of global -> LDS copies: each wave issues 8 copy requests back
// to back (16 bytes per lane, 1 KB per request, L2-resident source), timing
// the issue alone with the shader clock; MODE 0: a new LDS address (M0) per
// request, 1: one M0 for all eight, 2: plain loads into registers instead.
template <int MODE>
__global__ void k_dma_issue(const uint4* src, uint32_t bytes, float* out, long long* clk) {
    __shared__ uint4 buf[8][1024];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(src), (short)0, (int)bytes, 0x00020000);
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)&buf[0][64 * (wave & 15)]);
    const uint32_t seg = bytes / 1024;
    uint4 acc = {0u, 0u, 0u, 0u};
    long long total = 0;
    for (int rep = 0; rep < 16; ++rep) {
        const uint32_t off0 = ((uint32_t)(blockIdx.x * 64 + rep * 8 + wave) % seg) * 1024 + 16 * lane;
        const long long t0 = clock64();
        if (MODE == 2) {
            uint4 v[8];
            for (int u = 0; u < 8; ++u)
                v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off0 + u * 4096), 0, 0));
            const long long t1 = clock64();
            total += t1 - t0;
            for (int u = 0; u < 8; ++u) acc.x ^= v[u].x ^ v[u].w;
        } else {
            for (int u = 0; u < 8; ++u) {
                const uint32_t m0 = MODE == 0 ? base + (uint32_t)u * 16384u : base;
                asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                             :
                             : "s"(m0), "v"(off0 + u * 4096), "s"(r)
                             : "memory", "m0");
            }
            const long long t1 = clock64();
            total += t1 - t0;
        }
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    out[blockIdx.x * blockDim.x + tid] = (float)(buf[tid & 7][tid].x + acc.x);
    if (lane == 0) clk[(blockIdx.x * blockDim.x + tid) / 64] = total;
}

// HBM streaming copy: grid-stride loop of 16-byte loads and stores.
__global__ void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

struct Timer {
    hipEvent_t a, b;
    Timer() {
        CHECK(hipEventCreate(&a));
        CHECK(hipEventCreate(&b));
    }
    void start() { CHECK(hipEventRecord(a, 0)); }
    double stop_ms() {
        CHECK(hipEventRecord(b, 0));
        CHECK(hipEventSynchronize(b));
        float ms = 0.f;
        CHECK(hipEventElapsedTime(&ms, a, b));
        return ms;
    }
};

int g_cus = 0;
float* g_out = nullptr;
long long* g_clk = nullptr;
constexpr size_t kMaxThreads = 1 << 22;

// mean over waves of the per-wave shader-clock count
double mean_clk(int waves) {
    std::vector<long long> h(waves);
    CHECK(hipMemcpy(h.data(), g_clk, sizeof(long long) * waves, hipMemcpyDeviceToHost));
    double s = 0;
    for (long long x : h) s += (double)x;
    return s / waves;
}

// Launch `launch(blocks)` once to warm up, then time it; returns ms.
template <class F>
double timed(F launch) {
    launch();
    CHECK(hipDeviceSynchronize());
    Timer t;
    t.start();
    launch();
    return t.stop_ms();
}

void run_rate(const char* name, const char* unit_what, double per_wave_iter_ops, int waves_per_simd, int iters,
              void (*kern)(float*, int, long long*), double ops_per_inst) {
    const int threads = 64 * 4 * waves_per_simd;  // one workgroup per CU, waves_per_simd waves on each SIMD
    const int blocks = g_cus;
    const double ms = timed([&] { hipLaunchKernelGGL(kern, dim3(blocks), dim3(threads), 0, 0, g_out, iters, g_clk); });
    const int waves = blocks * threads / 64;
    const double clk = mean_clk(waves);
    const double insts = (double)iters * kChains;  // per wave
    const double total = per_wave_iter_ops * iters * waves;
    printf("{\"test\": \"%s\", \"waves_per_simd\": %d, \"ms\": %.4f, \"rate\": %.4g, \"rate_unit\": \"%s\", "
           "\"clk_per_inst_per_wave\": %.3f, \"simd_clk_per_inst\": %.3f, \"ops_per_inst\": %.0f}\n",
           name, waves_per_simd, ms, total / (ms * 1e-3), unit_what, clk / insts, clk / insts / waves_per_simd,
           ops_per_inst);
    fflush(stdout);
}

void test_mfma() {
    for (int w : {1, 2, 4})
        run_rate("mfma_16x16x32_bf16", "FLOP/s", 16384.0 * kChains, w, 4096, k_mfma, 16384);
}
void test_exp() {
    for (int w : {1, 2, 4}) run_rate("v_exp_f32", "exp/s", 64.0 * kChains, w, 4096, k_exp, 64);
}
void test_fma() {
    for (int w : {1, 2, 4}) {
        const int threads = 256 * w, blocks = g_cus, iters = 4096;
        const double ms = timed([&] {
            hipLaunchKernelGGL(k_fma, dim3(blocks), dim3(threads), 0, 0, g_out, iters, g_clk, 0.999f, 0.001f);
        });
        const int waves = blocks * threads / 64;
        const double clk = mean_clk(waves), insts = (double)iters * kChains;
        printf("{\"test\": \"v_fma_f32\", \"waves_per_simd\": %d, \"ms\": %.4f, \"rate\": %.4g, \"rate_unit\": "
               "\"FLOP/s\", \"clk_per_inst_per_wave\": %.3f, \"simd_clk_per_inst\": %.3f}\n",
               w, ms, 128.0 * insts * waves / (ms * 1e-3), clk / insts, clk / insts / w);
        fflush(stdout);
    }
}
void test_cvt() {
    for (int w : {1, 2, 4}) run_rate("v_cvt_pk_bf16_f32", "cvt/s", 128.0 * kChains, w, 4096, k_cvt, 128);
}

template <int E, bool FMA = false>
void mix_one() {
    for (int w : {1, 2}) {
        const int threads = 256 * w, blocks = g_cus, iters = 8192;
        const double ms = timed([&] { hipLaunchKernelGGL((k_mix<E, FMA>), dim3(blocks), dim3(threads), 0, 0, g_out, iters, g_clk); });
        const int waves = blocks * threads / 64;
        const double clk = mean_clk(waves);
        printf("{\"test\": \"mfma_plus_%s\", \"vector_per_mfma\": %d, \"waves_per_simd\": %d, \"ms\": %.4f, "
               "\"clk_per_iter_per_wave\": %.3f, \"simd_clk_per_iter\": %.3f}\n",
               FMA ? "fma" : "exp", E, w, ms, clk / iters, clk / iters / w);
        fflush(stdout);
    }
}
void test_mix() {
    mix_one<0>();
    mix_one<1>();
    mix_one<2>();
    mix_one<4>();
    mix_one<1, true>();
    mix_one<2, true>();
    mix_one<4, true>();
    mix_one<8, true>();
}

template <int KIND>
void coissue_one(const char* kind) {
    // alone: MFMA waves only (vector loop of 0), vector waves only (MFMA loop of 0), then both
    const int blocks = g_cus, threads = 512;
    const int vec_iters = KIND == 0 ? 4096 : KIND == 1 ? 16384 : 2048;
    for (auto cfg : {std::pair<int, int>{4096, 0}, {0, vec_iters}, {4096, vec_iters}}) {
        const double ms = timed([&] {
            hipLaunchKernelGGL(k_coissue<KIND>, dim3(blocks), dim3(threads), 0, 0, g_out, cfg.first, cfg.second, g_clk);
        });
        const int waves = blocks * threads / 64;
        std::vector<long long> h(waves);
        CHECK(hipMemcpy(h.data(), g_clk, sizeof(long long) * waves, hipMemcpyDeviceToHost));
        double cm = 0, ce = 0;
        for (int i = 0; i < waves; ++i) ((i % 8) < 4 ? cm : ce) += (double)h[i];
        cm /= waves / 2, ce /= waves / 2;
        printf("{\"test\": \"coissue_%s\", \"mfma_per_wave\": %d, \"vector_iters_per_wave\": %d, \"ms\": %.4f, "
               "\"mfma_wave_clk\": %.0f, \"vector_wave_clk\": %.0f}\n",
               kind, cfg.first * kChains, cfg.second, ms, cm, ce);
        fflush(stdout);
    }
}
void test_coissue() {
    coissue_one<0>("exp");
    coissue_one<1>("fma");
    coissue_one<2>("softmax_mix");
}

void test_lds() {
    for (int w : {1, 2, 4}) {
        const int threads = 256 * w, blocks = g_cus, iters = 2048;
        const double ms = timed([&] { hipLaunchKernelGGL(k_lds, dim3(blocks), dim3(threads), 0, 0, g_out, iters, g_clk); });
        const int waves = blocks * threads / 64;
        const double clk = mean_clk(waves);
        const double bytes_per_cu = 1024.0 * 8 * iters * (threads / 64);
        printf("{\"test\": \"ds_read_b128\", \"waves_per_cu\": %d, \"ms\": %.4f, \"bytes_per_clk_per_cu\": %.1f, "
               "\"TB_per_s_total\": %.2f}\n",
               threads / 64, ms, bytes_per_cu / clk, bytes_per_cu * blocks / (ms * 1e-3) / 1e12);
        fflush(stdout);
    }
}

void test_dma() {
    const uint32_t bytes = 4u << 20;  // 4 MB: stays in each XCD's L2
    uint4* src;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMemset(src, 1, bytes));
    for (int w : {4, 8, 16}) {
        const int threads = 64 * w, blocks = g_cus, iters = 512;
        const double ms = timed([&] {
            hipLaunchKernelGGL(k_dma, dim3(blocks), dim3(threads), 0, 0, src, bytes, g_out, iters, g_clk);
        });
        const int waves = blocks * threads / 64;
        const double clk = mean_clk(waves);
        const double bytes_per_cu = 1024.0 * 8 * iters * w;
        printf("{\"test\": \"global_to_lds_from_L2\", \"waves_per_cu\": %d, \"ms\": %.4f, "
               "\"bytes_per_clk_per_cu\": %.1f, \"TB_per_s_total\": %.2f}\n",
               w, ms, bytes_per_cu / clk, bytes_per_cu * blocks / (ms * 1e-3) / 1e12);
        fflush(stdout);
    }
    CHECK(hipFree(src));
}

template <int MODE>
void dma_issue_one(const char* mode, const uint4* src, uint32_t bytes) {
    for (int w : {1, 4, 8, 16}) {
        const int threads = 64 * w, blocks = g_cus;
        timed([&] { hipLaunchKernelGGL(k_dma_issue<MODE>, dim3(blocks), dim3(threads), 0, 0, src, bytes, g_out, g_clk); });
        const double clk = mean_clk(blocks * w);
        printf("{\"test\": \"dma_issue\", \"mode\": \"%s\", \"waves_per_cu\": %d, "
               "\"shader_clk_per_8_requests\": %.0f}\n", mode, w, clk / 16);
        fflush(stdout);
    }
}
void test_dma_issue() {
    const uint32_t bytes = 4u << 20;
    uint4* src;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMemset(src, 1, bytes));
    dma_issue_one<0>("lds_new_m0", src, bytes);
    dma_issue_one<1>("lds_same_m0", src, bytes);
    dma_issue_one<2>("to_registers", src, bytes);
    CHECK(hipFree(src));
}

void test_hbm() {
    const size_t bytes = size_t(1) << 30;  // 1 GiB read + 1 GiB written
    uint4 *src, *dst;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMalloc(&dst, bytes));
    CHECK(hipMemset(src, 1, bytes));
    CHECK(hipMemset(dst, 0, bytes));
    const size_t n = bytes / 16;
    for (int per_cu : {4, 8}) {
        const double ms =
            timed([&] { hipLaunchKernelGGL(k_copy, dim3(g_cus * per_cu), dim3(256), 0, 0, src, dst, n); });
        printf("{\"test\": \"hbm_copy\", \"bytes_read\": %zu, \"bytes_written\": %zu, \"workgroups_per_cu\": %d, "
               "\"ms\": %.4f, \"TB_per_s\": %.3f}\n",
               bytes, bytes, per_cu, ms, 2.0 * bytes / (ms * 1e-3) / 1e12);
        fflush(stdout);
    }
    CHECK(hipFree(src));
    CHECK(hipFree(dst));
}

}  // namespace

int main(int argc, char** argv) {
    hipDeviceProp_t prop;
    CHECK(hipGetDeviceProperties(&prop, 0));
    g_cus = prop.multiProcessorCount;
    int clk_khz = 0;
    CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, 0));
    printf("{\"device\": \"%s\", \"gcn_arch\": \"%s\", \"cus\": %d, \"max_clock_mhz\": %d}\n", prop.name,
           prop.gcnArchName, g_cus, clk_khz / 1000);
    CHECK(hipMalloc(&g_out, sizeof(float) * kMaxThreads));
    CHECK(hipMalloc(&g_clk, sizeof(long long) * kMaxThreads / 64));
    std::vector<std::string> tests;
    for (int i = 1; i < argc; ++i) tests.push_back(argv[i]);
    if (tests.empty()) tests = {"mfma", "exp", "fma", "cvt", "mix", "coissue", "lds", "dma", "dmaissue", "hbm"};
    for (const auto& t : tests) {
        if (t == "mfma") test_mfma();
        else if (t == "exp") test_exp();
        else if (t == "fma") test_fma();
        else if (t == "cvt") test_cvt();
        else if (t == "mix") test_mix();
        else if (t == "coissue") test_coissue();
        else if (t == "lds") test_lds();
        else if (t == "dma") test_dma();
        else if (t == "hbm") test_hbm();
        else if (t == "dmaissue") test_dma_issue();
        else {
            fprintf(stderr, "unknown test %s\n", t.c_str());
            return 2;
        }
    }
    CHECK(hipFree(g_out));
    CHECK(hipFree(g_clk));
    return 0;
}
