// fp32 forward kernels.
//
// Compute, per query row, softmax(q.K^T / sqrt(D) + mask + pair) . V and the
// natural-log LSE (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
// hmyw.cn, sections 4, 5.2 and 5.4) with fp32 operands and fp32 arithmetic
// throughout.
//
// fwd_f32_mfma (D = 8, 16, 32, 64, any bias strides; D = 8 zero-padded to
// 16): both products on
// the matrix cores with v_mfma_f32_16x16x4f32, which multiplies fp32 values
// and accumulates in fp32.  The layout follows the 16-bit kernel: scores are
// formed transposed (S^T = K.Q^T, lane c + 16g holds query c and keys 4g ..
// 4g+3 of a 16-key tile), so the probabilities a lane computes are exactly
// the B operand the P.V product needs (its contraction slice r takes key 4g +
// r from lane group g), with no data exchange.  The contraction over d is
// split so that lane group g holds the contiguous d-range [gD/4, (g+1)D/4) of
// its row (slice s takes d = gD/4 + s), which makes every Q and K operand one
// run of 16-byte loads.  Q is scaled by 1/sqrt(D) in fp32 when loaded; the
// biases enter as the accumulator's starting value (each wave's pair rows
// straight from global memory into registers, one block ahead; the mask row
// through LDS), so S^T comes out of the matrix cores in natural-log units.
// The softmax is the exact online one per 64-key block (block maximum,
// rescale, exponentials in base 2), on the vector ALUs.  K and V blocks go
// global -> LDS with direct copies, one block ahead, double buffered, in a
// layout whose 16-byte chunks are XOR-swizzled by row so that the operand
// reads spread over the banks.  Infinite and NaN values follow IEEE
// arithmetic: a -inf bias gives its key zero weight, a row of all -inf gives
// out = 0 and lse = -inf, and NaN propagates.  Bias rows that do not start
// 16-byte aligned (STAGED) are read with unaligned 16-byte loads over the
// exact range, and the mask row passes through registers into LDS.
//
// fwd_f32_kernel (layouts whose offsets the matrix-core kernel cannot form in
// 32 bits): the vector ALUs.  One 64-lane wavefront per (b, n, h, block of 64
// queries); each lane owns one query and keeps q, the output accumulator and
// its running max / sum in registers.  Keys are visited in blocks of 64
// staged in LDS, and each key updates the lane's state with a one-pass
// (online) softmax.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "evo_attn_launch.h"
#include "gfx950_common.h"

namespace evo {
namespace {

using gfx::f32x4;
using gfx::Rsrc;
using gfx::make_rsrc;
using gfx::bload16;
using gfx::bload16_any;
using gfx::dma16_untracked;
using gfx::kOOB;
using gfx::kLog2e;

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

// ---------------------------------------------------------------------------
// Matrix-core fp32 kernel.
// ---------------------------------------------------------------------------
constexpr int kMWaves = 4;
constexpr int kMQTiles = 2;                  // 16-query tiles per wavefront
constexpr int kMWaveQ = 16 * kMQTiles;       // 32 queries per wavefront
constexpr int kMBlockQ = kMWaves * kMWaveQ;  // 128 queries per workgroup
constexpr int kMKB = 64;                     // keys per block
constexpr int kMKT = kMKB / 16;              // 16-key tiles per block

// LDS of one block.  K and V rows of D floats are stored as D/4 chunks of 16
// bytes; chunk j of row r sits at slot r * (D/4) + (j ^ msw<D>(r)).  The
// swizzle gives the 16 rows that one operand read touches distinct 16-byte
// bank groups (D = 32, 64) or at most two rows per group (D = 16).
template <int D>
__device__ __host__ constexpr int msw(int r) {
    return D == 16 ? ((r >> 1) & 3) : (r & 7);
}
template <int D>
struct MBuf {
    f32x4 k[kMKB * D / 4];
    f32x4 v[kMKB * D / 4];
    f32x4 mt[kMKB / 4];  // the mask of the block's keys
};

struct MParams {
    const float *q, *k, *v, *mask, *pair;
    float *out, *lse;
    int64_t N, L, H;
    gfx::FastDiv qblocks, nd, hd;
    int64_t total;
    Strides st;
    float scale;  // 1 / sqrt(D)
};

// D = 8 runs as D = 16 (KD): the 16-byte chunks of a row past D read as zero
// (an offset beyond the buffer range), which pads Q and K with zero dimensions
// and V with zero columns; the output rows past D are not stored.
template <int D, bool PAIR, bool MASK, bool STAGED>
__global__ __launch_bounds__(kMWaves * 64, 2) void fwd_f32_mfma(MParams p) {
    constexpr int KD = D < 16 ? 16 : D;  // the width the tiles are laid out for
    constexpr int kCPR = KD / 4;      // 16-byte chunks per row
    constexpr int kS = KD / 4;        // contraction slices of the score product (4 d-values each)
    constexpr int kDT = KD / 16;      // 16-wide d tiles of the output
    constexpr int kRPS = 256 / KD;    // K / V rows per 1 KB copy request
    constexpr int kSegs = kMKB / kRPS;  // copy requests per tensor and block
    static_assert(D == 8 || D == 16 || D == 32 || D == 64, "head dimensions 8, 16, 32, 64");
    static_assert(kSegs % kMWaves == 0, "copy requests per wave");
    __shared__ __attribute__((aligned(16))) MBuf<KD> sm[2];

    const uint32_t id = (uint32_t)gfx::logical_block(blockIdx.x, p.total);
    const uint32_t r1 = gfx::fdiv(id, p.qblocks), r2 = gfx::fdiv(r1, p.hd), r3 = gfx::fdiv(r2, p.nd);
    const int64_t qb = id - r1 * p.qblocks.d;
    const int64_t h = r1 - r2 * p.hd.d, n = r2 - r3 * p.nd.d, b = r3;
    const Strides& st = p.st;
    const int L = (int)p.L;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nblocks = (L + kMKB - 1) / kMKB;
    const int q0 = (int)qb * kMBlockQ + wave * kMWaveQ;  // first query of the wave

    const uint32_t rowq = (uint32_t)st.q[2] * 4, rowk = (uint32_t)st.k[2] * 4, rowv = (uint32_t)st.v[2] * 4;
    const Rsrc rq = make_rsrc(p.q + b * st.q[0] + n * st.q[1] + h * st.q[3], (uint32_t)(L - 1) * rowq + D * 4);
    const Rsrc rk = make_rsrc(p.k + b * st.k[0] + n * st.k[1] + h * st.k[3], (uint32_t)(L - 1) * rowk + D * 4);
    const Rsrc rv = make_rsrc(p.v + b * st.v[0] + n * st.v[1] + h * st.v[3], (uint32_t)(L - 1) * rowv + D * 4);
    // bias ranges: rows 16-byte aligned, up to the 16-byte boundary after the
    // last element (that granule lies in the page of the last element);
    // STAGED, exactly the elements, whose last chunk bload16_any then reads
    // element by element
    const uint32_t rowp = (uint32_t)st.pi * 4;
    const uint32_t pbytes = (uint32_t)(L - 1) * rowp + (uint32_t)L * 4u, mbytes = (uint32_t)L * 4u;
    const Rsrc rp = make_rsrc(PAIR ? p.pair + b * st.pb + h * st.ph : p.q,
                              PAIR ? (STAGED ? pbytes : (pbytes + 15u) & ~15u) : 0u);
    const Rsrc rm = make_rsrc(MASK ? p.mask + b * st.mb + n * st.mn : p.q,
                              MASK ? (STAGED ? mbytes : (mbytes + 15u) & ~15u) : 0u);

    // Q operands, scaled: lane (c + 16g) holds q[q0 + 16t + c][gD/4 + s] / sqrt(D)
    // for slice s; rows past L read as zero
    float qop[kMQTiles][kS];
    for (int t = 0; t < kMQTiles; ++t) {
        const uint32_t row = (uint32_t)(q0 + 16 * t + c);
        for (int j = 0; j < kS / 4; ++j) {
            const uint32_t d0 = (uint32_t)(kS * g + 4 * j);
            const uint4 w = bload16(rq, (D >= 16 || d0 < (uint32_t)D) ? row * rowq + 4u * d0 : kOOB);
            qop[t][4 * j + 0] = __builtin_bit_cast(float, w.x) * p.scale;
            qop[t][4 * j + 1] = __builtin_bit_cast(float, w.y) * p.scale;
            qop[t][4 * j + 2] = __builtin_bit_cast(float, w.z) * p.scale;
            qop[t][4 * j + 3] = __builtin_bit_cast(float, w.w) * p.scale;
        }
    }

    // ---- copies of one block: K and V rows into LDS (wave w takes requests
    // w, w + 4, ... of each tensor; lane l of request I holds row I*kRPS +
    // l / kCPR, slot position l % kCPR, i.e. chunk (l % kCPR) ^ msw(row)), the
    // mask row (wave 0, lanes 0..15) ----
    uint32_t kvo[kSegs / kMWaves][2];
    for (int i = 0; i < kSegs / kMWaves; ++i) {
        const int seg = wave + kMWaves * i;
        const int row = seg * kRPS + lane / kCPR;
        const uint32_t chunk = (uint32_t)((lane % kCPR) ^ msw<KD>(row));
        // chunks past D: kOOB, to which a block's k0 * row adds less than 2^31
        const bool din = KD == D || chunk < D / 4;
        kvo[i][0] = din ? (uint32_t)row * rowk + 16u * chunk : kOOB;
        kvo[i][1] = din ? (uint32_t)row * rowv + 16u * chunk : kOOB;
    }
    uint4 mstage;  // STAGED: the mask chunk between its load and its landing in LDS
    auto copy_block = [&](int blk, MBuf<KD>* __restrict__ dst) {
        const uint32_t k0 = (uint32_t)blk * kMKB;
        for (int i = 0; i < kSegs / kMWaves; ++i) {
            const int seg = wave + kMWaves * i;
            dma16_untracked(rk, &dst->k[64 * seg], kvo[i][0] + k0 * rowk);
            dma16_untracked(rv, &dst->v[64 * seg], kvo[i][1] + k0 * rowv);
        }
        if (MASK && wave == 0 && lane < 16) {
            if (STAGED) mstage = bload16_any(rm, 16u * lane + k0 * 4u, mbytes);
            else dma16_untracked(rm, &dst->mt[0], 16u * lane + k0 * 4u);
        }
    };
    auto land_mask = [&](MBuf<KD>* __restrict__ dst) {
        if (STAGED && MASK && wave == 0 && lane < 16) dst->mt[lane] = __builtin_bit_cast(f32x4, mstage);
    };
    // ---- the wave's pair rows for one block, straight into registers in the
    // score layout: tile t, key tile kt -> pair[q0 + 16t + c][k0 + 16kt + 4g .. +3] ----
    f32x4 pr[kMQTiles][kMKT];
    auto load_pair = [&](int blk) {
        const uint32_t k0 = (uint32_t)blk * kMKB;
        for (int t = 0; t < kMQTiles; ++t) {
            // query rows past L: their results are never stored; rows past the
            // matrix read as zero
            const uint32_t row = (uint32_t)(q0 + 16 * t + c);
            for (int kt = 0; kt < kMKT; ++kt) {
                const uint32_t off = row * rowp + 4u * (k0 + 16 * kt + 4 * g);
                pr[t][kt] = __builtin_bit_cast(f32x4, STAGED ? bload16_any(rp, off, pbytes) : bload16(rp, off));
            }
        }
    };

    f32x4 oacc[kMQTiles][kDT];
    float mrun[kMQTiles], lrun[kMQTiles];
    for (int t = 0; t < kMQTiles; ++t) {
        for (int dt = 0; dt < kDT; ++dt) oacc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        mrun[t] = -INFINITY;
        lrun[t] = 0.f;  // this lane's part of the row sum (its 4 keys of every tile)
    }

    copy_block(0, &sm[0]);
    land_mask(&sm[0]);
    if (PAIR) load_pair(0);
    gfx::wait_all();
    __syncthreads();

    for (int it = 0; it < nblocks; ++it) {
        const MBuf<KD>* __restrict__ cur = &sm[it & 1];
        const int k0 = it * kMKB;
        // the next block's K, V and mask: their buffer was last read before the
        // barrier that ended the previous step; the copies are untracked, so
        // this block's LDS reads below do not wait for them
        if (it + 1 < nblocks) copy_block(it + 1, &sm[(it & 1) ^ 1]);
        // ---- S^T = K.Q^T/sqrt(D) + pair + mask, tile by tile ----
        f32x4 acc[kMQTiles][kMKT];
        for (int kt = 0; kt < kMKT; ++kt) {
            f32x4 mk = f32x4{0.f, 0.f, 0.f, 0.f};
            if (MASK) mk = cur->mt[4 * kt + g];
            for (int t = 0; t < kMQTiles; ++t) acc[t][kt] = PAIR ? (MASK ? pr[t][kt] + mk : pr[t][kt]) : mk;
        }
        if (PAIR && it + 1 < nblocks) load_pair(it + 1);  // the registers just consumed take the next block's rows
        for (int kt = 0; kt < kMKT; ++kt) {
            // A[m = key][k]: lane (c + 16g) takes key 16kt + c, d = gD/4 + s
            const int row = 16 * kt + c;
            float kf[kS];
            for (int j = 0; j < kS / 4; ++j) {
                const f32x4 w = cur->k[row * kCPR + ((kS / 4 * g + j) ^ msw<KD>(row))];
                kf[4 * j + 0] = w[0], kf[4 * j + 1] = w[1], kf[4 * j + 2] = w[2], kf[4 * j + 3] = w[3];
            }
            for (int s2 = 0; s2 < kS; ++s2)
                for (int t = 0; t < kMQTiles; ++t)
                    acc[t][kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[s2], qop[t][s2], acc[t][kt], 0, 0, 0);
        }
        // ---- online softmax, exact per block ----
        for (int t = 0; t < kMQTiles; ++t) {
            if (k0 + kMKB > L)  // keys past L take no weight
                for (int kt = 0; kt < kMKT; ++kt)
                    for (int r = 0; r < 4; ++r)
                        if (k0 + 16 * kt + 4 * g + r >= L) acc[t][kt][r] = -INFINITY;
            float bm = acc[t][0][0];
            for (int kt = 0; kt < kMKT; ++kt)
                for (int r = 0; r < 4; ++r) bm = fmaxf(bm, acc[t][kt][r]);
            const float mnew = fmaxf(mrun[t], gfx::max_over_groups(bm));
            const float ms = mnew == -INFINITY ? 0.f : mnew;  // every key so far -inf: weights stay 0
            const float alpha = __builtin_amdgcn_exp2f((mrun[t] - ms) * kLog2e);  // 0 when mrun = -inf
            mrun[t] = mnew;
            const float msl = ms * kLog2e;
            float ls = 0.f;
            for (int kt = 0; kt < kMKT; ++kt)
                for (int r = 0; r < 4; ++r) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(acc[t][kt][r], kLog2e, -msl));
                    acc[t][kt][r] = e;
                    ls += e;
                }
            lrun[t] = fmaf(lrun[t], alpha, ls);
            for (int dt = 0; dt < kDT; ++dt) oacc[t][dt] *= alpha;
        }
        // ---- O^T += V^T . P^T: slice r of key tile kt takes key 16kt + 4g + r
        // from lane group g, which is element r of the lane's probabilities;
        // the V operand A[m = d][k = r]: lane (c + 16g) takes V[key 16kt + 4g + r][16dt + c] ----
        for (int kt = 0; kt < kMKT; ++kt)
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * kt + 4 * g + r;
                const float* vrow = reinterpret_cast<const float*>(&cur->v[row * kCPR]);
                for (int dt = 0; dt < kDT; ++dt) {
                    const int d = 16 * dt + c;
                    const float vf = vrow[4 * ((d >> 2) ^ msw<KD>(row)) + (d & 3)];
                    for (int t = 0; t < kMQTiles; ++t)
                        oacc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, acc[t][kt][r], oacc[t][dt], 0, 0, 0);
                }
            }
        if (it + 1 < nblocks) land_mask(&sm[(it & 1) ^ 1]);
        gfx::wait_all();  // the next block's copies and pair rows have landed
        __syncthreads();
    }

    // ---- epilogue: lane (c + 16g) holds O^T[d = 16dt + 4g + i][query c] ----
    for (int t = 0; t < kMQTiles; ++t) {
        const float l = gfx::sum_over_groups(lrun[t]);
        const int i = q0 + 16 * t + c;
        if (i >= L) continue;
        // a row sum of 0 (every key -inf) gives out = 0; a NaN one stays NaN
        const float inv = l > 0.f ? 1.f / l : (l == 0.f ? 0.f : l);
        for (int dt = 0; dt < kDT; ++dt) {
            if (D < 16 && 16 * dt + 4 * g >= D) continue;  // the padded output rows
            const f32x4 o = oacc[t][dt] * inv;
            *reinterpret_cast<f32x4*>(p.out + b * st.o[0] + n * st.o[1] + h * st.o[3] + (int64_t)i * st.o[2] +
                                      16 * dt + 4 * g) = o;
        }
        if (p.lse && g == 0)
            p.lse[((b * p.N + n) * p.H + h) * st.lrow + i] =
                l > 0.f ? mrun[t] + logf(l) : (l == 0.f ? -INFINITY : l);
    }
}

template <int D, bool PAIR, bool MASK>
hipError_t launch_mfma_variant(MParams& p, hipStream_t stream) {
    void* args[] = {&p};
    // bias rows that do not all start 16-byte aligned are staged
    const Strides& s = p.st;
    const bool staged = (PAIR && (s.pb % 4 || s.ph % 4 || s.pi % 4)) || (MASK && (s.mb % 4 || s.mn % 4));
    const void* k = staged ? reinterpret_cast<const void*>(&fwd_f32_mfma<D, PAIR, MASK, true>)
                           : reinterpret_cast<const void*>(&fwd_f32_mfma<D, PAIR, MASK, false>);
    return hipLaunchKernel(k, dim3((unsigned)p.total), dim3(kMWaves * 64), args, 0, stream);
}

template <int D>
hipError_t launch_mfma_dim(MParams& p, hipStream_t stream) {
    const bool pair = p.pair != nullptr, mask = p.mask != nullptr;
    if (pair && mask) return launch_mfma_variant<D, true, true>(p, stream);
    if (pair) return launch_mfma_variant<D, true, false>(p, stream);
    if (mask) return launch_mfma_variant<D, false, true>(p, stream);
    return launch_mfma_variant<D, false, false>(p, stream);
}

// Whether the matrix-core kernel takes these arguments: D in {8, 16, 32, 64}
// and every byte offset it forms (rows of one slice or pair matrix, up to 128
// rows past L) below 2^31.
bool mfma_eligible(const FwdArgs& a) {
    if (a.D != 8 && a.D != 16 && a.D != 32 && a.D != 64) return false;
    constexpr int64_t kLim = int64_t(1) << 31;
    for (int64_t rs : {a.st.q[2], a.st.k[2], a.st.v[2]})
        if ((a.L + kMBlockQ) * rs * 4 + a.D * 4 >= kLim) return false;
    if (a.pair && ((a.L + kMBlockQ) * a.st.pi + a.L + kMKB) * 4 >= kLim) return false;
    if (a.mask && (a.L + kMKB) * 4 >= kLim) return false;
    const int64_t total = a.B * a.N * a.H * ((a.L + kMBlockQ - 1) / kMBlockQ);
    return total < kLim;
}

hipError_t launch_mfma(const FwdArgs& a, hipStream_t stream) {
    MParams p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.mask = static_cast<const float*>(a.mask);
    p.pair = static_cast<const float*>(a.pair);
    p.out = static_cast<float*>(a.out);
    p.lse = a.lse;
    p.N = a.N, p.L = a.L, p.H = a.H;
    const int64_t qblocks = (a.L + kMBlockQ - 1) / kMBlockQ;
    p.total = a.B * a.N * a.H * qblocks;
    p.qblocks = gfx::make_fastdiv((uint32_t)qblocks);
    p.nd = gfx::make_fastdiv((uint32_t)a.N);
    p.hd = gfx::make_fastdiv((uint32_t)a.H);
    p.st = a.st;
    p.scale = (float)(1.0 / std::sqrt((double)a.D));
    if (a.D == 8) return launch_mfma_dim<8>(p, stream);
    if (a.D == 16) return launch_mfma_dim<16>(p, stream);
    if (a.D == 32) return launch_mfma_dim<32>(p, stream);
    return launch_mfma_dim<64>(p, stream);
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
    if (mfma_eligible(a)) return launch_mfma(a, stream);
    switch (a.D) {
    case 8: return launch<8>(a, stream);
    case 16: return launch<16>(a, stream);
    case 32: return launch<32>(a, stream);
    case 64: return launch<64>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace evo
