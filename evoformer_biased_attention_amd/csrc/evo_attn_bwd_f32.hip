// Backward pass for fp32 inputs on the matrix cores: the dq (+ delta), the
// dk / dv / dmask and the pair-gradient stages with v_mfma_f32_16x16x4f32
// (fp32 operands, fp32 accumulation).
//
// The gradients (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
// hmyw.cn, sections 4 and 5.4: the weights are recomputed from the saved
// log-sum-exp, and delta_i = dO_i . out_i), with P_ij = exp(s_ij - lse_i):
//   dS_ij = P_ij (dO_i . v_j - delta_i)
//   dq_i = sum_j dS_ij k_j / sqrt(D),  dk_j = sum_i dS_ij q_i / sqrt(D),
//   dv_j = sum_i P_ij dO_i,  dmask[b,n,j] = sum over h, i of dS.
//
// A 16x16x4 MFMA leaves column n of its result in lanes n, n+16, n+32, n+48,
// rows 4g .. 4g+3 in lane group g, and takes contraction index g of its
// operands from lane group g.  A product whose result rows are the next
// product's contraction index therefore chains without data exchange: slice
// r of a 16-row tile takes row 4g + r from lane group g, which is element r
// of that lane's result.  The products whose contraction runs over d split it
// so that lane group g holds the contiguous range [gD/4, (g+1)D/4) of its row
// (slice s takes d = gD/4 + s), which makes those operands runs of 16-byte
// reads.
//   bwd_dq_f32_mfma    scores transposed (S^T = K.Q^T: keys are result rows),
//                      so dQ^T = K^T . dS^T contracts over them.  Also delta.
//   bwd_dkdv_f32_mfma  scores upright (S = Q.K^T: queries are result rows),
//                      so dV^T = dO^T . P and dK^T = Q^T . dS contract over
//                      them; the workgroup visits every head, so the mask
//                      gradient of its keys is complete when it ends.
//   bwd_dpair_f32_mfma scores transposed; the workgroup owns a 64 x 64 tile of
//                      one (b, h) and sums dS over a range of n; with more
//                      than one range, bwd_dpair_reduce_f32 adds the ranges.
// LDS tiles of rows of D floats keep 16-byte chunks XOR-swizzled by row (as in
// the fp32 forward), so that a 16-row operand read and a 4-row transposed read
// spread over the banks.  Copies into LDS are untracked (see
// dma16_untracked) and waited for explicitly before each barrier.  Buffer
// resources return zeros past their range: rows past L read as zero.  Bias
// rows that do not start 16-byte aligned (STAGED) are read with unaligned
// 16-byte loads over their exact range, the mask row passing through
// registers into LDS, and the pair gradient is written element by element.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "evo_attn_launch.h"
#include "gfx950_common.h"

namespace evo {
namespace {

using gfx::bload16;
using gfx::bload16_any;
using gfx::dma16_untracked;
using gfx::f32x4;
using gfx::kLog2e;
using gfx::kOOB;
using gfx::make_rsrc;
using gfx::Rsrc;

constexpr int kWaves = 4;
constexpr int kKB = 64;         // keys (dq) or queries (dk/dv) per LDS block
constexpr int kKT = kKB / 16;   // 16-row tiles per block

// chunk j of row r of an LDS tile of D-float rows sits at slot r*(D/4) + (j ^ sw<D>(r))
template <int D>
__device__ constexpr int sw(int r) {
    return D == 16 ? ((r >> 1) & 3) : (r & 7);
}
// one float of an LDS tile: row r, column d
template <int D>
__device__ inline float tile_at(const f32x4* t, int r, int d) {
    return reinterpret_cast<const float*>(t)[4 * (r * (D / 4) + ((d >> 2) ^ sw<D>(r))) + (d & 3)];
}
// the kS = D/4 floats of lane group g's d-range of row r
template <int D>
__device__ inline void tile_run(const f32x4* t, int r, int g, float (&out)[D / 4]) {
    for (int j = 0; j < D / 16; ++j) {
        const f32x4 w = t[r * (D / 4) + ((D / 16 * g + j) ^ sw<D>(r))];
        out[4 * j] = w[0], out[4 * j + 1] = w[1], out[4 * j + 2] = w[2], out[4 * j + 3] = w[3];
    }
}

struct BParams {
    const float *q, *k, *v, *mask, *pair, *out, *dout, *lse;
    float *dq, *dk, *dv, *dmask, *dpair, *delta;
    int64_t N, L, H;
    gfx::FastDiv rblocks, nd, hd;  // row blocks (dq_rows<D>() queries for dq, 64 keys for dk/dv), N, H
    int64_t total;
    Strides st;
    float scale;  // 1 / sqrt(D)
};

// lse * log2(e); +inf for a row without softmax (lse = -inf) or past L, so
// that every weight of the row is exactly zero
__device__ inline float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Copy requests of one block of 64 rows of a [L][row] fp32 tensor into an LDS
// tile of KD-float rows: lane l of request I holds row I*(256/KD) + l/(KD/4),
// slot position l % (KD/4), i.e. chunk (l % (KD/4)) ^ sw(row); wave w takes
// requests w, w + 4, ...  Chunks past the D floats of a row (D = 8 in a tile
// laid out for 16) read from kOOB and land as zeros; a block's base offset
// (below 2^31) keeps them past the range.
template <int KD, int D = KD>
struct RowCopy {
    static constexpr int kRPS = 256 / KD;      // rows per 1 KB request
    static constexpr int kSegs = kKB / kRPS;   // requests per block
    static constexpr int kPer = kSegs / kWaves;
    static_assert(kSegs % kWaves == 0, "requests per wave");
    uint32_t off[kPer];
    __device__ void init(int wave, int lane, uint32_t rowbytes) {
        for (int i = 0; i < kPer; ++i) {
            const int seg = wave + kWaves * i, row = seg * kRPS + lane / (KD / 4);
            const uint32_t chunk = (uint32_t)((lane % (KD / 4)) ^ sw<KD>(row));
            off[i] = (KD == D || chunk < D / 4) ? (uint32_t)row * rowbytes + 16u * chunk : kOOB;
        }
    }
    __device__ void issue(Rsrc r, f32x4* dst, int wave, uint32_t base) const {
        for (int i = 0; i < kPer; ++i) dma16_untracked(r, &dst[64 * (wave + kWaves * i)], off[i] + base);
    }
};

// ---------------------------------------------------------------------------
// The three kernels run D = 8 as D = 16 (KD, the width the tiles are laid out
// for): the 16-byte chunks of a row past D read as zero (an offset beyond the
// buffer range), which pads Q, K, V and dO with zero columns, adds nothing to
// the scores, dP and delta, and leaves the gradient rows past D unstored.
//
// dq and delta.  Workgroup = 128 queries of one (b, n, h); wave w owns
// queries 32w .. 32w+31 as two 16-query tiles; key blocks of 64 in LDS.  At
// D = 64 a wave owns one 16-query tile (64 queries per workgroup), which
// keeps its registers within two waves per SIMD.
// ---------------------------------------------------------------------------
template <int D>
constexpr int tile_width() { return D < 16 ? 16 : D; }
template <int D>
constexpr int dq_tiles() { return D == 64 ? 1 : 2; }
template <int D>
constexpr int dq_rows() { return kWaves * 16 * dq_tiles<D>(); }

template <int D>
struct DqBuf {
    f32x4 k[kKB * D / 4];
    f32x4 v[kKB * D / 4];
    f32x4 mt[kKB / 4];
};

template <int D, bool PAIR, bool MASK, bool STAGED>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_dq_f32_mfma(BParams p) {
    constexpr int KD = tile_width<D>();
    constexpr int kS = KD / 4, kDT = KD / 16, kQT = dq_tiles<D>();
    __shared__ __attribute__((aligned(16))) DqBuf<KD> sm[2];

    const uint32_t id = (uint32_t)gfx::logical_block(blockIdx.x, p.total);
    const uint32_t r1 = gfx::fdiv(id, p.rblocks), r2 = gfx::fdiv(r1, p.hd), r3 = gfx::fdiv(r2, p.nd);
    const int64_t qb = id - r1 * p.rblocks.d;
    const int64_t h = r1 - r2 * p.hd.d, n = r2 - r3 * p.nd.d, b = r3;
    const Strides& st = p.st;
    const int L = (int)p.L;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nblocks = (L + kKB - 1) / kKB;
    const int q0 = (int)qb * dq_rows<D>() + wave * 16 * kQT;

    const uint32_t rowq = (uint32_t)st.q[2] * 4, rowk = (uint32_t)st.k[2] * 4, rowv = (uint32_t)st.v[2] * 4;
    const uint32_t rowo = (uint32_t)st.o[2] * 4, rowp = (uint32_t)st.pi * 4;
    const int64_t os = b * st.o[0] + n * st.o[1] + h * st.o[3];
    const Rsrc rq = make_rsrc(p.q + b * st.q[0] + n * st.q[1] + h * st.q[3], (uint32_t)(L - 1) * rowq + D * 4);
    const Rsrc rk = make_rsrc(p.k + b * st.k[0] + n * st.k[1] + h * st.k[3], (uint32_t)(L - 1) * rowk + D * 4);
    const Rsrc rv = make_rsrc(p.v + b * st.v[0] + n * st.v[1] + h * st.v[3], (uint32_t)(L - 1) * rowv + D * 4);
    const Rsrc ro = make_rsrc(p.out + os, (uint32_t)(L - 1) * rowo + D * 4);
    const Rsrc rdo = make_rsrc(p.dout + os, (uint32_t)(L - 1) * rowo + D * 4);
    const uint32_t pbytes = (uint32_t)(L - 1) * rowp + (uint32_t)L * 4u, mbytes = (uint32_t)L * 4u;
    const Rsrc rp = make_rsrc(PAIR ? p.pair + b * st.pb + h * st.ph : p.q,
                              PAIR ? (STAGED ? pbytes : (pbytes + 15u) & ~15u) : 0u);
    const Rsrc rm = make_rsrc(MASK ? p.mask + b * st.mb + n * st.mn : p.q,
                              MASK ? (STAGED ? mbytes : (mbytes + 15u) & ~15u) : 0u);
    const int64_t lrow = ((b * p.N + n) * p.H + h) * st.lrow;

    // per query: Q/sqrt(D) and dO (B operands, lane group g's d-range), delta, lse
    float qop[kQT][kS], dop[kQT][kS], lse2[kQT], ndelta[kQT];
    for (int t = 0; t < kQT; ++t) {
        const int i = q0 + 16 * t + c;
        const uint32_t rq_off = (uint32_t)i * rowq, ro_off = (uint32_t)i * rowo;
        float part = 0.f;
        for (int j = 0; j < kS / 4; ++j) {
            const uint32_t e0 = (uint32_t)(kS * g + 4 * j), d0 = 4u * e0;
            const bool din = D >= 16 || e0 < (uint32_t)D;
            const uint4 wq = bload16(rq, din ? rq_off + d0 : kOOB), wd = bload16(rdo, din ? ro_off + d0 : kOOB);
            const uint4 wo = bload16(ro, din ? ro_off + d0 : kOOB);
            const float qv[4] = {__builtin_bit_cast(float, wq.x), __builtin_bit_cast(float, wq.y),
                                 __builtin_bit_cast(float, wq.z), __builtin_bit_cast(float, wq.w)};
            const float dv4[4] = {__builtin_bit_cast(float, wd.x), __builtin_bit_cast(float, wd.y),
                                  __builtin_bit_cast(float, wd.z), __builtin_bit_cast(float, wd.w)};
            const float ov[4] = {__builtin_bit_cast(float, wo.x), __builtin_bit_cast(float, wo.y),
                                 __builtin_bit_cast(float, wo.z), __builtin_bit_cast(float, wo.w)};
            for (int e = 0; e < 4; ++e) {
                qop[t][4 * j + e] = qv[e] * p.scale;
                dop[t][4 * j + e] = dv4[e];
                part = fmaf(dv4[e], ov[e], part);
            }
        }
        const float delta = gfx::sum_over_groups(part);
        ndelta[t] = -delta;
        lse2[t] = i < L ? lse2_of(p.lse[lrow + i]) : INFINITY;
        if (g == 0 && i < L) p.delta[lrow + i] = delta;
    }

    RowCopy<KD, D> ck, cv;
    ck.init(wave, lane, rowk);
    cv.init(wave, lane, rowv);
    uint4 mstage;  // STAGED: the mask chunk between its load and its landing in LDS
    auto copy_block = [&](int blk, DqBuf<KD>* __restrict__ dst) {
        const uint32_t k0 = (uint32_t)blk * kKB;
        ck.issue(rk, dst->k, wave, k0 * rowk);
        cv.issue(rv, dst->v, wave, k0 * rowv);
        if (MASK && wave == 0 && lane < 16) {
            if (STAGED) mstage = bload16_any(rm, 16u * lane + k0 * 4u, mbytes);
            else dma16_untracked(rm, &dst->mt[0], 16u * lane + k0 * 4u);
        }
    };
    auto land_mask = [&](DqBuf<KD>* __restrict__ dst) {
        if (STAGED && MASK && wave == 0 && lane < 16) dst->mt[lane] = __builtin_bit_cast(f32x4, mstage);
    };
    // the wave's pair rows in the score layout: tile t, key tile kt -> pair[q0 + 16t + c][k0 + 16kt + 4g .. +3]
    f32x4 pr[kQT][kKT];
    auto load_pair = [&](int blk) {
        const uint32_t k0 = (uint32_t)blk * kKB;
        for (int t = 0; t < kQT; ++t)
            for (int kt = 0; kt < kKT; ++kt)
            {
                const uint32_t off = (uint32_t)(q0 + 16 * t + c) * rowp + 4u * (k0 + 16 * kt + 4 * g);
                pr[t][kt] = __builtin_bit_cast(f32x4, STAGED ? bload16_any(rp, off, pbytes) : bload16(rp, off));
            }
    };

    f32x4 dqacc[kQT][kDT];
    for (int t = 0; t < kQT; ++t)
        for (int dt = 0; dt < kDT; ++dt) dqacc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    copy_block(0, &sm[0]);
    land_mask(&sm[0]);
    if (PAIR) load_pair(0);
    gfx::wait_all();
    __syncthreads();

    for (int it = 0; it < nblocks; ++it) {
        const DqBuf<KD>* __restrict__ cur = &sm[it & 1];
        const int k0 = it * kKB;
        if (it + 1 < nblocks) copy_block(it + 1, &sm[(it & 1) ^ 1]);
        // S^T (keys 16kt + 4g + i, query c) from pair + mask, then K.Q^T/sqrt(D)
        f32x4 acc[kQT][kKT], dpm[kQT][kKT];
        for (int kt = 0; kt < kKT; ++kt) {
            f32x4 mk = f32x4{0.f, 0.f, 0.f, 0.f};
            if (MASK) mk = cur->mt[4 * kt + g];
            for (int t = 0; t < kQT; ++t) {
                acc[t][kt] = PAIR ? (MASK ? pr[t][kt] + mk : pr[t][kt]) : mk;
                dpm[t][kt] = f32x4{ndelta[t], ndelta[t], ndelta[t], ndelta[t]};
            }
        }
        if (PAIR && it + 1 < nblocks) load_pair(it + 1);
        for (int kt = 0; kt < kKT; ++kt) {
            float kf[kS], vf[kS];
            tile_run<KD>(cur->k, 16 * kt + c, g, kf);
            tile_run<KD>(cur->v, 16 * kt + c, g, vf);
            for (int s = 0; s < kS; ++s)
                for (int t = 0; t < kQT; ++t) {
                    acc[t][kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[s], qop[t][s], acc[t][kt], 0, 0, 0);
                    // dP^T - delta = V.dO^T - delta
                    dpm[t][kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[s], dop[t][s], dpm[t][kt], 0, 0, 0);
                }
        }
        // dS^T = P^T (dP^T - delta), in place of the scores
        for (int t = 0; t < kQT; ++t)
            for (int kt = 0; kt < kKT; ++kt)
                for (int r = 0; r < 4; ++r) {
                    const bool live = k0 + 16 * kt + 4 * g + r < L;
                    const float w = __builtin_amdgcn_exp2f(fmaf(acc[t][kt][r], kLog2e, -lse2[t]));
                    acc[t][kt][r] = live ? w * dpm[t][kt][r] : 0.f;
                }
        // dQ^T += K^T . dS^T: slice r of key tile kt takes key 16kt + 4g + r from
        // lane group g; the K operand A[m = d][k]: lane (c + 16g) takes K[16kt + 4g + r][16dt + c]
        for (int kt = 0; kt < kKT; ++kt)
            for (int r = 0; r < 4; ++r)
                for (int dt = 0; dt < kDT; ++dt) {
                    const float kv = tile_at<KD>(cur->k, 16 * kt + 4 * g + r, 16 * dt + c);
                    for (int t = 0; t < kQT; ++t)
                        dqacc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv, acc[t][kt][r], dqacc[t][dt], 0, 0, 0);
                }
        if (it + 1 < nblocks) land_mask(&sm[(it & 1) ^ 1]);
        gfx::wait_all();  // the next block's copies and pair rows have landed
        __syncthreads();
    }

    // lane (c + 16g) holds dQ^T[d = 16dt + 4g + i][query c]
    const int64_t qs = b * st.q[0] + n * st.q[1] + h * st.q[3];
    for (int t = 0; t < kQT; ++t) {
        const int i = q0 + 16 * t + c;
        if (i >= L) continue;
        for (int dt = 0; dt < kDT; ++dt)
            if (D >= 16 || 16 * dt + 4 * g < D)
                *reinterpret_cast<f32x4*>(p.dq + qs + (int64_t)i * st.q[2] + 16 * dt + 4 * g) = dqacc[t][dt] * p.scale;
    }
}

// ---------------------------------------------------------------------------
// dk, dv (every head) and dmask.  Workgroup = 64 keys of one (b, n); wave w
// owns keys 16w .. 16w+15 (one tile) and visits every head in order, taking
// the queries in blocks of 64 (four 16-query tiles) from LDS.  Scores
// upright: lane (c + 16g) holds S[query 16qt + 4g + i][key c].
// ---------------------------------------------------------------------------
template <int D>
struct KvBuf {
    f32x4 q[kKB * D / 4];
    f32x4 dout[kKB * D / 4];
    f32x4 ls[kKB / 4];  // lse * log2(e) of the block's queries (+inf past L or without softmax)
    f32x4 dl[kKB / 4];  // -delta of the block's queries
};

template <int D, bool PAIR, bool MASK>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_dkdv_f32_mfma(BParams p) {
    constexpr int KD = tile_width<D>();
    constexpr int kS = KD / 4, kDT = KD / 16;
    __shared__ __attribute__((aligned(16))) KvBuf<KD> sm[2];

    const uint32_t id = (uint32_t)gfx::logical_block(blockIdx.x, p.total);
    const uint32_t r1 = gfx::fdiv(id, p.rblocks), r2 = gfx::fdiv(r1, p.nd);
    const int64_t kb = id - r1 * p.rblocks.d;
    const int64_t n = r1 - r2 * p.nd.d, b = r2;
    const Strides& st = p.st;
    const int L = (int)p.L, H = (int)p.H;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nqb = (L + kKB - 1) / kKB;  // query blocks per head
    const int nsteps = H * nqb;
    const int key = (int)kb * kKB + 16 * wave + c;  // this lane's key
    const bool key_live = key < L;

    // rows of every head: buffers cover the (b, n) slice, offsets within 32 bits (the launcher checks)
    const uint32_t rowq = (uint32_t)st.q[2] * 4, rowk = (uint32_t)st.k[2] * 4, rowv = (uint32_t)st.v[2] * 4;
    const uint32_t rowo = (uint32_t)st.o[2] * 4;
    const uint32_t hq = (uint32_t)st.q[3] * 4, hk = (uint32_t)st.k[3] * 4, hv = (uint32_t)st.v[3] * 4;
    const uint32_t ho = (uint32_t)st.o[3] * 4;
    const uint32_t last = (uint32_t)(L - 1), lasth = (uint32_t)(H - 1);
    const int64_t qbn = b * st.q[0] + n * st.q[1], kbn = b * st.k[0] + n * st.k[1];
    const int64_t vbn = b * st.v[0] + n * st.v[1], obn = b * st.o[0] + n * st.o[1];
    const Rsrc rq = make_rsrc(p.q + qbn, last * rowq + lasth * hq + D * 4);
    const Rsrc rk = make_rsrc(p.k + kbn, last * rowk + lasth * hk + D * 4);
    const Rsrc rv = make_rsrc(p.v + vbn, last * rowv + lasth * hv + D * 4);
    const Rsrc rdo = make_rsrc(p.dout + obn, last * rowo + lasth * ho + D * 4);
    const float mkey = MASK && key_live ? p.mask[b * st.mb + n * st.mn + key] : 0.f;

    RowCopy<KD, D> cq, cdo;
    cq.init(wave, lane, rowq);
    cdo.init(wave, lane, rowo);
    float lsv = INFINITY, dlv = 0.f;  // wave 0: this lane's query of the step being copied
    auto copy_step = [&](int it, KvBuf<KD>* __restrict__ dst) {
        const int hh = it / nqb, q0 = (it - hh * nqb) * kKB;
        cq.issue(rq, dst->q, wave, (uint32_t)q0 * rowq + (uint32_t)hh * hq);
        cdo.issue(rdo, dst->dout, wave, (uint32_t)q0 * rowo + (uint32_t)hh * ho);
        if (wave == 0) {
            const int i = q0 + lane;
            const int64_t row = ((b * p.N + n) * p.H + hh) * st.lrow + i;
            lsv = i < L ? lse2_of(p.lse[row]) : INFINITY;
            dlv = i < L ? -p.delta[row] : 0.f;
        }
    };
    auto put_rows = [&](KvBuf<KD>* __restrict__ dst) {
        if (wave == 0) {
            reinterpret_cast<float*>(dst->ls)[lane] = lsv;
            reinterpret_cast<float*>(dst->dl)[lane] = dlv;
        }
    };
    // the pair bias of this lane's key for the step's queries, in the score
    // layout: query tile qt -> pair[h][q0 + 16qt + 4g + i][key], i = 0..3
    f32x4 pr[kKT];
    auto load_pair = [&](int it) {
        const int hh = it / nqb, q0 = (it - hh * nqb) * kKB;
        const float* pm = p.pair + b * st.pb + hh * st.ph;
        for (int qt = 0; qt < kKT; ++qt)
            for (int i = 0; i < 4; ++i) {
                const int qi = q0 + 16 * qt + 4 * g + i;
                pr[qt][i] = (qi < L && key_live) ? pm[(int64_t)qi * st.pi + key] : 0.f;
            }
    };

    float kop[kS], vop[kS];
    f32x4 dkacc[kDT], dvacc[kDT];
    float dmask = 0.f;

    copy_step(0, &sm[0]);
    put_rows(&sm[0]);
    if (PAIR) load_pair(0);
    gfx::wait_all();
    __syncthreads();

    for (int it = 0; it < nsteps; ++it) {
        const KvBuf<KD>* __restrict__ cur = &sm[it & 1];
        const int hh = it / nqb, qblk = it - hh * nqb;
        if (qblk == 0) {
            // a new head: this lane's K/sqrt(D) and V rows (B operands of S and dP)
            const int kr = key_live ? key : L - 1;
            for (int j = 0; j < kS / 4; ++j) {
                const uint32_t e0 = (uint32_t)(kS * g + 4 * j), d0 = 4u * e0;
                const bool din = D >= 16 || e0 < (uint32_t)D;
                const uint4 wk = bload16(rk, din ? (uint32_t)kr * rowk + (uint32_t)hh * hk + d0 : kOOB);
                const uint4 wv = bload16(rv, din ? (uint32_t)kr * rowv + (uint32_t)hh * hv + d0 : kOOB);
                kop[4 * j] = __builtin_bit_cast(float, wk.x) * p.scale;
                kop[4 * j + 1] = __builtin_bit_cast(float, wk.y) * p.scale;
                kop[4 * j + 2] = __builtin_bit_cast(float, wk.z) * p.scale;
                kop[4 * j + 3] = __builtin_bit_cast(float, wk.w) * p.scale;
                vop[4 * j] = __builtin_bit_cast(float, wv.x);
                vop[4 * j + 1] = __builtin_bit_cast(float, wv.y);
                vop[4 * j + 2] = __builtin_bit_cast(float, wv.z);
                vop[4 * j + 3] = __builtin_bit_cast(float, wv.w);
            }
            for (int dt = 0; dt < kDT; ++dt) dkacc[dt] = dvacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const f32x4 pcur[kKT] = {pr[0], pr[1], pr[2], pr[3]};
        if (it + 1 < nsteps) {
            copy_step(it + 1, &sm[(it & 1) ^ 1]);
            if (PAIR) load_pair(it + 1);
        }
        for (int qt = 0; qt < kKT; ++qt) {
            // S (queries 16qt + 4g + i, key c) = Q.K^T/sqrt(D) + pair + mask, and dP - delta = dO.V^T - delta
            f32x4 s4 = PAIR ? pcur[qt] + mkey : f32x4{mkey, mkey, mkey, mkey};
            f32x4 dpm = cur->dl[4 * qt + g];
            float qf[kS], df[kS];
            tile_run<KD>(cur->q, 16 * qt + c, g, qf);
            tile_run<KD>(cur->dout, 16 * qt + c, g, df);
            for (int s = 0; s < kS; ++s) {
                s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[s], kop[s], s4, 0, 0, 0);
                dpm = __builtin_amdgcn_mfma_f32_16x16x4f32(df[s], vop[s], dpm, 0, 0, 0);
            }
            const f32x4 l2 = cur->ls[4 * qt + g];
            f32x4 pw, ds;
            for (int i = 0; i < 4; ++i) {
                pw[i] = __builtin_amdgcn_exp2f(fmaf(s4[i], kLog2e, -l2[i]));
                ds[i] = pw[i] * dpm[i];
                dmask += ds[i];
            }
            // dV^T += dO^T . P and dK^T += Q^T . dS: slice r takes query 16qt + 4g + r
            // from lane group g; operands A[m = d][k]: lane (c + 16g) takes row 16qt + 4g + r, column 16dt + c
            for (int r = 0; r < 4; ++r)
                for (int dt = 0; dt < kDT; ++dt) {
                    const float dov = tile_at<KD>(cur->dout, 16 * qt + 4 * g + r, 16 * dt + c);
                    const float qv = tile_at<KD>(cur->q, 16 * qt + 4 * g + r, 16 * dt + c);
                    dvacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(dov, pw[r], dvacc[dt], 0, 0, 0);
                    dkacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qv, ds[r], dkacc[dt], 0, 0, 0);
                }
        }
        if (it + 1 < nsteps) put_rows(&sm[(it & 1) ^ 1]);
        if (qblk == nqb - 1 && key_live) {
            // the head's dK^T[d = 16dt + 4g + i][key c] and dV^T
            const int64_t ko = kbn + (int64_t)hh * st.k[3] + (int64_t)key * st.k[2];
            const int64_t vo = vbn + (int64_t)hh * st.v[3] + (int64_t)key * st.v[2];
            for (int dt = 0; dt < kDT; ++dt) {
                if (D < 16 && 16 * dt + 4 * g >= D) continue;  // the padded rows
                *reinterpret_cast<f32x4*>(p.dk + ko + 16 * dt + 4 * g) = dkacc[dt] * p.scale;
                *reinterpret_cast<f32x4*>(p.dv + vo + 16 * dt + 4 * g) = dvacc[dt];
            }
        }
        gfx::wait_all();  // the next step's copies have landed and its rows are written
        __syncthreads();
    }
    dmask = gfx::sum_over_groups(dmask);
    if (p.dmask && g == 0 && key_live) p.dmask[b * st.mb + n * st.mn + key] = dmask;
}

// ---------------------------------------------------------------------------
// dpair.  Workgroup = one (b, h) tile of 64 queries x 64 keys and one range
// [n0, n1) of the N axis; wave w owns queries 16w .. 16w+15 against the 64
// keys, scores transposed (lane c + 16g holds keys 16kt + 4g + i of query
// 16w + c).  The pair rows of the tile are the same for every n and are read
// once.  Per n the tile's K and V rows (and its 64 mask values) come through
// LDS, shared by the four waves, one n ahead; each lane's own Q and dO
// d-range, lse and delta go straight to registers, also one n ahead.  dS is
// summed over the range in registers, n in order.  With one range the
// workgroup writes dpair; with several it writes its range's sum to the
// workspace and bwd_dpair_reduce_f32 adds the ranges in order.
// ---------------------------------------------------------------------------
template <int D>
struct PrBuf {
    f32x4 k[kKB * D / 4];
    f32x4 v[kKB * D / 4];
    f32x4 mt[kKB / 4];
};

struct PairParams {
    BParams p;
    float* ws;           // [chunks][B][H][L][bwd_ws_row(L)] fp32, or nullptr (one range: dpair itself)
    int64_t chunks;      // N is split into this many contiguous ranges
    gfx::FastDiv tiles;  // 64 x 64 tiles per (b, h): ceil(L/64)^2
    gfx::FastDiv tdim;   // ceil(L/64)
    gfx::FastDiv chd;    // chunks
    int64_t bh;          // B * H
};

template <int D, bool MASK, bool STAGED>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_dpair_f32_mfma(PairParams pp) {
    constexpr int KD = tile_width<D>();
    constexpr int kS = KD / 4;
    const BParams& p = pp.p;
    __shared__ __attribute__((aligned(16))) PrBuf<KD> sm[2];

    // order (b, h, range, query tile, key tile): the tiles of one (b, h,
    // range) run on one XCD together and share each n's rows in its L2
    const uint32_t id = (uint32_t)gfx::logical_block(blockIdx.x, p.total);
    const uint32_t r1 = gfx::fdiv(id, pp.tiles), r2 = gfx::fdiv(r1, pp.chd), r3 = gfx::fdiv(r2, p.hd);
    const uint32_t tile = id - r1 * pp.tiles.d;
    const uint32_t ti = gfx::fdiv(tile, pp.tdim), tj = tile - ti * pp.tdim.d;
    const int64_t chunk = r1 - r2 * pp.chd.d, h = r2 - r3 * p.hd.d, b = r3;
    const Strides& st = p.st;
    const int L = (int)p.L;
    const int64_t N = p.N;
    const int64_t n0 = chunk * N / pp.chunks, n1 = (chunk + 1) * N / pp.chunks;
    const int i0 = (int)ti * kKB, j0 = (int)tj * kKB;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int qi = i0 + 16 * wave + c;  // this lane's query
    const bool q_live = qi < L;

    const uint32_t rowq = (uint32_t)st.q[2] * 4, rowk = (uint32_t)st.k[2] * 4, rowv = (uint32_t)st.v[2] * 4;
    const uint32_t rowo = (uint32_t)st.o[2] * 4, rowp = (uint32_t)st.pi * 4;
    const uint32_t last = (uint32_t)(L - 1);

    // pair[b, h, qi, j0 + 16kt + 4g .. +3]: the accumulator input of every S^T product
    f32x4 pbs[kKT];
    {
        const uint32_t pbytes = last * rowp + (uint32_t)L * 4u;
        const Rsrc rp = make_rsrc(p.pair + b * st.pb + h * st.ph, STAGED ? pbytes : (pbytes + 15u) & ~15u);
        for (int kt = 0; kt < kKT; ++kt) {
            const uint32_t off = (uint32_t)qi * rowp + 4u * (uint32_t)(j0 + 16 * kt + 4 * g);
            pbs[kt] = __builtin_bit_cast(f32x4, STAGED ? bload16_any(rp, off, pbytes) : bload16(rp, off));
        }
    }

    RowCopy<KD, D> ck, cv;
    ck.init(wave, lane, rowk);
    cv.init(wave, lane, rowv);
    uint4 mstage;  // STAGED: the mask chunk between its load and its landing in LDS
    auto copy_step = [&](int64_t n, PrBuf<KD>* __restrict__ dst) {
        const Rsrc rk = make_rsrc(p.k + b * st.k[0] + n * st.k[1] + h * st.k[3], last * rowk + D * 4);
        const Rsrc rv = make_rsrc(p.v + b * st.v[0] + n * st.v[1] + h * st.v[3], last * rowv + D * 4);
        ck.issue(rk, dst->k, wave, (uint32_t)j0 * rowk);
        cv.issue(rv, dst->v, wave, (uint32_t)j0 * rowv);
        if (MASK && wave == 0 && lane < 16) {
            const uint32_t mbytes = (uint32_t)L * 4u;
            const Rsrc rm = make_rsrc(p.mask + b * st.mb + n * st.mn, STAGED ? mbytes : (mbytes + 15u) & ~15u);
            if (STAGED) mstage = bload16_any(rm, 16u * lane + (uint32_t)j0 * 4u, mbytes);
            else dma16_untracked(rm, &dst->mt[0], 16u * lane + (uint32_t)j0 * 4u);
        }
    };
    auto land_mask = [&](PrBuf<KD>* __restrict__ dst) {
        if (STAGED && MASK && wave == 0 && lane < 16) dst->mt[lane] = __builtin_bit_cast(f32x4, mstage);
    };
    // this lane's Q and dO d-range, lse and delta at sequence n, as loaded
    // (converted when used, so that the loads stay in flight meanwhile)
    uint4 qraw[kS / 4], draw[kS / 4];
    float lsraw = -INFINITY, dlraw = 0.f;
    auto load_rows = [&](int64_t n) {
        const Rsrc rq = make_rsrc(p.q + b * st.q[0] + n * st.q[1] + h * st.q[3], last * rowq + D * 4);
        const Rsrc rd = make_rsrc(p.dout + b * st.o[0] + n * st.o[1] + h * st.o[3], last * rowo + D * 4);
        for (int j = 0; j < kS / 4; ++j) {
            const uint32_t e0 = (uint32_t)(kS * g + 4 * j), d0 = 4u * e0;
            const bool din = D >= 16 || e0 < (uint32_t)D;
            qraw[j] = bload16(rq, din ? (uint32_t)qi * rowq + d0 : kOOB);
            draw[j] = bload16(rd, din ? (uint32_t)qi * rowo + d0 : kOOB);
        }
        if (q_live) {
            const int64_t row = ((b * N + n) * p.H + h) * st.lrow + qi;
            lsraw = p.lse[row];
            dlraw = p.delta[row];
        }
    };

    f32x4 ds[kKT];
    for (int kt = 0; kt < kKT; ++kt) ds[kt] = f32x4{0.f, 0.f, 0.f, 0.f};

    copy_step(n0, &sm[0]);
    land_mask(&sm[0]);
    load_rows(n0);
    gfx::wait_all();
    __syncthreads();

    for (int64_t n = n0; n < n1; ++n) {
        const int it = (int)(n - n0);
        const PrBuf<KD>* __restrict__ cur = &sm[it & 1];
        // Q/sqrt(D) and dO as B operands (lane group g's d-range of query c)
        float qop[kS], dop[kS];
        for (int j = 0; j < kS / 4; ++j) {
            const uint4 wq = qraw[j], wd = draw[j];
            qop[4 * j] = __builtin_bit_cast(float, wq.x) * p.scale;
            qop[4 * j + 1] = __builtin_bit_cast(float, wq.y) * p.scale;
            qop[4 * j + 2] = __builtin_bit_cast(float, wq.z) * p.scale;
            qop[4 * j + 3] = __builtin_bit_cast(float, wq.w) * p.scale;
            dop[4 * j] = __builtin_bit_cast(float, wd.x);
            dop[4 * j + 1] = __builtin_bit_cast(float, wd.y);
            dop[4 * j + 2] = __builtin_bit_cast(float, wd.z);
            dop[4 * j + 3] = __builtin_bit_cast(float, wd.w);
        }
        const float lse2 = q_live ? lse2_of(lsraw) : INFINITY;
        const float ndl = q_live ? -dlraw : 0.f;
        if (n + 1 < n1) {
            copy_step(n + 1, &sm[(it & 1) ^ 1]);
            load_rows(n + 1);
        }
        for (int kt = 0; kt < kKT; ++kt) {
            // S^T = K.Q^T/sqrt(D) + pair + mask and dP^T - delta = V.dO^T - delta
            f32x4 acc = pbs[kt];
            if (MASK) acc += cur->mt[4 * kt + g];
            f32x4 dpm = f32x4{ndl, ndl, ndl, ndl};
            float kf[kS], vf[kS];
            tile_run<KD>(cur->k, 16 * kt + c, g, kf);
            tile_run<KD>(cur->v, 16 * kt + c, g, vf);
            for (int s = 0; s < kS; ++s) {
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[s], qop[s], acc, 0, 0, 0);
                dpm = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[s], dop[s], dpm, 0, 0, 0);
            }
            for (int r = 0; r < 4; ++r)
                ds[kt][r] = fmaf(__builtin_amdgcn_exp2f(fmaf(acc[r], kLog2e, -lse2)), dpm[r], ds[kt][r]);
        }
        if (n + 1 < n1) land_mask(&sm[(it & 1) ^ 1]);
        gfx::wait_all();  // the next n's copies and rows have landed
        __syncthreads();
    }

    // lane c + 16g: query qi, keys j0 + 16kt + 4g + 0..3 (those past L are not written)
    if (!q_live) return;
    for (int kt = 0; kt < kKT; ++kt) {
        const int j = j0 + 16 * kt + 4 * g;
        if (j >= L) continue;
        if (pp.ws) {
            *reinterpret_cast<f32x4*>(pp.ws + ((chunk * pp.bh + b * p.H + h) * p.L + qi) * bwd_ws_row(p.L) + j) = ds[kt];
        } else {
            float* dst = p.dpair + b * st.pb + h * st.ph + (int64_t)qi * st.pi + j;
            if (!STAGED && j + 4 <= L) *reinterpret_cast<f32x4*>(dst) = ds[kt];
            else
                for (int e = 0; e < 4 && e < L - j; ++e) dst[e] = ds[kt][e];
        }
    }
}

// dpair[b,h,i,j] = sum over the workspace's ranges of their partial sums, in
// range order; four consecutive keys per thread.  The workspace is dense
// [chunks][B][H][L][bwd_ws_row(L)]; keys past L are skipped.
struct ReduceF32 {
    const float* ws;
    float* dpair;
    int64_t quads, chunks;  // B*H*L*bwd_ws_row(L) / 4; ranges
    int64_t L, H;
    int64_t pb, ph, pi;     // strides of dpair
    int aligned;            // dpair rows start 16-byte aligned
};

__global__ __launch_bounds__(256) void bwd_dpair_reduce_f32(ReduceF32 r) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= r.quads) return;
    f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t ch = 0; ch < r.chunks; ++ch) t += reinterpret_cast<const f32x4*>(r.ws)[ch * r.quads + q];
    const int64_t rq = bwd_ws_row(r.L) / 4, row = q / rq, j = 4 * (q - row * rq);  // row = (b * H + h) * L + i
    if (j >= r.L) return;
    const int64_t bh = row / r.L, i = row - bh * r.L, b = bh / r.H, h = bh - b * r.H;
    float* dst = r.dpair + b * r.pb + h * r.ph + i * r.pi + j;
    if (r.aligned && j + 4 <= r.L) *reinterpret_cast<f32x4*>(dst) = t;
    else
        for (int e = 0; e < 4 && e < r.L - j; ++e) dst[e] = t[e];
}

template <int D, bool MASK>
hipError_t launch_dpair(const BParams& base, int64_t B, float* ws, int64_t chunks, bool staged, hipStream_t stream) {
    PairParams pp;
    pp.p = base;
    const int64_t tdim = (base.L + kKB - 1) / kKB;
    pp.p.total = B * base.H * chunks * tdim * tdim;
    if (pp.p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    pp.ws = ws;
    pp.chunks = chunks;
    pp.tiles = gfx::make_fastdiv((uint32_t)(tdim * tdim));
    pp.tdim = gfx::make_fastdiv((uint32_t)tdim);
    pp.chd = gfx::make_fastdiv((uint32_t)chunks);
    pp.bh = B * base.H;
    void* args[] = {&pp};
    const void* kern = staged ? reinterpret_cast<const void*>(&bwd_dpair_f32_mfma<D, MASK, true>)
                              : reinterpret_cast<const void*>(&bwd_dpair_f32_mfma<D, MASK, false>);
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)pp.p.total), dim3(kWaves * 64), args, 0, stream);
    if (e != hipSuccess || !ws) return e;
    ReduceF32 r;
    r.ws = ws;
    r.dpair = base.dpair;
    r.quads = B * base.H * base.L * bwd_ws_row(base.L) / 4;
    r.chunks = chunks;
    r.L = base.L;
    r.H = base.H;
    r.pb = base.st.pb, r.ph = base.st.ph, r.pi = base.st.pi;
    r.aligned = !(r.pb % 4 || r.ph % 4 || r.pi % 4);
    const int64_t blocks = (r.quads + 255) / 256;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    void* rargs[] = {&r};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dpair_reduce_f32), dim3((unsigned)blocks), dim3(256),
                           rargs, 0, stream);
}

template <int D, bool PAIR, bool MASK>
hipError_t launch_stage(BParams p, int64_t B, unsigned stage, bool staged, hipStream_t stream) {
    const int64_t L = p.L;
    void* args[] = {&p};
    if (stage == kStageDq) {
        const int64_t qblocks = (L + dq_rows<D>() - 1) / dq_rows<D>();
        p.total = B * p.N * p.H * qblocks;
        p.rblocks = gfx::make_fastdiv((uint32_t)qblocks);
        const void* kern = staged ? reinterpret_cast<const void*>(&bwd_dq_f32_mfma<D, PAIR, MASK, true>)
                                  : reinterpret_cast<const void*>(&bwd_dq_f32_mfma<D, PAIR, MASK, false>);
        return hipLaunchKernel(kern, dim3((unsigned)p.total), dim3(kWaves * 64), args, 0, stream);
    }
    const int64_t kblocks = (L + kKB - 1) / kKB;
    p.total = B * p.N * kblocks;
    p.rblocks = gfx::make_fastdiv((uint32_t)kblocks);
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_f32_mfma<D, PAIR, MASK>), dim3((unsigned)p.total),
                           dim3(kWaves * 64), args, 0, stream);
}

template <int D>
hipError_t launch_stage_dim(const BParams& p, int64_t B, bool pair, bool mask, unsigned stage, bool staged,
                            hipStream_t stream) {
    if (pair && mask) return launch_stage<D, true, true>(p, B, stage, staged, stream);
    if (pair) return launch_stage<D, true, false>(p, B, stage, staged, stream);
    if (mask) return launch_stage<D, false, true>(p, B, stage, staged, stream);
    return launch_stage<D, false, false>(p, B, stage, false, stream);
}

}  // namespace

const unsigned kBwdF32MfmaStages = kStageDq | kStageDkDv | kStageDpair;

// D in {8, 16, 32, 64}; q, k, v, out rows 16-byte aligned (the C ABI checks
// that); bias rows at any stride (unaligned ones are staged).  Each row of
// q, k, v and out spans every head (row stride at least (H - 1) head
// strides + D), so that rows past L fall beyond the
// buffer of a (b, n) slice and read as zero: the dk/dv kernel sums over its
// query rows, and those past L must add exactly nothing.  Every byte offset
// the kernels form stays below 2^31: rows up to 128 past L of every head,
// pair rows up to 128 past L plus 64 keys.  The grids stay below 2^31
// workgroups (the pair-gradient grid is at most its tile count + 2048).
bool bwd_f32_mfma_eligible(const BwdArgs& a) {
    constexpr int64_t kLim = int64_t(1) << 31, kBig = int64_t(1) << 40;
    const int64_t L = a.L, H = a.H, D = a.D;
    if (D != 8 && D != 16 && D != 32 && D != 64) return false;
    if (a.N >= kLim || H >= kLim || L >= kLim) return false;
    for (const int64_t* t : {a.st.q, a.st.k, a.st.v, a.st.o}) {
        const int64_t row = t[2], head = t[3];
        if (row < 0 || head < 0 || row >= kBig || head >= kBig) return false;
        if (row < (H - 1) * head + D) return false;
        if (((L + 128) * row + (H - 1) * head + D) * 4 >= kLim) return false;
    }
    if (a.pair && (a.st.pi >= kBig || ((L + 128) * a.st.pi + L + kKB) * 4 >= kLim)) return false;
    if (a.mask && (L + kKB) * 4 >= kLim) return false;
    const int64_t tdim = (L + kKB - 1) / kKB;
    if (a.B * H * tdim * tdim + 2048 >= kLim) return false;
    return a.B * a.N * H * ((L + 63) / 64) < kLim;
}

hipError_t launch_bwd_f32_mfma(const BwdArgs& a, unsigned stages, hipStream_t stream) {
    BParams p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.mask = static_cast<const float*>(a.mask);
    p.pair = static_cast<const float*>(a.pair);
    p.out = static_cast<const float*>(a.out);
    p.dout = static_cast<const float*>(a.dout);
    p.lse = a.lse;
    p.dq = static_cast<float*>(a.dq);
    p.dk = static_cast<float*>(a.dk);
    p.dv = static_cast<float*>(a.dv);
    p.dmask = static_cast<float*>(a.dmask);
    p.dpair = static_cast<float*>(a.dpair);
    p.delta = a.delta;
    p.N = a.N, p.L = a.L, p.H = a.H;
    p.nd = gfx::make_fastdiv((uint32_t)a.N);
    p.hd = gfx::make_fastdiv((uint32_t)a.H);
    p.total = 0;
    p.st = a.st;
    p.scale = (float)(1.0 / std::sqrt((double)a.D));
    const bool pair = a.pair != nullptr, mask = a.mask != nullptr;
    // bias rows that do not all start 16-byte aligned are staged
    const bool staged = (pair && (a.st.pb % 4 || a.st.ph % 4 || a.st.pi % 4)) || (mask && (a.st.mb % 4 || a.st.mn % 4));
    hipError_t e = hipSuccess;
    for (unsigned stage : {kStageDq, kStageDkDv}) {
        if (!(stages & stage)) continue;
        if (a.D == 8) e = launch_stage_dim<8>(p, a.B, pair, mask, stage, staged, stream);
        else if (a.D == 16) e = launch_stage_dim<16>(p, a.B, pair, mask, stage, staged, stream);
        else if (a.D == 32) e = launch_stage_dim<32>(p, a.B, pair, mask, stage, staged, stream);
        else e = launch_stage_dim<64>(p, a.B, pair, mask, stage, staged, stream);
        if (e != hipSuccess) return e;
    }
    if ((stages & kStageDpair) && a.dpair) {
        // with a workspace of at least two ranges, split N; else one range per tile
        float* ws = a.ws && a.ws_chunks >= 2 ? a.ws : nullptr;
        const int64_t chunks = ws ? a.ws_chunks : 1;
        if (a.D == 8) e = mask ? launch_dpair<8, true>(p, a.B, ws, chunks, staged, stream)
                               : launch_dpair<8, false>(p, a.B, ws, chunks, staged, stream);
        else if (a.D == 16) e = mask ? launch_dpair<16, true>(p, a.B, ws, chunks, staged, stream)
                                : launch_dpair<16, false>(p, a.B, ws, chunks, staged, stream);
        else if (a.D == 32) e = mask ? launch_dpair<32, true>(p, a.B, ws, chunks, staged, stream)
                                     : launch_dpair<32, false>(p, a.B, ws, chunks, staged, stream);
        else e = mask ? launch_dpair<64, true>(p, a.B, ws, chunks, staged, stream)
                      : launch_dpair<64, false>(p, a.B, ws, chunks, staged, stream);
    }
    return e;
}

}  // namespace evo
