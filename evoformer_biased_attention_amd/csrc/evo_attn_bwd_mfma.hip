// Backward pass on the matrix cores (bf16 / f16, head dimension 8, 16, 32 or 64).
//
// The gradients (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
// hmyw.cn, sections 4 and 5.4: the backward pass recomputes the weights from
// the saved log-sum-exp and uses delta_i = dO_i . out_i) are, with
// P_ij = exp(s_ij - lse_i) and dS_ij = P_ij (dO_i . v_j - delta_i):
//   dq_i = sum_j dS_ij k_j / sqrt(D),  dk_j = sum_i dS_ij q_i / sqrt(D),
//   dv_j = sum_i P_ij dO_i, dmask = sum over h, i of dS, dpair = sum over n of dS.
//
// Every product runs on v_mfma_f32_16x16x32_{bf16,f16} (fp32 accumulation);
// the weights and dS enter the second products rounded to the input format.
// The result of a 16x16 MFMA leaves column n of the tile in lanes n, n+16,
// n+32, n+48, which is where the B operand of the next MFMA expects column n:
// a product whose result's row index is the next product's contraction index
// chains without any data exchange.  Hence two orientations:
//   bwd_dq_mfma   scores transposed (S^T = K.Q^T, one query per lane column):
//                 dQ^T = K^T . dS^T contracts over keys.  Also writes delta.
//   bwd_dkdv_mfma scores upright (S = Q.K^T, one key per lane column):
//                 dV^T = dO^T . P and dK^T = Q^T . dS contract over queries;
//                 the workgroup visits every head, so dmask is complete.
// The contraction index of a chained product is permuted (element e of a
// 32-wide chunk is row 16(e/4) + 4g + e%4 of the result tiles); the other
// operand is read through the transposing LDS read ds_read_b64_tr_b16 in the
// same order.
//
// Operand tiles move from global memory to LDS with buffer loads that write
// LDS directly, one block ahead, double buffered; buffer resources return
// zeros past their range, which pads rows past L and dimensions past D.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "evo_attn_launch.h"
#include "gfx950_common.h"

namespace evo {
namespace {

using namespace gfx;

constexpr int kWaves = 4;
constexpr int kWaveRows = 32;                // queries (dq kernel) or keys (dk/dv kernel) per wavefront
constexpr int kBlockRows = kWaves * kWaveRows;
constexpr int kKB = 64;                      // keys (dq kernel) or queries (dk/dv kernel) per LDS block
constexpr int kKT = kKB / 16;

// Byte range of a bias buffer of `bytes` bytes.  Direct copies need rows
// that start 16-byte aligned; their range ends at the 16-byte boundary after
// the last element, so that the last row's final chunk is read whole also
// when L % 8 != 0 (its elements past the row are keys past L, never used;
// that granule lies in the page of the last element).  Staged copies keep
// the exact range, which their element-wise reads at its end need.
__device__ inline uint32_t bias_range(uint32_t bytes, bool staged) { return staged ? bytes : (bytes + 15u) & ~15u; }

// Four consecutive 16-bit values at p of which the first n lie inside their
// row (n >= 1; the rest read as zero), at any 2-byte alignment.
__device__ inline uint2 load4(const u16* p, int n) {
    uint2 v = {0u, 0u};
    if (n >= 4) {
        __builtin_memcpy(&v, p, 8);
    } else {
        uint32_t e[3] = {0u, 0u, 0u};
        for (int q = 0; q < 3; ++q)
            if (q < n) e[q] = p[q];
        v = uint2{e[0] | (e[1] << 16), e[2]};
    }
    return v;
}

// The first n (>= 1) of four packed 16-bit values to p, at any 2-byte alignment.
__device__ inline void store4(u16* p, uint2 v, int n) {
    if (n >= 4) {
        __builtin_memcpy(p, &v, 8);
    } else {
        const u16 e[3] = {(u16)(v.x & 0xffffu), (u16)(v.x >> 16), (u16)(v.y & 0xffffu)};
        for (int q = 0; q < 3; ++q)
            if (q < n) p[q] = e[q];
    }
}

struct Params {
    const u16 *q, *k, *v, *mask, *pair, *out, *dout;
    const float* lse;
    u16 *dq, *dk, *dv, *dmask, *dpair;
    float* delta;
    int64_t N, L, H;
    FastDiv rblocks;  // ceil(L / 128): row blocks of the dq and dk/dv kernels
    FastDiv nd, hd;   // N, H
    int64_t total;    // workgroups of the launch
    float c1;         // log2(e) / sqrt(D): raw q.k -> base-2 exponent
    float scale;      // 1 / sqrt(D)
    Strides st;       // element strides; each gradient shares its tensor's (dout: out's, delta: lse's)
};

// Per-row constant of the exponent: lse * log2(e), or +inf for a row without
// softmax (lse = -inf) so that every weight of the row is exactly zero.
__device__ inline float lse_base2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ---------------------------------------------------------------------------
// dq (and delta).  Workgroup = 128 queries of one (b, n, h); wave w owns
// queries 32w .. 32w+31 as two 16-query tiles.  LDS per 64-key block, d-rows
// in 32-wide halves hh (two for D = 64):
//   k, v: half hh, slot 4*key + (chunk ^ ((key >> 2) & 3)), chunk = 8 d-values
//   pt:   slot 8*row + (chunk ^ (row & 7)), row = query of the workgroup, chunk = 8 keys
//   mt:   slot chunk (8 keys)
// ---------------------------------------------------------------------------
template <int DH>
struct DqBuf {
    uint4 k[DH][kKB * 4];
    uint4 v[DH][kKB * 4];
    uint4 pt[kBlockRows * 8];
    uint4 mt[8];
};

// STAGED: bias rows not 16-byte aligned (bias strides not multiples of 8
// elements); their tiles go global -> registers -> LDS through unaligned
// 16-byte loads, into the slots the direct copies would fill.
template <class E, int D, bool PAIR, bool MASK, bool STAGED>
__global__ __launch_bounds__(kWaves * 64, (D <= 32 && !STAGED) ? 3 : 2) void bwd_dq_mfma(Params p) {
    using V8 = typename E::v8;
    constexpr int kDC = D / 8;           // 16-byte chunks per row
    constexpr int kDH = (D + 31) / 32;   // 32-wide halves of a row
    constexpr int kDHT = (D + 15) / 16;  // 16-wide d tiles
    using Buf = DqBuf<kDH>;
    __shared__ __attribute__((aligned(16))) Buf sm[2];

    const uint32_t id = (uint32_t)logical_block(blockIdx.x, p.total);
    const uint32_t r1 = fdiv(id, p.rblocks), r2 = fdiv(r1, p.hd), r3 = fdiv(r2, p.nd);
    const int64_t qb = id - r1 * p.rblocks.d;
    const int64_t h = r1 - r2 * p.hd.d, n = r2 - r3 * p.nd.d, b = r3;
    const int L = (int)p.L;
    const Strides& st = p.st;
    // element offsets of (b, n, 0, h, 0) in q, k, v and out / dout
    const int64_t qs = b * st.q[0] + n * st.q[1] + h * st.q[3];
    const int64_t ks = b * st.k[0] + n * st.k[1] + h * st.k[3];
    const int64_t vs = b * st.v[0] + n * st.v[1] + h * st.v[3];
    const int64_t os = b * st.o[0] + n * st.o[1] + h * st.o[3];
    const int64_t rowbase = ((b * p.N + n) * p.H + h) * st.lrow;  // lse / delta index of query 0
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nblocks = (L + kKB - 1) / kKB;
    // bytes between consecutive rows; every offset below stays in 32 bits (the launcher checks)
    const uint32_t rowq = (uint32_t)st.q[2] * 2, rowk = (uint32_t)st.k[2] * 2, rowv = (uint32_t)st.v[2] * 2;
    const uint32_t rowo = (uint32_t)st.o[2] * 2, rowp = (uint32_t)st.pi * 2;
    const uint32_t last = (uint32_t)(L - 1);
    const Rsrc rq = make_rsrc(p.q + qs, last * rowq + D * 2);
    const Rsrc rk = make_rsrc(p.k + ks, last * rowk + D * 2);
    const Rsrc rv = make_rsrc(p.v + vs, last * rowv + D * 2);
    const Rsrc rdo = make_rsrc(p.dout + os, last * rowo + D * 2);
    const Rsrc ro = make_rsrc(p.out + os, last * rowo + D * 2);
    // bias buffers: direct copies read whole 16-byte granules at the end (bias_range)
    const Rsrc rp = make_rsrc(PAIR ? p.pair + b * st.pb + h * st.ph : p.q,
                              PAIR ? bias_range(last * rowp + (uint32_t)L * 2u, STAGED) : 0u);
    const Rsrc rm = make_rsrc(MASK ? p.mask + b * st.mb + n * st.mn : p.q, MASK ? bias_range((uint32_t)L * 2u, STAGED) : 0u);

    const int q0 = (int)qb * kBlockRows + wave * kWaveRows;
    // B operands of S^T = K.Q^T and dP^T = V.dO^T: lane (c + 16g) holds row
    // (query c of the tile), d-values 32hh + 8g .. +7 of half hh; rows past L
    // and chunks past D read as zero
    V8 qop[2][kDH], dop[2][kDH];
    float delta[2], lse2[2];
    for (int t = 0; t < 2; ++t) {
        const int i = q0 + 16 * t + c;
        float part = 0.f;
        for (int hh = 0; hh < kDH; ++hh) {
            const bool in = 4 * hh + g < kDC;
            const uint32_t offq = in ? (uint32_t)i * rowq + 64u * hh + 16u * g : kOOB;
            const uint32_t offo = in ? (uint32_t)i * rowo + 64u * hh + 16u * g : kOOB;
            const uint4 qq = bload16(rq, offq, 0), dd = bload16(rdo, offo, 0), oo = bload16(ro, offo, 0);
            qop[t][hh] = as_v8<E>(qq);
            dop[t][hh] = as_v8<E>(dd);
            const uint32_t dw[4] = {dd.x, dd.y, dd.z, dd.w}, ow[4] = {oo.x, oo.y, oo.z, oo.w};
            for (int e = 0; e < 4; ++e) {
                const f32x2 a = unpack2<E>(dw[e]), o = unpack2<E>(ow[e]);
                part = fmaf(a[0], o[0], part);
                part = fmaf(a[1], o[1], part);
            }
        }
        delta[t] = sum_over_groups(part);
        lse2[t] = i < L ? lse_base2(p.lse[rowbase + i]) : INFINITY;
        if (g == 0 && i < L) p.delta[rowbase + i] = delta[t];
    }

    // copies of one 64-key block (same addressing as the forward kernel)
    const uint32_t qwg = (uint32_t)(qb * kBlockRows);
    const uint32_t kvchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t kvrow = (uint32_t)(16 * wave + (lane >> 2));
    uint32_t ko[kDH], vo[kDH];
    for (int hh = 0; hh < kDH; ++hh) {
        const bool in = 4 * hh + (int)kvchunk < kDC;
        ko[hh] = in ? kvrow * rowk + 64u * hh + 16u * kvchunk : kOOB;
        vo[hh] = in ? kvrow * rowv + 64u * hh + 16u * kvchunk : kOOB;
    }
    uint32_t pvo[4];
    for (int j = 0; j < 4; ++j) {
        // rows past L start beyond the pair range (its row stride is at least L)
        const uint32_t row = 8u * (4 * wave + j) + (lane >> 3);
        pvo[j] = (qwg + row) * rowp + 16u * ((lane & 7) ^ (lane >> 3));
    }
    uint4 pstage[4], mstage;  // STAGED: chunks between their load and their landing in LDS
    const uint32_t prange = PAIR ? last * rowp + (uint32_t)L * 2u : 0u;
    // The copies of a block: the direct ones (K, V and, with aligned rows, the
    // bias tiles) go straight into LDS as untracked copies, waited for by
    // wait_all() before the step's barrier; STAGED bias chunks go through
    // registers (copy_staged), after the step's LDS reads, whose registers they reuse.
    auto copy_direct = [&](int blk, Buf* __restrict__ dst) {
        const uint32_t k0 = (uint32_t)blk * kKB;
        for (int hh = 0; hh < kDH; ++hh) {
            dma16_untracked(rk, &dst->k[hh][64 * wave], ko[hh] + k0 * rowk);
            dma16_untracked(rv, &dst->v[hh][64 * wave], vo[hh] + k0 * rowv);
        }
        if (!STAGED) {
            if (PAIR)
                for (int j = 0; j < 4; ++j) dma16_untracked(rp, &dst->pt[64 * (4 * wave + j)], pvo[j] + k0 * 2u);
            if (MASK && wave == 0 && lane < 8) dma16_untracked(rm, &dst->mt[0], 16u * lane + k0 * 2u);
        }
    };
    auto copy_staged = [&](int blk) {
        if (!STAGED) return;
        const uint32_t k0 = (uint32_t)blk * kKB;
        if (PAIR)
            for (int j = 0; j < 4; ++j) pstage[j] = bload16_any(rp, pvo[j] + k0 * 2u, prange);
        if (MASK && wave == 0 && lane < 8) mstage = bload16_any(rm, 16u * lane + k0 * 2u, (uint32_t)L * 2u);
    };
    auto land_block = [&](Buf* __restrict__ dst) {
        if (!STAGED) return;
        if (PAIR)
            for (int j = 0; j < 4; ++j) dst->pt[64 * (4 * wave + j) + lane] = pstage[j];
        if (MASK && wave == 0 && lane < 8) dst->mt[lane] = mstage;
    };

    f32x4 dqacc[2][kDHT];
    for (int t = 0; t < 2; ++t)
        for (int dh = 0; dh < kDHT; ++dh) dqacc[t][dh] = f32x4{0.f, 0.f, 0.f, 0.f};

    copy_direct(0, &sm[0]);
    copy_staged(0);
    land_block(&sm[0]);
    wait_all();
    __syncthreads();

    auto step = [&](int it, const Buf* __restrict__ cur, Buf* __restrict__ nxt, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int k0 = it * kKB;
        // the next block's direct copies first (the other buffer's readers all
        // passed the previous barrier), its staged chunks after the reads
        if (it + 1 < nblocks) copy_direct(it + 1, nxt);
        // A operands: K and V rows (key 16kt + c, chunk g) and transposed K
        // for dQ^T = K^T.dS^T (column 16dh + c over keys 32cc + 4g + 0..3 and
        // 32cc + 16 + 4g + 0..3)
        V8 kop[kKT][kDH], vop[kKT][kDH], ktr[2][kDHT];
        for (int kt = 0; kt < kKT; ++kt)
            for (int hh = 0; hh < kDH; ++hh) {
                kop[kt][hh] = as_v8<E>(cur->k[hh][64 * kt + 4 * c + (g ^ ((c >> 2) & 3))]);
                vop[kt][hh] = as_v8<E>(cur->v[hh][64 * kt + 4 * c + (g ^ ((c >> 2) & 3))]);
            }
        for (int cc = 0; cc < 2; ++cc)
            for (int dh = 0; dh < kDHT; ++dh) {
                const int key = 32 * cc + 4 * g + (c >> 2);
                const int chunk = (2 * (dh & 1) + ((c & 3) >> 1)) ^ g;
                const char* base = reinterpret_cast<const char*>(&cur->k[dh >> 1][4 * key + chunk]) + 8 * (c & 1);
                const uint2 lo = ds_read_tr(base);
                const uint2 hi = ds_read_tr(base + 16 * 4 * 16);
                ktr[cc][dh] = as_v8<E>(uint4{lo.x, lo.y, hi.x, hi.y});
            }
        // biases of lane (c + 16g): keys 16kt + 4g + 0..3 (8 bytes), query c of each tile
        uint2 pb[2][kKT], mb[kKT];
        for (int kt = 0; kt < kKT; ++kt) {
            const int chunk = 2 * kt + (g >> 1);
            if (MASK) mb[kt] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(&cur->mt[chunk]) + 8 * (g & 1));
            if (PAIR)
                for (int t = 0; t < 2; ++t) {
                    const int row = wave * kWaveRows + 16 * t + c;
                    pb[t][kt] = *reinterpret_cast<const uint2*>(
                        reinterpret_cast<const char*>(&cur->pt[8 * row + (chunk ^ (c & 7))]) + 8 * (g & 1));
                }
        }

        if (STAGED && it + 1 < nblocks) copy_staged(it + 1);

        f32x4 s[2][kKT], dp[2][kKT];
        for (int kt = 0; kt < kKT; ++kt)
            for (int t = 0; t < 2; ++t) {
                s[t][kt] = dp[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int hh = 0; hh < kDH; ++hh) {
                    s[t][kt] = E::mfma(kop[kt][hh], qop[t][hh], s[t][kt]);
                    dp[t][kt] = E::mfma(vop[kt][hh], dop[t][hh], dp[t][kt]);
                }
            }
        V8 dsop[2][2];
        for (int t = 0; t < 2; ++t) {
            uint32_t w[8];
            for (int kt = 0; kt < kKT; ++kt) {
                float bias[4] = {0.f, 0.f, 0.f, 0.f};
                if (MASK) {
                    const f32x2 m01 = unpack2<E>(mb[kt].x), m23 = unpack2<E>(mb[kt].y);
                    bias[0] = m01[0], bias[1] = m01[1], bias[2] = m23[0], bias[3] = m23[1];
                }
                if (PAIR) {
                    const f32x2 a01 = unpack2<E>(pb[t][kt].x), a23 = unpack2<E>(pb[t][kt].y);
                    bias[0] += a01[0], bias[1] += a01[1], bias[2] += a23[0], bias[3] += a23[1];
                }
                float ds[4];
                for (int r = 0; r < 4; ++r) {
                    float x = fmaf(s[t][kt][r], p.c1, fmaf(bias[r], kLog2e, -lse2[t]));
                    if (TAIL && k0 + 16 * kt + 4 * g + r >= L) x = -INFINITY;  // keys past L take no weight
                    ds[r] = __builtin_amdgcn_exp2f(x) * (dp[t][kt][r] - delta[t]);
                }
                w[2 * kt] = pack2<E>(ds[0], ds[1]);
                w[2 * kt + 1] = pack2<E>(ds[2], ds[3]);
            }
            // element e of 32-key chunk cc is key 32cc + 16(e/4) + 4g + e%4
            dsop[t][0] = as_v8<E>(uint4{w[0], w[1], w[2], w[3]});
            dsop[t][1] = as_v8<E>(uint4{w[4], w[5], w[6], w[7]});
        }
        for (int cc = 0; cc < 2; ++cc)
            for (int dh = 0; dh < kDHT; ++dh)
                for (int t = 0; t < 2; ++t) dqacc[t][dh] = E::mfma(ktr[cc][dh], dsop[t][cc], dqacc[t][dh]);

        if (it + 1 < nblocks) land_block(nxt);
        wait_all();
        __syncthreads();
    };
    for (int it = 0; it + 1 < nblocks; ++it) step(it, &sm[it & 1], &sm[(it & 1) ^ 1], std::false_type{});
    {
        const int it = nblocks - 1;
        if (L % kKB) step(it, &sm[it & 1], &sm[(it & 1) ^ 1], std::true_type{});
        else step(it, &sm[it & 1], &sm[(it & 1) ^ 1], std::false_type{});
    }

    // lane (c + 16g) holds dQ^T[d = 16dh + 4g + r][query c]
    for (int t = 0; t < 2; ++t) {
        const int64_t i = q0 + 16 * t + c;
        if (i >= L) continue;
        for (int dh = 0; dh < kDHT; ++dh) {
            if (16 * dh + 4 * g >= D) continue;
            const f32x4 o = dqacc[t][dh] * p.scale;
            *reinterpret_cast<uint2*>(p.dq + qs + i * st.q[2] + 16 * dh + 4 * g) =
                uint2{pack2<E>(o[0], o[1]), pack2<E>(o[2], o[3])};
        }
    }
}

// ---------------------------------------------------------------------------
// dk, dv and dmask.  Workgroup = 64 KT keys of one (b, n); wave w owns keys
// 16 KT w .. as KT 16-key tiles and keeps their K and V rows (B operands of
// S = Q.K^T and dP = dO.V^T) in registers.  The workgroup walks every (head,
// QS-query block) pair in order.  KT = 1 (one 16-key tile per wave, which
// keeps a step within the registers of three waves per SIMD); QS = 64 for
// head dimensions up to 32, QS = 32 for D = 64 (two 32-wide halves of every
// row), so that each step's q and dO tiles are one wave-wide copy per wave.
// LDS per step, d-rows in 32-wide halves hh:
//   q, dO: half hh, slot 4*row + (chunk ^ ((row >> 2) & 3)), row = query of the block, chunk = 8 d-values
//   pt:    slot (8 KT)*row + (chunk ^ 2(row & (4 KT - 1))), chunk = 8 of the workgroup's keys
//   ls:    lse * log2(e) of the block's queries (+inf past L or for a row without softmax)
//   dl:    -delta of the block's queries (the accumulator input of dP)
// Queries past L read as zero rows with ls = +inf, so they add nothing; keys
// past L are computed on zero rows and never stored.
// ---------------------------------------------------------------------------
template <int QS, int DH, int KT>
struct KvBuf {
    uint4 q[DH][QS * 4];
    uint4 dout[DH][QS * 4];
    uint4 pt[QS * 8 * KT];
    float ls[QS];
    float dl[QS];
};

template <int D>
struct DkdvShape {
    static constexpr int KT = 1;                 // 16-key tiles per wave
    static constexpr int QS = D > 32 ? 32 : 64;  // queries per step
    static constexpr int BK = kWaves * 16 * KT;  // keys per workgroup
};

template <class E, int D, bool PAIR, bool MASK, bool STAGED>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_dkdv_mfma(Params p) {
    using V8 = typename E::v8;
    constexpr int kDC = D / 8;
    constexpr int kDH = (D + 31) / 32;        // 32-wide halves of a row
    constexpr int kDHT = (D + 15) / 16;       // 16-wide d tiles
    constexpr int KT = DkdvShape<D>::KT, QS = DkdvShape<D>::QS, BK = DkdvShape<D>::BK;
    constexpr int QT = QS / 16, CC = QS / 32; // 16-query tiles and 32-query chunks of a step
    constexpr int CPR = 8 * KT;               // 16-byte pair chunks per row of the tile
    constexpr int RPI = 64 / CPR;             // pair rows per wave-wide copy
    constexpr int PCW = QS / RPI / kWaves;    // pair copies per wave and step
    constexpr int RG = QS / 16;               // 16-row groups of a half (q and dO copies)
    // the q and dO copies take one wave-wide copy per wave and tensor
    static_assert(QS * 4 * kDH == 64 * kWaves, "q/dO tile must be one wave-wide copy per wave");
    static_assert(PCW >= 1 && PCW * RPI * kWaves == QS, "pair tile must split evenly over the waves");
    __shared__ __attribute__((aligned(16))) KvBuf<QS, kDH, KT> sm[2];

    const uint32_t id = (uint32_t)logical_block(blockIdx.x, p.total);
    const uint32_t r1 = fdiv(id, p.rblocks), r2 = fdiv(r1, p.nd);
    const int64_t kb = id - r1 * p.rblocks.d;
    const int64_t n = r1 - r2 * p.nd.d, b = r2;
    const int L = (int)p.L, H = (int)p.H;
    const Strides& st = p.st;
    const int64_t bn = b * p.N + n;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nqb = (L + QS - 1) / QS;  // query blocks per head
    const int nsteps = H * nqb;
    // element offsets of (b, n, 0, 0, 0) in q, k, v and out / dout; bytes
    // between rows and between heads.  A buffer covers every head of the
    // sequence; its offsets stay in 32 bits (the launcher checks).
    const int64_t qbn = b * st.q[0] + n * st.q[1], kbn = b * st.k[0] + n * st.k[1];
    const int64_t vbn = b * st.v[0] + n * st.v[1], obn = b * st.o[0] + n * st.o[1];
    const uint32_t rowq = (uint32_t)st.q[2] * 2, rowk = (uint32_t)st.k[2] * 2, rowv = (uint32_t)st.v[2] * 2;
    const uint32_t rowo = (uint32_t)st.o[2] * 2, rowp = (uint32_t)st.pi * 2;
    const uint32_t hq = (uint32_t)st.q[3] * 2, hk = (uint32_t)st.k[3] * 2, hv = (uint32_t)st.v[3] * 2;
    const uint32_t ho = (uint32_t)st.o[3] * 2;
    const uint32_t last = (uint32_t)(L - 1), lasth = (uint32_t)(H - 1);
    const Rsrc rq = make_rsrc(p.q + qbn, last * rowq + lasth * hq + D * 2);
    const Rsrc rk = make_rsrc(p.k + kbn, last * rowk + lasth * hk + D * 2);
    const Rsrc rv = make_rsrc(p.v + vbn, last * rowv + lasth * hv + D * 2);
    const Rsrc rdo = make_rsrc(p.dout + obn, last * rowo + lasth * ho + D * 2);
    const int kw0 = (int)kb * BK + wave * 16 * KT;  // first key of the wave
    const int64_t mrow = b * st.mb + n * st.mn;     // mask row of (b, n)

    // per-key mask term (base 2), constant over heads and queries
    float mk[KT];
    for (int t = 0; t < KT; ++t) {
        const int j = kw0 + 16 * t + c;
        mk[t] = MASK && j < L ? E::widen(p.mask[mrow + j]) * kLog2e : 0.f;
    }

    // copies of step `it` (head it / nqb, queries QS (it % nqb) ..).  q and
    // dO: wave w fills 16-row group w % RG of half w / RG; lane l holds row
    // 16 (w % RG) + l/4 at slot position l%4, chunk (l%4) ^ ((row >> 2) & 3).
    const int qhh = wave / RG, qrg = wave % RG;
    const uint32_t qdchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t qdrow = (uint32_t)(16 * qrg + (lane >> 2));
    const bool qdin = 4 * qhh + (int)qdchunk < kDC;
    const uint32_t qoff = qdin ? qdrow * rowq + 64u * qhh + 16u * qdchunk : kOOB;
    const uint32_t dooff = qdin ? qdrow * rowo + 64u * qhh + 16u * qdchunk : kOOB;
    // pair tile: rows of CPR chunks; wave w fills copies PCW w .. PCW w + PCW - 1,
    // RPI rows each; lane l holds row RPI I + l / CPR at position l % CPR
    uint32_t pvo[PCW];
    for (int j = 0; j < PCW; ++j) {
        // rows past L start beyond the pair range (its row stride is at least L)
        const uint32_t row = (uint32_t)(RPI * (PCW * wave + j) + lane / CPR);
        pvo[j] = row * rowp + (uint32_t)kb * BK * 2u + 16u * ((lane % CPR) ^ (2 * (row & (CPR / 2 - 1))));
    }
    float lsv = 0.f, dlv = 0.f;  // wave 0: this lane's query of the step being copied
    uint4 pstage[PCW];           // STAGED: pair chunks between their load and their landing in LDS
    // The step copied next: head ch, queries from cq0; its byte offsets within
    // the q and dO buffers, its pair matrix and its lse / delta rows.  All are
    // advanced step by step (no division or 64-bit product inside the loop).
    int ch = 0, cq0 = 0;
    uint32_t cqo = 0, cdo = 0;
    const u16* cpair = PAIR ? p.pair + b * st.pb : p.q;
    const float* clse = p.lse + bn * p.H * st.lrow;
    const float* cdelta = p.delta + bn * p.H * st.lrow;
    // The copies of the step at the cursor: the direct ones (q, dO and, with
    // aligned rows, the pair tile) go straight into LDS as untracked copies,
    // waited for by wait_all() before the step's barrier; copy_rest loads the
    // lse / delta rows and (STAGED) the pair chunks into registers.
    auto copy_direct = [&](KvBuf<QS, kDH, KT>* __restrict__ dst) {
        dma16_untracked(rq, &dst->q[qhh][64 * qrg], qoff + cqo);
        dma16_untracked(rdo, &dst->dout[qhh][64 * qrg], dooff + cdo);
        if (PAIR && !STAGED) {
            const Rsrc rp = make_rsrc(cpair, bias_range(last * rowp + (uint32_t)L * 2u, false));
            for (int j = 0; j < PCW; ++j)
                dma16_untracked(rp, &dst->pt[64 * (PCW * wave + j)], pvo[j] + (uint32_t)cq0 * rowp);
        }
    };
    auto copy_rest = [&]() {
        if (PAIR && STAGED) {
            const uint32_t prange = last * rowp + (uint32_t)L * 2u;
            const Rsrc rp = make_rsrc(cpair, bias_range(prange, true));
            for (int j = 0; j < PCW; ++j) pstage[j] = bload16_any(rp, pvo[j] + (uint32_t)cq0 * rowp, prange);
        }
        if (wave == 0 && lane < QS) {
            const int i = cq0 + lane;
            lsv = i < L ? lse_base2(clse[i]) : INFINITY;
            dlv = i < L ? -cdelta[i] : 0.f;  // negated: the accumulator input of dP
        }
    };
    auto next_copy = [&]() {
        cq0 += QS;
        cqo += (uint32_t)QS * rowq;
        cdo += (uint32_t)QS * rowo;
        if (cq0 >= L) {  // the next head
            cq0 = 0;
            ++ch;
            cqo = (uint32_t)ch * hq;
            cdo = (uint32_t)ch * ho;
            cpair += st.ph;
            clse += st.lrow;
            cdelta += st.lrow;
        }
    };
    auto put_rows = [&](KvBuf<QS, kDH, KT>* __restrict__ dst) {
        if (wave == 0 && lane < QS) {
            dst->ls[lane] = lsv;
            dst->dl[lane] = dlv;
        }
        if (STAGED && PAIR)
            for (int j = 0; j < PCW; ++j) dst->pt[64 * (PCW * wave + j) + lane] = pstage[j];
    };

    V8 kop[KT][kDH], vop[KT][kDH];
    f32x4 dkacc[KT][kDHT], dvacc[KT][kDHT];
    float dm[KT];
    for (int t = 0; t < KT; ++t) dm[t] = 0.f;

    copy_direct(&sm[0]);
    copy_rest();
    next_copy();
    put_rows(&sm[0]);
    wait_all();
    __syncthreads();

    // the wave's K and V rows of head hd (A operands over d, key 16t + c, chunk g of each half)
    auto load_kv = [&](int hd) {
        for (int t = 0; t < KT; ++t) {
            const uint32_t j = (uint32_t)(kw0 + 16 * t + c);
            for (int hh = 0; hh < kDH; ++hh) {
                const bool in = 4 * hh + g < kDC;
                kop[t][hh] = as_v8<E>(bload16(rk, in ? j * rowk + (uint32_t)hd * hk + 64u * hh + 16u * g : kOOB, 0));
                vop[t][hh] = as_v8<E>(bload16(rv, in ? j * rowv + (uint32_t)hd * hv + 64u * hh + 16u * g : kOOB, 0));
            }
        }
    };
    int h = 0, qbk = 0;  // the step's head and query block
    for (int it = 0; it < nsteps; ++it) {
        const KvBuf<QS, kDH, KT>* __restrict__ cur = &sm[it & 1];
        KvBuf<QS, kDH, KT>* __restrict__ nxt = &sm[(it & 1) ^ 1];
        // the next step's direct copies first (see the dq kernel); STAGED
        // loads its registers after the step's reads
        if (it + 1 < nsteps) {
            copy_direct(nxt);
            if (!STAGED) {
                copy_rest();
                next_copy();
            }
        }
        if (qbk == 0) {
            // aligned bias rows: later heads were loaded during the previous
            // head's last step (STAGED has no registers to spare for that)
            if (h == 0 || STAGED) load_kv(h);
            for (int t = 0; t < KT; ++t)
                for (int dh = 0; dh < kDHT; ++dh) dkacc[t][dh] = dvacc[t][dh] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // A operands: Q and dO rows (query 16qt + c, chunk g of each half);
        // transposed Q and dO for the products over queries (column 16dh + c
        // over queries 32cc + 4g + 0..3 and 32cc + 16 + 4g + 0..3)
        V8 aq[QT][kDH], ado[QT][kDH], qtr[CC][kDHT], dotr[CC][kDHT];
        for (int qt = 0; qt < QT; ++qt)
            for (int hh = 0; hh < kDH; ++hh) {
                aq[qt][hh] = as_v8<E>(cur->q[hh][64 * qt + 4 * c + (g ^ ((c >> 2) & 3))]);
                ado[qt][hh] = as_v8<E>(cur->dout[hh][64 * qt + 4 * c + (g ^ ((c >> 2) & 3))]);
            }
        for (int cc = 0; cc < CC; ++cc)
            for (int dh = 0; dh < kDHT; ++dh) {
                const int row = 32 * cc + 4 * g + (c >> 2);
                const int chunk = (2 * (dh & 1) + ((c & 3) >> 1)) ^ g;
                const int off = 16 * (4 * row + chunk) + 8 * (c & 1);
                const char* bq = reinterpret_cast<const char*>(cur->q[dh >> 1]) + off;
                const char* bd = reinterpret_cast<const char*>(cur->dout[dh >> 1]) + off;
                const uint2 ql = ds_read_tr(bq), qh = ds_read_tr(bq + 16 * 4 * 16);
                const uint2 dl = ds_read_tr(bd), dhh = ds_read_tr(bd + 16 * 4 * 16);
                qtr[cc][dh] = as_v8<E>(uint4{ql.x, ql.y, qh.x, qh.y});
                dotr[cc][dh] = as_v8<E>(uint4{dl.x, dl.y, dhh.x, dhh.y});
            }
        // pair bias of lane (c + 16g): queries 16qt + 4g + 0..3, key 16t + c of the wave
        uint2 pb[QT][KT];
        if (PAIR)
            for (int qt = 0; qt < QT; ++qt)
                for (int t = 0; t < KT; ++t) {
                    const int row = 16 * qt + 4 * g + (c >> 2);
                    const int chunk = 2 * KT * wave + 2 * t + ((c & 3) >> 1);
                    pb[qt][t] = ds_read_tr(
                        reinterpret_cast<const char*>(&cur->pt[CPR * row + (chunk ^ (2 * (row & (CPR / 2 - 1))))]) +
                        8 * (c & 1));
                }
        float4 lsq[QT], dlq[QT];
        for (int qt = 0; qt < QT; ++qt) {
            lsq[qt] = *reinterpret_cast<const float4*>(&cur->ls[16 * qt + 4 * g]);
            dlq[qt] = *reinterpret_cast<const float4*>(&cur->dl[16 * qt + 4 * g]);
        }

        if (STAGED && it + 1 < nsteps) {
            copy_rest();
            next_copy();
        }

        f32x4 sc[QT][KT], dp[QT][KT];
        for (int qt = 0; qt < QT; ++qt)
            for (int t = 0; t < KT; ++t) {
                sc[qt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                dp[qt][t] = f32x4{dlq[qt].x, dlq[qt].y, dlq[qt].z, dlq[qt].w};  // -delta: dP - delta comes out
                for (int hh = 0; hh < kDH; ++hh) {
                    sc[qt][t] = E::mfma(aq[qt][hh], kop[t][hh], sc[qt][t]);
                    dp[qt][t] = E::mfma(ado[qt][hh], vop[t][hh], dp[qt][t]);
                }
            }
        // the head's last step: its K and V rows are no longer needed, so the
        // next head's are loaded now and land during the rest of the step
        if (!STAGED && qbk == nqb - 1 && h + 1 < H) load_kv(h + 1);
        // lane (c + 16g) holds S[query 16qt + 4g + r][key 16t + c]
        V8 pm[KT][CC], dsm[KT][CC];
        for (int t = 0; t < KT; ++t) {
            uint32_t wp[2 * QT], wd[2 * QT];
            for (int qt = 0; qt < QT; ++qt) {
                const float lsr[4] = {lsq[qt].x, lsq[qt].y, lsq[qt].z, lsq[qt].w};
                float bias[4] = {0.f, 0.f, 0.f, 0.f};
                if (PAIR) {
                    const f32x2 a01 = unpack2<E>(pb[qt][t].x), a23 = unpack2<E>(pb[qt][t].y);
                    bias[0] = a01[0], bias[1] = a01[1], bias[2] = a23[0], bias[3] = a23[1];
                }
                float pr[4], ds[4];
                for (int r = 0; r < 4; ++r) {
                    const float x = fmaf(sc[qt][t][r], p.c1, fmaf(bias[r], kLog2e, mk[t] - lsr[r]));
                    pr[r] = __builtin_amdgcn_exp2f(x);
                    ds[r] = pr[r] * dp[qt][t][r];
                    dm[t] += ds[r];
                }
                wp[2 * qt] = pack2<E>(pr[0], pr[1]);
                wp[2 * qt + 1] = pack2<E>(pr[2], pr[3]);
                wd[2 * qt] = pack2<E>(ds[0], ds[1]);
                wd[2 * qt + 1] = pack2<E>(ds[2], ds[3]);
            }
            // element e of 32-query chunk cc is query 32cc + 16(e/4) + 4g + e%4
            for (int cc = 0; cc < CC; ++cc) {
                pm[t][cc] = as_v8<E>(uint4{wp[4 * cc], wp[4 * cc + 1], wp[4 * cc + 2], wp[4 * cc + 3]});
                dsm[t][cc] = as_v8<E>(uint4{wd[4 * cc], wd[4 * cc + 1], wd[4 * cc + 2], wd[4 * cc + 3]});
            }
        }
        for (int cc = 0; cc < CC; ++cc)
            for (int dh = 0; dh < kDHT; ++dh)
                for (int t = 0; t < KT; ++t) {
                    dvacc[t][dh] = E::mfma(dotr[cc][dh], pm[t][cc], dvacc[t][dh]);
                    dkacc[t][dh] = E::mfma(qtr[cc][dh], dsm[t][cc], dkacc[t][dh]);
                }

        if (it + 1 < nsteps) put_rows(nxt);
        wait_all();
        __syncthreads();

        if (qbk == nqb - 1) {
            // lane (c + 16g) holds dK^T, dV^T[d = 16dh + 4g + r][key 16t + c]
            for (int t = 0; t < KT; ++t) {
                const int64_t j = kw0 + 16 * t + c;
                if (j >= L) continue;
                for (int dh = 0; dh < kDHT; ++dh) {
                    if (16 * dh + 4 * g >= D) continue;
                    const int64_t d0 = 16 * dh + 4 * g;
                    const f32x4 dk = dkacc[t][dh] * p.scale, dv = dvacc[t][dh];
                    *reinterpret_cast<uint2*>(p.dk + kbn + j * st.k[2] + h * st.k[3] + d0) =
                        uint2{pack2<E>(dk[0], dk[1]), pack2<E>(dk[2], dk[3])};
                    *reinterpret_cast<uint2*>(p.dv + vbn + j * st.v[2] + h * st.v[3] + d0) =
                        uint2{pack2<E>(dv[0], dv[1]), pack2<E>(dv[2], dv[3])};
                }
            }
        }
        if (++qbk == nqb) qbk = 0, ++h;
    }
    if (MASK && p.dmask)
        for (int t = 0; t < KT; ++t) {
            const float tot = sum_over_groups(dm[t]);
            const int j = kw0 + 16 * t + c;
            if (g == 0 && j < L) {
                const uint32_t w = pack2<E>(tot, 0.f);
                p.dmask[mrow + j] = (u16)(w & 0xffffu);
            }
        }
}

template <class E, int D, bool PAIR, bool MASK, bool STAGED>
hipError_t launch_dkdv(Params& p, int64_t B, hipStream_t stream) {
    const int64_t rblocks = (p.L + DkdvShape<D>::BK - 1) / DkdvShape<D>::BK;
    p.total = B * p.N * rblocks;
    if (p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    p.rblocks = make_fastdiv((uint32_t)rblocks);
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_mfma<E, D, PAIR, MASK, STAGED>), dim3((unsigned)p.total),
                           dim3(kWaves * 64), args, 0, stream);
}

// ---------------------------------------------------------------------------
// dpair.  Workgroup = one (b, h) tile of 16 kZQ queries x 16 kZK keys; its kZW
// waves split the N axis (wave w takes n = w, w + kZW, ...), each computing
// the whole tile per n with scores transposed (S^T = K.Q^T: lane c + 16g
// holds keys 4g + 0..3 of a key tile for query c of a query tile) and
// accumulating dS in registers.  The operands of one n come straight from
// global memory into registers, those of the wave's next n loaded while the
// current one is processed.  The kZW partial sums are then added in wave
// order through LDS, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
constexpr int kZW = 8;  // waves per dpair workgroup
constexpr int kZQ = 2;  // 16-query tiles per dpair workgroup
constexpr int kZK = 2;  // 16-key tiles per dpair workgroup

template <class E, int D, bool MASK>
__global__ __launch_bounds__(kZW * 64, 1) void bwd_dpair_mfma(Params p) {
    using V8 = typename E::v8;
    constexpr int kDC = D / 8;
    constexpr int kDH = (D + 31) / 32;  // 32-wide halves of a row
    constexpr int kAcc = kZQ * kZK * 4;  // accumulators per lane
    __shared__ float red[kZW][kAcc][64];

    // tile order (b, h, query tile, key tile), key tile fastest
    const uint32_t id = (uint32_t)logical_block(blockIdx.x, p.total);
    const uint32_t r1 = fdiv(id, p.nd), r2 = fdiv(r1, p.rblocks), r3 = fdiv(r2, p.hd);
    const int64_t kt0 = id - r1 * p.nd.d;   // nd holds the number of key tiles here
    const int64_t qt0 = r1 - r2 * p.rblocks.d;
    const int64_t h = r2 - r3 * p.hd.d, b = r3;
    const int L = (int)p.L;
    const int64_t N = p.N;
    const Strides& st = p.st;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int i0 = (int)qt0 * 16 * kZQ, j0 = (int)kt0 * 16 * kZK;
    const uint32_t rowq = (uint32_t)st.q[2] * 2, rowk = (uint32_t)st.k[2] * 2, rowv = (uint32_t)st.v[2] * 2;
    const uint32_t rowo = (uint32_t)st.o[2] * 2;
    const uint32_t last = (uint32_t)(L - 1);
    const int64_t pmat = b * st.pb + h * st.ph;  // pair matrix of (b, h)

    // pair bias (base 2) of lane c + 16g: query i0 + 16qt + c, keys j0 + 16kt + 4g + 0..3
    float pb[kZQ][kZK][4];
    {
        const u16* pm = p.pair + pmat;
        for (int qt = 0; qt < kZQ; ++qt)
            for (int kt = 0; kt < kZK; ++kt) {
                const int i = i0 + 16 * qt + c, j = j0 + 16 * kt + 4 * g;
                uint2 w = {0u, 0u};
                if (i < L && j < L) w = load4(pm + (int64_t)i * st.pi + j, L - j);
                const f32x2 a = unpack2<E>(w.x), bb = unpack2<E>(w.y);
                pb[qt][kt][0] = a[0] * kLog2e, pb[qt][kt][1] = a[1] * kLog2e;
                pb[qt][kt][2] = bb[0] * kLog2e, pb[qt][kt][3] = bb[1] * kLog2e;
            }
    }

    struct Ops {
        V8 k[kZK][kDH], v[kZK][kDH], q[kZQ][kDH], d[kZQ][kDH];
        float ls[kZQ], dl[kZQ];
        uint2 mk[kZK];
    };
    auto load = [&](int64_t n) {
        Ops o;
        const Rsrc rk = make_rsrc(p.k + b * st.k[0] + n * st.k[1] + h * st.k[3], last * rowk + D * 2);
        const Rsrc rv = make_rsrc(p.v + b * st.v[0] + n * st.v[1] + h * st.v[3], last * rowv + D * 2);
        const Rsrc rq = make_rsrc(p.q + b * st.q[0] + n * st.q[1] + h * st.q[3], last * rowq + D * 2);
        const Rsrc rd = make_rsrc(p.dout + b * st.o[0] + n * st.o[1] + h * st.o[3], last * rowo + D * 2);
        for (int kt = 0; kt < kZK; ++kt) {
            const uint32_t j = (uint32_t)(j0 + 16 * kt + c);
            for (int hh = 0; hh < kDH; ++hh) {
                const bool in = 4 * hh + g < kDC;
                o.k[kt][hh] = as_v8<E>(bload16(rk, in ? j * rowk + 64u * hh + 16u * g : kOOB, 0));
                o.v[kt][hh] = as_v8<E>(bload16(rv, in ? j * rowv + 64u * hh + 16u * g : kOOB, 0));
            }
            const int jm = j0 + 16 * kt + 4 * g;
            o.mk[kt] = (MASK && jm < L) ? load4(p.mask + b * st.mb + n * st.mn + jm, L - jm) : uint2{0u, 0u};
        }
        for (int qt = 0; qt < kZQ; ++qt) {
            const int i = i0 + 16 * qt + c;
            for (int hh = 0; hh < kDH; ++hh) {
                const bool in = 4 * hh + g < kDC;
                o.q[qt][hh] = as_v8<E>(bload16(rq, in ? (uint32_t)i * rowq + 64u * hh + 16u * g : kOOB, 0));
                o.d[qt][hh] = as_v8<E>(bload16(rd, in ? (uint32_t)i * rowo + 64u * hh + 16u * g : kOOB, 0));
            }
            const int64_t row = ((b * N + n) * p.H + h) * st.lrow + i;
            o.ls[qt] = i < L ? lse_base2(p.lse[row]) : INFINITY;
            o.dl[qt] = i < L ? p.delta[row] : 0.f;
        }
        return o;
    };

    f32x4 acc[kZQ][kZK];
    for (int qt = 0; qt < kZQ; ++qt)
        for (int kt = 0; kt < kZK; ++kt) acc[qt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave < N) {
        Ops cur = load(wave);
        for (int64_t n = wave; n < N; n += kZW) {
            const Ops nxt = load(n + kZW < N ? n + kZW : n);
            for (int kt = 0; kt < kZK; ++kt) {
                float m2[4] = {0.f, 0.f, 0.f, 0.f};
                if (MASK) {
                    const f32x2 a = unpack2<E>(cur.mk[kt].x), bb = unpack2<E>(cur.mk[kt].y);
                    m2[0] = a[0] * kLog2e, m2[1] = a[1] * kLog2e, m2[2] = bb[0] * kLog2e, m2[3] = bb[1] * kLog2e;
                }
                for (int qt = 0; qt < kZQ; ++qt) {
                    const float ndl = -cur.dl[qt];  // dP starts from -delta
                    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f}, dp = f32x4{ndl, ndl, ndl, ndl};
                    for (int hh = 0; hh < kDH; ++hh) {
                        sc = E::mfma(cur.k[kt][hh], cur.q[qt][hh], sc);
                        dp = E::mfma(cur.v[kt][hh], cur.d[qt][hh], dp);
                    }
                    for (int r = 0; r < 4; ++r) {
                        const float x = fmaf(sc[r], p.c1, pb[qt][kt][r]) + (m2[r] - cur.ls[qt]);
                        acc[qt][kt][r] = fmaf(__builtin_amdgcn_exp2f(x), dp[r], acc[qt][kt][r]);
                    }
                }
            }
            cur = nxt;
        }
    }

    // add the waves' partial sums in wave order
    for (int qt = 0; qt < kZQ; ++qt)
        for (int kt = 0; kt < kZK; ++kt)
            for (int r = 0; r < 4; ++r) red[wave][(qt * kZK + kt) * 4 + r][lane] = acc[qt][kt][r];
    __syncthreads();
    if (tid < 64 * kZQ * kZK) {
        const int l = tid & 63, f = tid >> 6, qt = f / kZK, kt = f % kZK;
        float tot[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < kZW; ++w)
            for (int r = 0; r < 4; ++r) tot[r] += red[w][4 * f + r][l];
        const int i = i0 + 16 * qt + (l & 15), j = j0 + 16 * kt + 4 * (l >> 4);
        if (i < L && j < L)
            store4(p.dpair + pmat + (int64_t)i * st.pi + j, uint2{pack2<E>(tot[0], tot[1]), pack2<E>(tot[2], tot[3])},
                   L - j);
    }
}

template <class E, int D, bool MASK>
hipError_t launch_dpair(Params p, int64_t B, hipStream_t stream) {
    const int64_t qtiles = (p.L + 16 * kZQ - 1) / (16 * kZQ), ktiles = (p.L + 16 * kZK - 1) / (16 * kZK);
    p.total = B * p.H * qtiles * ktiles;
    if (p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    p.rblocks = make_fastdiv((uint32_t)qtiles);
    p.nd = make_fastdiv((uint32_t)ktiles);  // the dpair kernel decodes key tiles with this divisor
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dpair_mfma<E, D, MASK>), dim3((unsigned)p.total),
                           dim3(kZW * 64), args, 0, stream);
}

// ---------------------------------------------------------------------------
// dpair with a workspace.  Workgroup = one (b, h) tile of 64 queries x 64 keys
// and one chunk of the N axis; all four waves take the same n at a time, so
// the chunk's Q, dO, K and V rows for the tile are copied into LDS once per n
// and shared (one block ahead, double buffered).  Wave w owns queries 16w ..
// 16w+15 against all 64 keys, scores transposed (lane c + 16g holds keys
// 16kt + 4g + 0..3 of query 16w + c).  Each workgroup writes its chunk's
// partial sum (fp32) to the workspace; bwd_dpair_reduce then adds the chunks
// in chunk order.  LDS per step, with the swizzle of the dq kernel:
//   q, dout, k, v: slot 4*row + (chunk ^ ((row >> 2) & 3)), row of the tile, chunk = 8 d-values
//   mt: the tile's 64 mask values; ls, dl: lse * log2(e) and -delta of the tile's queries
// ---------------------------------------------------------------------------
template <int DH>
struct PairBuf {
    uint4 q[DH][64 * 4];
    uint4 dout[DH][64 * 4];
    uint4 k[DH][64 * 4];
    uint4 v[DH][64 * 4];
    uint4 mt[8];
    float ls[64];
    float dl[64];
};

struct PartParams {
    Params p;
    float* ws;        // [chunks][B][H][L][bwd_ws_row(L)] fp32
    int64_t chunks;   // N is split into this many contiguous ranges
    FastDiv tiles;    // 64 x 64 tiles per (b, h): ceil(L/64)^2
    FastDiv tdim;     // ceil(L/64)
    FastDiv chd;      // chunks
    int64_t bh;       // B * H
};

template <class E, int D, bool MASK, bool STAGED>
__global__ __launch_bounds__(kWaves * 64, 2) void bwd_dpair_part(PartParams pp) {
    using V8 = typename E::v8;
    constexpr int kDC = D / 8;
    constexpr int kDH = (D + 31) / 32;  // 32-wide halves of a row (each its own LDS tile)
    using Buf = PairBuf<kDH>;
    const Params& p = pp.p;
    __shared__ __attribute__((aligned(16))) Buf sm[2];

    // order (b, h, chunk, query tile, key tile): the tiles of one (b, h, chunk)
    // run on one XCD together and share each n's rows in its L2
    const uint32_t id = (uint32_t)logical_block(blockIdx.x, p.total);
    const uint32_t r1 = fdiv(id, pp.tiles), r2 = fdiv(r1, pp.chd), r3 = fdiv(r2, p.hd);
    const uint32_t tile = id - r1 * pp.tiles.d;
    const uint32_t ti = fdiv(tile, pp.tdim), tj = tile - ti * pp.tdim.d;
    const int64_t chunk = r1 - r2 * pp.chd.d, h = r2 - r3 * p.hd.d, b = r3;
    const int L = (int)p.L;
    const int64_t N = p.N;
    const Strides& st = p.st;
    const int64_t n0 = chunk * N / pp.chunks, n1 = (chunk + 1) * N / pp.chunks;
    const int i0 = (int)ti * 64, j0 = (int)tj * 64;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const uint32_t rowq = (uint32_t)st.q[2] * 2, rowk = (uint32_t)st.k[2] * 2, rowv = (uint32_t)st.v[2] * 2;
    const uint32_t rowo = (uint32_t)st.o[2] * 2;
    const uint32_t last = (uint32_t)(L - 1);

    // pair bias of lane c + 16g (query i0 + 16 wave + c, keys j0 + 16kt + 4g
    // + 0..3) times sqrt(D): the accumulator input of every S^T product, so
    // that S^T comes out as q.k + sqrt(D) pair, which the exponent's factor
    // log2(e) / sqrt(D) maps to q.k log2(e) / sqrt(D) + pair log2(e)
    f32x4 pbs[kKT];
    {
        const float sqd = __builtin_sqrtf((float)D);
        const u16* pm = p.pair + b * st.pb + h * st.ph;
        const int i = i0 + 16 * wave + c;
        for (int kt = 0; kt < kKT; ++kt) {
            const int j = j0 + 16 * kt + 4 * g;
            uint2 w = {0u, 0u};
            if (i < L && j < L) w = load4(pm + (int64_t)i * st.pi + j, L - j);
            const f32x2 a = unpack2<E>(w.x), bb = unpack2<E>(w.y);
            pbs[kt] = f32x4{a[0] * sqd, a[1] * sqd, bb[0] * sqd, bb[1] * sqd};
        }
    }

    // copies of step n: rows 16 wave + lane/4 of the tile, chunk (lane & 3) ^ ((lane >> 4) & 3)
    const uint32_t dchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t trow = (uint32_t)(16 * wave + (lane >> 2));
    uint32_t qoff[kDH], dooff[kDH], koff[kDH], voff[kDH];
    for (int hh = 0; hh < kDH; ++hh) {
        const bool din = 4 * hh + (int)dchunk < kDC;
        qoff[hh] = din ? ((uint32_t)i0 + trow) * rowq + 64u * hh + 16u * dchunk : kOOB;
        dooff[hh] = din ? ((uint32_t)i0 + trow) * rowo + 64u * hh + 16u * dchunk : kOOB;
        koff[hh] = din ? ((uint32_t)j0 + trow) * rowk + 64u * hh + 16u * dchunk : kOOB;
        voff[hh] = din ? ((uint32_t)j0 + trow) * rowv + 64u * hh + 16u * dchunk : kOOB;
    }
    float lsv = 0.f, dlv = 0.f;
    uint4 mstage;  // STAGED: the mask chunk between its load and its landing in LDS
    // slices of the sequence copied next (n0 first), advanced by one n per step
    // (no 64-bit product inside the loop)
    const u16* cq = p.q + b * st.q[0] + n0 * st.q[1] + h * st.q[3];
    const u16* cd = p.dout + b * st.o[0] + n0 * st.o[1] + h * st.o[3];
    const u16* ck = p.k + b * st.k[0] + n0 * st.k[1] + h * st.k[3];
    const u16* cv = p.v + b * st.v[0] + n0 * st.v[1] + h * st.v[3];
    const u16* cm = MASK ? p.mask + b * st.mb + n0 * st.mn : p.q;
    const int64_t lstep = p.H * st.lrow;  // lse / delta elements between consecutive n
    const float* clse = p.lse + ((b * N + n0) * p.H + h) * st.lrow;
    const float* cdelta = p.delta + ((b * N + n0) * p.H + h) * st.lrow;
    auto next_step = [&]() {
        cq += st.q[1], cd += st.o[1], ck += st.k[1], cv += st.v[1];
        if (MASK) cm += st.mn;
        clse += lstep, cdelta += lstep;
    };
    // The copies of the step at the cursor: the direct ones (q, dO, k, v and,
    // with aligned rows, the mask chunk) go straight into LDS as untracked
    // copies, waited for by wait_all() before the step's barrier; copy_rest
    // loads the lse / delta rows and (STAGED) the mask chunk into registers.
    auto copy_direct = [&](Buf* __restrict__ dst) {
        const Rsrc rq = make_rsrc(cq, last * rowq + D * 2);
        const Rsrc rd = make_rsrc(cd, last * rowo + D * 2);
        const Rsrc rk = make_rsrc(ck, last * rowk + D * 2);
        const Rsrc rv = make_rsrc(cv, last * rowv + D * 2);
        for (int hh = 0; hh < kDH; ++hh) {
            dma16_untracked(rq, &dst->q[hh][64 * wave], qoff[hh]);
            dma16_untracked(rd, &dst->dout[hh][64 * wave], dooff[hh]);
            dma16_untracked(rk, &dst->k[hh][64 * wave], koff[hh]);
            dma16_untracked(rv, &dst->v[hh][64 * wave], voff[hh]);
        }
        if (MASK && !STAGED && wave == 0 && lane < 8) {
            const Rsrc rm = make_rsrc(cm, bias_range((uint32_t)L * 2u, false));
            dma16_untracked(rm, &dst->mt[0], (uint32_t)j0 * 2u + 16u * lane);
        }
    };
    auto copy_rest = [&]() {
        if (MASK && STAGED && wave == 0 && lane < 8) {
            const Rsrc rm = make_rsrc(cm, bias_range((uint32_t)L * 2u, true));
            mstage = bload16_any(rm, (uint32_t)j0 * 2u + 16u * lane, (uint32_t)L * 2u);
        }
        if (wave == 1) {
            const int i = i0 + lane;
            lsv = i < L ? lse_base2(clse[i]) : INFINITY;
            dlv = i < L ? -cdelta[i] : 0.f;  // negated: the accumulator input of dP
        }
    };
    auto put_rows = [&](Buf* __restrict__ dst) {
        if (wave == 1) {
            dst->ls[lane] = lsv;
            dst->dl[lane] = dlv;
        }
        if (STAGED && MASK && wave == 0 && lane < 8) dst->mt[lane] = mstage;
    };

    f32x4 acc[kKT];
    for (int kt = 0; kt < kKT; ++kt) acc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};

    copy_direct(&sm[0]);
    copy_rest();
    next_step();
    put_rows(&sm[0]);
    wait_all();
    __syncthreads();
    for (int64_t n = n0; n < n1; ++n) {
        const int it = (int)(n - n0);
        const Buf* __restrict__ cur = &sm[it & 1];
        Buf* __restrict__ nxt = &sm[(it & 1) ^ 1];
        // the next step's direct copies first (see the dq kernel); STAGED
        // loads its registers after the step's reads
        if (n + 1 < n1) {
            copy_direct(nxt);
            if (!STAGED) {
                copy_rest();
                next_step();
            }
        }
        const int sw = g ^ ((c >> 2) & 3);
        V8 qop[kDH], dop[kDH], kop[kKT][kDH], vop[kKT][kDH];
        for (int hh = 0; hh < kDH; ++hh) {
            qop[hh] = as_v8<E>(cur->q[hh][64 * wave + 4 * c + sw]);
            dop[hh] = as_v8<E>(cur->dout[hh][64 * wave + 4 * c + sw]);
        }
        uint2 mb[kKT];
        for (int kt = 0; kt < kKT; ++kt) {
            for (int hh = 0; hh < kDH; ++hh) {
                kop[kt][hh] = as_v8<E>(cur->k[hh][64 * kt + 4 * c + sw]);
                vop[kt][hh] = as_v8<E>(cur->v[hh][64 * kt + 4 * c + sw]);
            }
            if (MASK) mb[kt] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(&cur->mt[2 * kt + (g >> 1)]) + 8 * (g & 1));
        }
        const float lsq = cur->ls[16 * wave + c], dlq = cur->dl[16 * wave + c];
        if (STAGED && n + 1 < n1) {
            copy_rest();
            next_step();
        }
        for (int kt = 0; kt < kKT; ++kt) {
            f32x4 sc = pbs[kt], dp = f32x4{dlq, dlq, dlq, dlq};  // -delta: dP - delta comes out
            for (int hh = 0; hh < kDH; ++hh) {
                sc = E::mfma(kop[kt][hh], qop[hh], sc);
                dp = E::mfma(vop[kt][hh], dop[hh], dp);
            }
            float mraw[4] = {0.f, 0.f, 0.f, 0.f};
            if (MASK) {
                const f32x2 a = unpack2<E>(mb[kt].x), bb = unpack2<E>(mb[kt].y);
                mraw[0] = a[0], mraw[1] = a[1], mraw[2] = bb[0], mraw[3] = bb[1];
            }
            for (int r = 0; r < 4; ++r) {
                const float x = fmaf(sc[r], p.c1, MASK ? fmaf(mraw[r], kLog2e, -lsq) : -lsq);
                acc[kt][r] = fmaf(__builtin_amdgcn_exp2f(x), dp[r], acc[kt][r]);
            }
        }
        if (n + 1 < n1) put_rows(nxt);
        wait_all();
        __syncthreads();
    }

    // lane c + 16g: query i0 + 16 wave + c, keys j0 + 16kt + 4g + 0..3
    const int i = i0 + 16 * wave + c;
    if (i < L)
        for (int kt = 0; kt < kKT; ++kt) {
            const int j = j0 + 16 * kt + 4 * g;
            if (j < L)
                *reinterpret_cast<f32x4*>(pp.ws + ((chunk * pp.bh + b * p.H + h) * p.L + i) * bwd_ws_row(p.L) + j) =
                    acc[kt];
        }
}

// dpair[b,h,i,j] = sum over the workspace's chunks of their partial sums, in
// chunk order; four consecutive keys per thread.  The workspace is dense
// [B][H][L][bwd_ws_row(L)]; keys past L are skipped.
struct ReduceParams {
    const float* ws;
    u16* dpair;
    int64_t quads, chunks;  // B*H*L*bwd_ws_row(L) / 4; N-chunks
    int64_t L, H;
    int64_t pb, ph, pi;     // strides of dpair
};

template <class E>
__global__ __launch_bounds__(256) void bwd_dpair_reduce(ReduceParams r) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= r.quads) return;
    f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t ch = 0; ch < r.chunks; ++ch) t += reinterpret_cast<const f32x4*>(r.ws)[ch * r.quads + q];
    const int64_t rq = bwd_ws_row(r.L) / 4, row = q / rq, j = 4 * (q - row * rq);  // row = (b * H + h) * L + i
    if (j >= r.L) return;
    const int64_t bh = row / r.L, i = row - bh * r.L, b = bh / r.H, h = bh - b * r.H;
    store4(r.dpair + b * r.pb + h * r.ph + i * r.pi + j, uint2{pack2<E>(t[0], t[1]), pack2<E>(t[2], t[3])},
           (int)(r.L - j));
}

template <class E, int D, bool MASK, bool STAGED>
hipError_t launch_dpair_ws(const Params& base, int64_t B, float* ws, int64_t chunks, hipStream_t stream) {
    PartParams pp;
    pp.p = base;
    const int64_t tdim = (base.L + 63) / 64;
    pp.p.total = B * base.H * chunks * tdim * tdim;
    if (pp.p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    pp.ws = ws;
    pp.chunks = chunks;
    pp.tiles = make_fastdiv((uint32_t)(tdim * tdim));
    pp.tdim = make_fastdiv((uint32_t)tdim);
    pp.chd = make_fastdiv((uint32_t)chunks);
    pp.bh = B * base.H;
    void* args[] = {&pp};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dpair_part<E, D, MASK, STAGED>),
                                   dim3((unsigned)pp.p.total), dim3(kWaves * 64), args, 0, stream);
    if (e != hipSuccess) return e;
    ReduceParams r;
    r.ws = ws;
    r.dpair = base.dpair;
    r.quads = B * base.H * base.L * bwd_ws_row(base.L) / 4;
    r.chunks = chunks;
    r.L = base.L;
    r.H = base.H;
    r.pb = base.st.pb, r.ph = base.st.ph, r.pi = base.st.pi;
    const int64_t blocks = (r.quads + 255) / 256;
    if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    void* rargs[] = {&r};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dpair_reduce<E>), dim3((unsigned)blocks), dim3(256),
                           rargs, 0, stream);
}

template <class E, int D, bool PAIR, bool MASK, bool STAGED>
hipError_t launch_dq(Params& p, int64_t B, hipStream_t stream) {
    const int64_t rblocks = (p.L + kBlockRows - 1) / kBlockRows;
    p.total = B * p.N * p.H * rblocks;
    if (p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    p.rblocks = make_fastdiv((uint32_t)rblocks);
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_mfma<E, D, PAIR, MASK, STAGED>), dim3((unsigned)p.total),
                           dim3(kWaves * 64), args, 0, stream);
}

template <class E, int D>
hipError_t launch_dim(const BwdArgs& a, unsigned stages, hipStream_t stream) {
    Params p;
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.mask = static_cast<const u16*>(a.mask);
    p.pair = static_cast<const u16*>(a.pair);
    p.out = static_cast<const u16*>(a.out);
    p.dout = static_cast<const u16*>(a.dout);
    p.lse = a.lse;
    p.dq = static_cast<u16*>(a.dq);
    p.dk = static_cast<u16*>(a.dk);
    p.dv = static_cast<u16*>(a.dv);
    p.dmask = static_cast<u16*>(a.dmask);
    p.dpair = static_cast<u16*>(a.dpair);
    p.delta = a.delta;
    p.N = a.N;
    p.L = a.L;
    p.H = a.H;
    p.nd = make_fastdiv((uint32_t)a.N);
    p.hd = make_fastdiv((uint32_t)a.H);
    p.c1 = (float)(1.4426950408889634 / std::sqrt((double)D));
    p.scale = (float)(1.0 / std::sqrt((double)D));
    p.st = a.st;
    const bool pair = a.pair != nullptr, mask = a.mask != nullptr;
    // bias rows copied in 16-byte pieces straight into LDS need rows that
    // start 16-byte aligned (any L); other rows are staged through registers
    const Strides& s = a.st;
    const bool staged = (pair && (s.pb % 8 || s.ph % 8 || s.pi % 8)) || (mask && (s.mb % 8 || s.mn % 8));
    hipError_t e = hipSuccess;
    if (stages & kStageDq) {
        if (staged) {
            if (pair && mask) e = launch_dq<E, D, true, true, true>(p, a.B, stream);
            else if (pair) e = launch_dq<E, D, true, false, true>(p, a.B, stream);
            else if (mask) e = launch_dq<E, D, false, true, true>(p, a.B, stream);
            else e = launch_dq<E, D, false, false, true>(p, a.B, stream);
        } else {
            if (pair && mask) e = launch_dq<E, D, true, true, false>(p, a.B, stream);
            else if (pair) e = launch_dq<E, D, true, false, false>(p, a.B, stream);
            else if (mask) e = launch_dq<E, D, false, true, false>(p, a.B, stream);
            else e = launch_dq<E, D, false, false, false>(p, a.B, stream);
        }
    }
    if (e == hipSuccess && (stages & kStageDkDv)) {
        // the dk/dv kernel reads the mask per key, so only the pair tile is staged
        if (pair && mask) e = staged ? launch_dkdv<E, D, true, true, true>(p, a.B, stream)
                                     : launch_dkdv<E, D, true, true, false>(p, a.B, stream);
        else if (pair) e = staged ? launch_dkdv<E, D, true, false, true>(p, a.B, stream)
                                  : launch_dkdv<E, D, true, false, false>(p, a.B, stream);
        else if (mask) e = launch_dkdv<E, D, false, true, false>(p, a.B, stream);
        else e = launch_dkdv<E, D, false, false, false>(p, a.B, stream);
    }
    if (e == hipSuccess && (stages & kStageDpair) && a.dpair) {
        if (a.ws && a.ws_chunks >= 1) {
            if (mask) e = staged ? launch_dpair_ws<E, D, true, true>(p, a.B, a.ws, a.ws_chunks, stream)
                                 : launch_dpair_ws<E, D, true, false>(p, a.B, a.ws, a.ws_chunks, stream);
            else e = launch_dpair_ws<E, D, false, false>(p, a.B, a.ws, a.ws_chunks, stream);
        } else {
            e = mask ? launch_dpair<E, D, true>(p, a.B, stream) : launch_dpair<E, D, false>(p, a.B, stream);
        }
    }
    return e;
}

template <class E>
hipError_t launch_format(const BwdArgs& a, unsigned stages, hipStream_t stream) {
    switch (a.D) {
    case 8: return launch_dim<E, 8>(a, stages, stream);
    case 16: return launch_dim<E, 16>(a, stages, stream);
    case 32: return launch_dim<E, 32>(a, stages, stream);
    case 64: return launch_dim<E, 64>(a, stages, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

const unsigned kBwdMfmaStages = kStageDq | kStageDkDv | kStageDpair;

int64_t bwd_dpair_chunks(int64_t B, int64_t N, int64_t L, int64_t H) {
    // The split kernels run about four workgroups per CU at once, so a launch
    // proceeds in rounds of 1,024; a workgroup's time is its number of n.
    // Take the split into at least two chunks of at least 8 values of n that
    // minimises rounds x n per workgroup, the smallest such one (fewer partial
    // sums to add): a mostly empty last round costs as much as a full one.
    // (A single chunk would run the single-pass kernel, which is slower.)
    constexpr int64_t kSlots = 1024, kMaxChunks = 4096;
    const int64_t tdim = (L + 63) / 64;
    if (B > (int64_t(1) << 40) / H || B * H > (int64_t(1) << 40) / (tdim * tdim)) return 0;  // no split
    const int64_t tiles = B * H * tdim * tdim;  // below 2^40: tiles * c stays in range
    const int64_t cmax = N / 8 < kMaxChunks ? N / 8 : kMaxChunks;
    int64_t best = 0;
    double best_cost = 0.0;
    for (int64_t c = 2; c <= cmax; ++c) {
        const double cost = (double)((tiles * c + kSlots - 1) / kSlots) * (double)((N + c - 1) / c);
        if (best == 0 || cost < best_cost) best = c, best_cost = cost;
    }
    return best;
}

namespace {

// Rows of one tensor, `row` elements apart with `head` elements between heads,
// as the matrix-core kernels address them: one buffer per sequence covering
// every head, 32-bit byte offsets.  The last element ends below 2^31, rows up
// to 128 past L stay below 2^32, and each row spans every head, so that rows
// past L fall beyond the buffer and read as zero.
bool rows_fit32(int64_t L, int64_t H, int64_t D, int64_t row, int64_t head) {
    constexpr int64_t kMax = int64_t(1) << 31, kLim = int64_t(1) << 40;
    if (row < 0 || head < 0 || row >= kLim || head >= kLim || L >= kLim || H >= kLim) return false;
    if (row < (H - 1) * head + D) return false;
    const int64_t end = ((L - 1) * row + (H - 1) * head + D) * 2, past = ((L + 128) * row + (H - 1) * head) * 2;
    return end < kMax && past < 2 * kMax;
}

}  // namespace

bool bwd_mfma_eligible(const BwdArgs& a, int dtype) {
    constexpr int64_t kMax = int64_t(1) << 31;
    const Strides& s = a.st;
    const int64_t L = a.L, H = a.H, D = a.D;
    if (!(dtype == 1 || dtype == 2) || !(D == 8 || D == 16 || D == 32 || D == 64) || a.N >= kMax || H >= kMax)
        return false;
    for (const int64_t* t : {s.q, s.k, s.v, s.o})
        if (t[2] % 8 || t[3] % 8 || !rows_fit32(L, H, D, t[2], t[3])) return false;
    // pair rows at least L apart (the C ABI checks); unaligned bias rows are
    // staged through registers
    if (a.pair && !rows_fit32(L, 1, L, s.pi, 0)) return false;
    return true;
}

hipError_t launch_bwd_mfma(const BwdArgs& a, int dtype, unsigned stages, hipStream_t stream) {
    return dtype == 2 ? launch_format<F16Fmt>(a, stages, stream) : launch_format<Bf16Fmt>(a, stages, stream);
}

}  // namespace evo
