// 16-bit (bf16, f16) forward kernel on gfx950 (MI355X): head dimensions 8, 16,
// 32 and 64.
//
// Operation (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
// hmyw.cn, sections 4, 5.2 and 5.4): for each (b, n, h) slice and query i,
//   out_i = softmax_j(q_i.k_j / sqrt(D) + mask[b,n,j] + pair[b,h,i,j]) . V,
//   lse_i = ln sum_j exp(...),
// with the [L, L] score matrix never written to memory.
//
// Design (CDNA4, wave64, v_mfma_f32_16x16x32_bf16 with fp32 accumulation):
//  * Scores are formed transposed, S^T = K . Q^T: the MFMA result puts one
//    query per lane column (lane c + 16g holds query c and keys 4g..4g+3 of a
//    16-key tile), so each query's softmax state lives in its own 4 lanes, and
//    those lanes' probabilities are exactly the B operand of the second MFMA,
//    O^T = V^T . P^T, whose result again has one query per lane column.
//  * The biases are added by the matrix cores too: an MFMA with an identity
//    A operand and the bias rows as B operand adds sqrt(D) * bias to the
//    accumulator before Q.K^T is accumulated on top.  sqrt(D) is split into a
//    bf16 high part and a bf16 low part (the two halves of the 32-wide
//    contraction), so the addition is exact to ~2^-16 relative and the biases
//    are consumed in their stored bf16 form.  Accumulator units are
//    "sqrt(D) * score"; one fma maps them to the base-2 exponent.  A bias of
//    +-inf would turn the identity's zeros into NaN, so -inf in the mask is
//    first clamped to a finite value whose weight is still exactly zero (see
//    clamp_neg_inf_bf16 / clamp_neg_inf_f16); any other infinity (+inf, or
//    -inf in the pair bias) makes a NaN row, and a workgroup that sees one
//    re-runs its slice on an exact VALU path.
//  * Online softmax with a lazy maximum.  The item's first block takes its
//    row maximum before the exponentials; every later block first uses the
//    running maximum as it stands and checks the block's row sums, which
//    bound each of their terms: only when a row sum exceeds 2^12 is the
//    maximum raised (O and l rescaled) and the block redone.  The common
//    block thus needs neither a max reduction nor cross-lane traffic, and
//    probabilities stay below 2^12.  The row sums are formed on the matrix
//    cores (an all-ones A operand against the same bf16 P that the P.V
//    product uses), so every lane of a query ends with the full row sum.
//  * D = 64 runs as two 32-wide halves: two products per score tile over the
//    two halves of Q and K, and four 16-wide output tiles; K and V sit in LDS
//    as two 32-wide half tiles in the D = 32 layout.
//  * Per block of 64 keys the workgroup copies K, V, the 128 x 64 pair-bias
//    tile of its queries and the mask row straight from global memory into
//    LDS (buffer loads with the LDS destination bit, no register staging),
//    one block ahead, double buffered, one barrier per block.  Every copy is
//    a full-line, 1 KB wave request; the LDS layouts are XOR-swizzled through
//    the choice of source address per lane so that the operand reads hit
//    distinct banks.  V stays [key][d] in LDS and is read with the
//    transposing ds_read_b64_tr_b16.
//  * Buffer resources (SGPR base + byte range) give 32-bit offsets and return
//    zeros past the range, so rows and keys beyond L need no compares except
//    the -inf assignment in the last, partial block.
//
// Workgroup = 4 wavefronts x 32 queries = 128 queries of one (b, n, h).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "evo_attn_launch.h"
#include "gfx950_common.h"

namespace evo {
namespace {

using namespace gfx;

constexpr int kWaves = 4;
constexpr int kQTiles = 2;                // 16-query MFMA tiles per wavefront
constexpr int kWaveQ = 16 * kQTiles;      // 32 queries per wavefront
constexpr int kBlockQ = kWaves * kWaveQ;  // 128 queries per workgroup
constexpr int kKB = 64;                   // keys per block
constexpr int kKT = kKB / 16;             // 16-key tiles per block
constexpr float kLazyLimit = 4096.f;      // bound of a block's row sum, and so of every probability

struct Params {
    const u16* q;
    const u16* k;
    const u16* v;
    const u16* mask;  // nullable
    const u16* pair;  // nullable
    u16* out;
    float* lse;       // nullable
    int64_t N, L, H;
    FastDiv qblocks;  // ceil(L / kBlockQ)
    FastDiv nd, hd;   // N, H
    int64_t total;    // number of workgroups, below 2^31
    Strides st;       // element strides of every tensor
    float c1;         // log2(e) / sqrt(D): accumulator units -> base-2 exponent
    uint32_t sqd;     // bf16 bits: low half = sqrt(D) high part, high half = low part
};

// LDS of the fast path, in 16-byte slots; DH = 32-wide halves of the head
// dimension (1, or 2 for D = 64).
//   k, v: half hh, slot 4*key + (chunk ^ ((key >> 2) & 3)), chunk = 8 d-values of the half
//   pt:   slot 8*row + (chunk ^ (row & 7)), row = query of the workgroup, chunk = 8 keys
//   mt:   slot chunk (8 keys)
template <int DH>
struct FastBuf {
    uint4 k[DH][kKB * 4];
    uint4 v[DH][kKB * 4];
    uint4 pt[kBlockQ * 8];
    uint4 mt[8];
};
template <int DH>
struct FastSmem {
    FastBuf<DH> buf[2];
};

// LDS of the exact path.
// The exact path also serves D = 64 (two 32-wide halves of the contraction).
constexpr int kExactMaxD = 64;
constexpr int kKStride = kExactMaxD + 8;  // row of K (one key), 16-bit elements
constexpr int kVtStride = kKB + 8;        // row of transposed V (one d), 16-bit elements
struct ExactSmem {
    u16 k[kKB * kKStride];
    u16 vt[kExactMaxD * kVtStride];
};

template <int DH>
union Smem {
    FastSmem<DH> f;
    ExactSmem e;
};

// binary16 cannot hold a large finite negative mask value: such masks come
// as -inf, which an identity product would turn into NaN (0 * inf).  They
// enter the product as the most negative finite value instead, whose
// weight exp2(-65504 * sqrt(D) * c1) is an exact 0 in fp32.  NaN stays NaN.
__device__ inline uint4 clamp_neg_inf_f16(uint4 x) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 lo = {(_Float16)-65504.0f, (_Float16)-65504.0f};
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
    for (int i = 0; i < 4; ++i)
        w[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_bit_cast(h2, w[i]), lo));
    return uint4{w[0], w[1], w[2], w[3]};
}

// bfloat16 masks of -inf stay on the fast path too.  Taken as unsigned
// 16-bit integers, -inf (0xff80) and the NaNs with the sign bit set
// (0xff81..0xffff) are the only patterns above the most negative finite value
// (0xff7f, -3.39e38), so one packed unsigned minimum per dword turns -inf into
// that value.  Its product with the identity weight (sqrt(D) >= 2.8 in its
// high part) overflows to -inf in fp32: the key takes exactly zero weight
// with no NaN, and a row whose every key is -inf ends with a zero row sum,
// which sends it to the exact path (out = 0, lse = -inf).  The negative NaNs
// the minimum would also turn into -inf are caught beforehand by
// any_neg_nan_bf16, so NaN still reaches the exact path.
__device__ inline uint4 clamp_neg_inf_bf16(uint4 x) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const us2 floor2 = {0xff7fu, 0xff7fu};
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
    for (int i = 0; i < 4; ++i)
        w[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(us2, w[i]), floor2));
    return uint4{w[0], w[1], w[2], w[3]};
}

// Whether one of the first n bfloat16 values of x is a NaN with the sign bit
// set (0xff81..0xffff).
__device__ inline bool any_neg_nan_bf16(uint4 x, int n) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    bool any = false;
    for (int i = 0; i < 4; ++i)
        any |= (2 * i < n && (w[i] & 0xffffu) > 0xff80u) || (2 * i + 1 < n && (w[i] >> 16) > 0xff80u);
    return any;
}

// The same for all 8 values (the whole chunk lies below L): one packed
// unsigned maximum over the chunk, then its two halves against 0xff80.
__device__ inline bool any_neg_nan_bf16_all(uint4 x) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    const us2 m = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_bit_cast(us2, x.x), __builtin_bit_cast(us2, x.y)),
        __builtin_elementwise_max(__builtin_bit_cast(us2, x.z), __builtin_bit_cast(us2, x.w)));
    return m[0] > 0xff80u || m[1] > 0xff80u;
}

// Whether one of the first n 16-bit values of x is other than -inf in
// binary16 (0xfc00).
__device__ inline bool any_not_neg_inf_f16(uint4 x, int n) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    bool any = false;
    for (int i = 0; i < 4; ++i)
        any |= (2 * i < n && (w[i] & 0xffffu) != 0xfc00u) || (2 * i + 1 < n && (w[i] >> 16) != 0xfc00u);
    return any;
}

__device__ inline uint4 load16(const u16* p) { return *reinterpret_cast<const uint4*>(p); }


struct Slice {
    int64_t b, n, h, q0;
    int64_t qb, kb, vb, ob;         // element offsets of (b, n, 0, h, 0) in q, k, v, out
    int64_t ql, kl, vl, ol, pi;     // row strides (elements) of q, k, v, out and the pair matrix
    const u16* mrow;   // mask row of (b, n) or nullptr
    const u16* pbase;  // pair matrix of (b, h) or nullptr
    float* lrow;       // lse row of (b, n, h) or nullptr
};

// ---------------------------------------------------------------------------
// Fast path.  Returns false (for the whole workgroup) when some row sum ended
// outside [2^-8, inf) (a bias of +-inf, or a row whose keys all carry one
// huge finite bias); nothing has been written in that case.
// Requires L * H * D * 2 < 2^31 and L * L * 2 < 2^31.  STAGED: the bias rows
// are not 16-byte aligned (bias strides not multiples of 8 elements); their
// tiles then go global -> registers -> LDS, with unaligned 16-byte loads,
// instead of straight into LDS.
// ---------------------------------------------------------------------------
template <class E, int D, bool PAIR, bool MASK, bool STAGED>
__device__ bool run_fast(const Params& p, const Slice& s, FastSmem<(D + 31) / 32>& sm, int tid) {
    using V8 = typename E::v8;
    using Buf = FastBuf<(D + 31) / 32>;
    // D < 32: the 16-byte chunks of a row past D read as zero (an offset
    // beyond the buffer range), which pads Q and K with zero dimensions and V
    // with zero columns; the d-tile of P.V past D is skipped.
    constexpr int kDC = D / 8;               // 16-byte chunks per row
    constexpr int kDH = (D + 31) / 32;       // 32-wide halves of the contraction over d
    constexpr int kDHT = (D + 15) / 16;      // 16-wide d tiles of the output
    const int L = (int)p.L;
    // the wave index is uniform: keep it (and every LDS address derived from
    // it, such as the copies' destinations) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int nblocks = (L + kKB - 1) / kKB;
    // bytes between consecutive rows of q, k, v and the pair matrix; every
    // row span is below kOOB (the launcher checks)
    const uint32_t rowq = (uint32_t)s.ql * 2, rowk = (uint32_t)s.kl * 2, rowv = (uint32_t)s.vl * 2;
    const uint32_t rowp = (uint32_t)s.pi * 2;
    const Rsrc rq = make_rsrc(p.q + s.qb, (uint32_t)(L - 1) * rowq + D * 2);
    const Rsrc rk = make_rsrc(p.k + s.kb, (uint32_t)(L - 1) * rowk + D * 2);
    const Rsrc rv = make_rsrc(p.v + s.vb, (uint32_t)(L - 1) * rowv + D * 2);
    // Bias buffers.  Direct copies (aligned rows): the range ends at the
    // 16-byte boundary after the last element, so that the last row's final
    // chunk is read whole even when L % 8 != 0 (its elements past the row are
    // keys past L; that granule lies in the page of the last element).
    // STAGED: the exact range, which the element-wise reads at its end need.
    const uint32_t pbytes = (uint32_t)(L - 1) * rowp + (uint32_t)L * 2u, mbytes = (uint32_t)L * 2u;
    const Rsrc rp = make_rsrc(PAIR ? s.pbase : p.q, PAIR ? (STAGED ? pbytes : (pbytes + 15u) & ~15u) : 0u);
    const Rsrc rm = make_rsrc(MASK ? s.mrow : p.q, MASK ? (STAGED ? mbytes : (mbytes + 15u) & ~15u) : 0u);

    // Identity A operand: slot (g, e) stands for key 8*(g%2) + e of a 16-key
    // tile, weighted by the high (g < 2) or low (g >= 2) part of sqrt(D).
    V8 ident;
    {
        const u16 wt = (u16)(g < 2 ? (p.sqd & 0xffffu) : (p.sqd >> 16));
        uint32_t w[4];
        for (int e2 = 0; e2 < 4; ++e2) {
            const int e = 2 * e2;
            const uint32_t lo = (c == 8 * (g & 1) + e) ? wt : 0u;
            const uint32_t hi = (c == 8 * (g & 1) + e + 1) ? wt : 0u;
            w[e2] = lo | (hi << 16);
        }
        ident = as_v8<E>(uint4{w[0], w[1], w[2], w[3]});
    }

    // Q operands (B of S^T = K.Q^T): lane (c + 16g) holds q[query c][32hh + 8g
    // .. 32hh + 8g + 7] for half hh; rows past L read as zero.
    V8 qop[kQTiles][kDH];
    for (int t = 0; t < kQTiles; ++t) {
        const uint32_t i = (uint32_t)(s.q0 + 16 * t + c);
        for (int hh = 0; hh < kDH; ++hh)
            qop[t][hh] = as_v8<E>(bload16(rq, 4 * hh + g < kDC ? i * rowq + 64 * hh + 16 * g : kOOB, 0));
    }

    // ---- copy of one block (keys [64 blk, 64 blk + 64)) into LDS buffer `buf` ----
    // K, V: wave w fills slots 64w .. 64w+63 of each half (keys 16w .. 16w+15);
    //   lane l holds key 16w + l/4 at slot position l%4, i.e. chunk (l%4) ^ ((key >> 2) & 3).
    // pair: wave w fills 1 KB segments 4w .. 4w+3; segment I holds query rows
    //   8I .. 8I+7, lane l row 8I + l/8 at position l%8, chunk (l%8) ^ (row & 7).
    //   Query rows past L fall outside the pair range and read as zero.
    // mask: wave 0 lanes 0..7, 8 keys each.
    const uint32_t qwg = (uint32_t)(s.q0 - wave * kWaveQ);  // first query of the workgroup
    const uint32_t kvchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t krow = (uint32_t)(16 * wave + (lane >> 2));
    uint32_t ko[kDH], vo[kDH];
    for (int hh = 0; hh < kDH; ++hh) {
        const bool in = 4 * hh + (int)kvchunk < kDC;
        ko[hh] = in ? krow * rowk + 64u * hh + 16u * kvchunk : kOOB;
        vo[hh] = in ? krow * rowv + 64u * hh + 16u * kvchunk : kOOB;
    }
    uint32_t pvo[4];
    for (int j = 0; j < 4; ++j) {
        const uint32_t row = 8u * (4 * wave + j) + (lane >> 3);
        // rows past L start beyond the range (the pair row stride is at least L)
        pvo[j] = (qwg + row) * rowp + 16u * ((lane & 7) ^ (lane >> 3));
    }
    // STAGED: the pair and mask chunks in flight between a block's copy and
    // its landing in LDS
    uint4 pstage[4], mstage;
    const uint32_t prange = PAIR ? pbytes : 0u;
    // K and V always go straight into LDS, as untracked copies (the compiler
    // would otherwise make every later LDS read, of the other buffer too,
    // wait for them); wait_all() at the end of the step waits for them
    // before the barrier.  The bias tiles go straight into LDS the same way,
    // or (STAGED) through registers.
    auto copy_kv = [&](int blk, Buf* __restrict__ dst) {
        const uint32_t k0 = (uint32_t)blk * kKB;
        for (int hh = 0; hh < kDH; ++hh) {
            dma16_untracked(rk, &dst->k[hh][64 * wave], ko[hh] + k0 * rowk);
            dma16_untracked(rv, &dst->v[hh][64 * wave], vo[hh] + k0 * rowv);
        }
    };
    auto copy_bias = [&](int blk, Buf* __restrict__ dst) {
        const uint32_t k0 = (uint32_t)blk * kKB;
        if (STAGED) {
            if (PAIR)
                for (int j = 0; j < 4; ++j) pstage[j] = bload16_any(rp, pvo[j] + k0 * 2u, prange);
            if (MASK && wave == 0 && lane < 8) mstage = bload16_any(rm, 16u * lane + k0 * 2u, mbytes);
        } else {
            if (PAIR)
                for (int j = 0; j < 4; ++j) dma16_untracked(rp, &dst->pt[64 * (4 * wave + j)], pvo[j] + k0 * 2u);
            if (MASK && wave == 0 && lane < 8) dma16_untracked(rm, &dst->mt[0], 16u * lane + k0 * 2u);
        }
    };
    // STAGED: the staged chunks into the slots the direct copies would fill
    auto land_block = [&](Buf* __restrict__ dst) {
        if (!STAGED) return;
        if (PAIR)
            for (int j = 0; j < 4; ++j) dst->pt[64 * (4 * wave + j) + lane] = pstage[j];
        if (MASK && wave == 0 && lane < 8) dst->mt[lane] = mstage;
    };

    f32x4 oacc[kQTiles][kDHT];
    float mused[kQTiles], msub[kQTiles], lsum[kQTiles];
    for (int t = 0; t < kQTiles; ++t) {
        for (int dh = 0; dh < kDHT; ++dh) oacc[t][dh] = f32x4{0.f, 0.f, 0.f, 0.f};
        mused[t] = -INFINITY;
        msub[t] = 0.f;
        lsum[t] = 0.f;
    }
    const V8 ones8 = as_v8<E>(uint4{E::kOnes2, E::kOnes2, E::kOnes2, E::kOnes2});  // 1.0

    // binary16 with a mask: every key of the sequence masked by -inf so far
    bool all_neg_inf = E::kF16 && MASK;
    // bfloat16 with a mask: a mask NaN with the sign bit set was seen
    bool mask_neg_nan = false;

    copy_kv(0, &sm.buf[0]);
    copy_bias(0, &sm.buf[0]);
    land_block(&sm.buf[0]);
    wait_all();
    __syncthreads();

    // S^T = sqrt(D)*(pair + mask) + K.Q^T for the block in `b`, in accumulator
    // units; MASKON adds the mask (only blocks whose mask has a nonzero entry).
    auto scores = [&](const Buf* __restrict__ b, f32x4 (&acc)[kQTiles][kKT], auto mask_tag) {
        constexpr bool MASKON = decltype(mask_tag)::value;
        // every operand first, then the products in three independent waves
        // of eight, so that no product waits for the one just issued
        V8 kop[kKT][kDH], pop[kQTiles][kKT], mop[kKT];
        for (int kt = 0; kt < kKT; ++kt) {
            // A[m = key][k = d]: lane (c + 16g) reads key 16kt + c, chunk g of each half
            for (int hh = 0; hh < kDH; ++hh) kop[kt][hh] = as_v8<E>(b->k[hh][64 * kt + 4 * c + (g ^ ((c >> 2) & 3))]);
            if (PAIR)
                for (int t = 0; t < kQTiles; ++t) {
                    // B[k = slot][n = query]: pair row of query c, keys 16kt + 8(g%2) .. +7
                    const int row = wave * kWaveQ + 16 * t + c;
                    pop[t][kt] = as_v8<E>(b->pt[8 * row + ((2 * kt + (g & 1)) ^ (c & 7))]);
                }
            if (MASKON) {
                uint4 m = b->mt[2 * kt + (g & 1)];
                m = E::kF16 ? clamp_neg_inf_f16(m) : clamp_neg_inf_bf16(m);
                mop[kt] = as_v8<E>(m);
            }
        }
        for (int kt = 0; kt < kKT; ++kt)
            for (int t = 0; t < kQTiles; ++t) acc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (PAIR)
            for (int kt = 0; kt < kKT; ++kt)
                for (int t = 0; t < kQTiles; ++t) acc[t][kt] = E::mfma(ident, pop[t][kt], acc[t][kt]);
        if (MASKON)
            for (int kt = 0; kt < kKT; ++kt)
                for (int t = 0; t < kQTiles; ++t) acc[t][kt] = E::mfma(ident, mop[kt], acc[t][kt]);
        for (int hh = 0; hh < kDH; ++hh)
            for (int kt = 0; kt < kKT; ++kt)
                for (int t = 0; t < kQTiles; ++t) acc[t][kt] = E::mfma(kop[kt][hh], qop[t][hh], acc[t][kt]);
    };

    // One block of keys; TAIL marks the last block when L % 64 != 0.  The
    // next block's direct copies are issued first (see below); with STAGED
    // the bias loads into registers come after the block's LDS reads, whose
    // registers they reuse.
    auto step = [&](int it, const Buf* __restrict__ cur, Buf* __restrict__ nxt, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const int k0 = it * kKB;

        // The next block's copies go first: the other buffer's readers all
        // passed the barrier that ended the previous step, and the copies
        // then have the whole step to land.  (STAGED: the bias loads into
        // registers keep their place below, where their registers are free.)
        if (it + 1 < nblocks) {
            copy_kv(it + 1, nxt);
            if (!STAGED) copy_bias(it + 1, nxt);
        }
        f32x4 acc[kQTiles][kKT];
        bool mask_on = false;
        if (MASK) {
            const uint4 mw = cur->mt[lane & 7];
            mask_on = wave_any((mw.x | mw.y | mw.z | mw.w) != 0);
            // binary16: remember whether any key so far escaped a -inf mask
            // (keys past L read as zero or as the next row and do not count)
            if (E::kF16)
                all_neg_inf = all_neg_inf && mask_on &&
                              !wave_any(any_not_neg_inf_f16(mw, L - k0 - 8 * (lane & 7)));
            else if (mask_on) {
                // a chunk that ends past L (only in the last block) needs the element-wise test
                const int nk = L - k0 - 8 * (lane & 7);
                bool nn;
                if (wave_any(nk < 8)) nn = any_neg_nan_bf16(mw, nk);
                else nn = any_neg_nan_bf16_all(mw);
                mask_neg_nan = mask_neg_nan || wave_any(nn);
            }
        }
        if (mask_on) scores(cur, acc, std::true_type{});
        else scores(cur, acc, std::false_type{});

        // V operands of O^T = V^T . P^T.  A[m = d][k]: lane (c + 16g) needs
        // V[key(g, e)][16dh + c].  Lane r of group g addresses key 32cc + 4g +
        // r/4, d-values 16dh + 4(r%4) .. +3 (16-byte chunk 2dh + (r%4)/2 of
        // the half, byte half r%2); the transposing read then hands lane c the
        // column 16dh + c over keys 32cc + 4g + 0..3, and a second read does
        // keys 32cc + 16 + 4g + 0..3.
        V8 vop[2][kDHT];
        for (int cc = 0; cc < 2; ++cc)
            for (int dh = 0; dh < kDHT; ++dh) {
                const int key = 32 * cc + 4 * g + (c >> 2);          // (key >> 2) & 3 == g
                const int chunk = (2 * (dh & 1) + ((c & 3) >> 1)) ^ g;
                const char* base = reinterpret_cast<const char*>(&cur->v[dh >> 1][4 * key + chunk]) + 8 * (c & 1);
                const uint2 lo = ds_read_tr(base);
                const uint2 hi = ds_read_tr(base + 16 * 4 * 16);      // 16 keys further
                vop[cc][dh] = as_v8<E>(uint4{lo.x, lo.y, hi.x, hi.y});
            }

        if (STAGED && it + 1 < nblocks) copy_bias(it + 1, nxt);  // lands while this block is processed

        if (TAIL)  // keys past L take no weight
            for (int kt = 0; kt < kKT; ++kt)
                for (int r = 0; r < 4; ++r)
                    if (k0 + 16 * kt + 4 * g + r >= L)
                        for (int t = 0; t < kQTiles; ++t) acc[t][kt][r] = -INFINITY;

        // ---- online softmax with a lazily raised maximum ----
        // The item's first block takes its maximum before the exponentials.
        // Later blocks use the running maximum as it stands, and the block's
        // row sum bounds each of its terms: when no row sum exceeds
        // kLazyLimit, no probability does either and the block is accepted;
        // else the maximum is raised and the block redone.
        V8 pmat[kQTiles][2];
        float bs[kQTiles];
        auto probs = [&]() {
            for (int t = 0; t < kQTiles; ++t) {
                uint32_t w[8];
                for (int kt = 0; kt < kKT; ++kt) {
                    float e[4];
                    for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(acc[t][kt][r], p.c1, -msub[t]));
                    w[2 * kt] = pack2<E>(e[0], e[1]);
                    w[2 * kt + 1] = pack2<E>(e[2], e[3]);
                }
                // B operand of O^T = V^T.P^T: element e of 32-key chunk cc is key 32cc + 16(e/4) + 4g + e%4
                pmat[t][0] = as_v8<E>(uint4{w[0], w[1], w[2], w[3]});
                pmat[t][1] = as_v8<E>(uint4{w[4], w[5], w[6], w[7]});
                // the block's row sum over the same bf16 probabilities, on the
                // matrix cores (an all-ones A operand): every lane of query c
                // receives the sum over all 64 keys
                const f32x4 sum4 = E::mfma(ones8, pmat[t][1], E::mfma(ones8, pmat[t][0], f32x4{0.f, 0.f, 0.f, 0.f}));
                bs[t] = sum4[0];
            }
        };
        auto raise_max = [&]() {
            for (int t = 0; t < kQTiles; ++t) {
                float m = acc[t][0][0];
                for (int kt = 0; kt < kKT; ++kt)
                    for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[t][kt][r]);
                const float mnew = fmaxf(mused[t], max_over_groups(m));
                if (mnew > mused[t]) {
                    const float alpha = __builtin_amdgcn_exp2f((mused[t] - mnew) * p.c1);  // 0 when mused = -inf
                    lsum[t] *= alpha;
                    for (int dh = 0; dh < kDHT; ++dh) oacc[t][dh] *= alpha;
                    mused[t] = mnew;
                    msub[t] = mnew * p.c1;
                }
            }
        };
        if (it == 0) {
            raise_max();
            probs();
        } else {
            probs();
            bool over = false;
            for (int t = 0; t < kQTiles; ++t) over |= !(bs[t] <= kLazyLimit);  // NaN counts as over
            if (wave_any(over)) {
                raise_max();
                probs();
            }
        }
        for (int t = 0; t < kQTiles; ++t) lsum[t] += bs[t];

        // ---- O^T += V^T . P^T ----
        for (int cc = 0; cc < 2; ++cc)
            for (int dh = 0; dh < kDHT; ++dh)
                for (int t = 0; t < kQTiles; ++t) oacc[t][dh] = E::mfma(vop[cc][dh], pmat[t][cc], oacc[t][dh]);

        if (it + 1 < nblocks) land_block(nxt);
        wait_all();  // the next block's copies have landed
        __syncthreads();
    };
    for (int it = 0; it + 1 < nblocks; ++it) step(it, &sm.buf[it & 1], &sm.buf[(it & 1) ^ 1], std::false_type{});
    {
        const int it = nblocks - 1;
        if (L % kKB) step(it, &sm.buf[it & 1], &sm.buf[(it & 1) ^ 1], std::true_type{});
        else step(it, &sm.buf[it & 1], &sm.buf[(it & 1) ^ 1], std::false_type{});
    }

    // ---- epilogue: normalise, write O (bf16) and LSE (fp32, natural log) ----
    float lt[kQTiles];
    bool bad = false;
    for (int t = 0; t < kQTiles; ++t) {
        lt[t] = lsum[t];  // every lane of query c holds the full row sum
        // The key that sets the running maximum adds exp2 of the rounding
        // error of msub, about 1, so a sound row sum lies in [2^-8, inf).
        // Outside it: NaN (an infinite bias), or a row whose largest score
        // is so large in magnitude (a huge finite bias on every key) that
        // this rounding error itself under- or overflows the exponential.
        bad |= !(lt[t] >= 0x1p-8f && lt[t] < INFINITY);
    }
    // a sequence whose keys are all masked by -inf: the exact path returns
    // out = 0 and lse = -inf for it
    bad |= all_neg_inf || mask_neg_nan;
    if (__syncthreads_or(bad)) return false;
    for (int t = 0; t < kQTiles; ++t) {
        const int64_t i = s.q0 + 16 * t + c;
        if (i >= L) continue;
        const float inv = lt[t] > 0.f ? 1.f / lt[t] : 0.f;
        for (int dh = 0; dh < kDHT; ++dh) {
            // lane (c + 16g) holds O^T[d = 16dh + 4g + r][query c], r = 0..3
            if (16 * dh + 4 * g >= D) continue;
            u16* dst = p.out + s.ob + i * s.ol + 16 * dh + 4 * g;
            const f32x4 o = oacc[t][dh] * inv;
            *reinterpret_cast<uint2*>(dst) = uint2{pack2<E>(o[0], o[1]), pack2<E>(o[2], o[3])};
        }
        if (s.lrow && g == 0) s.lrow[i] = lt[t] > 0.f ? (msub[t] + __log2f(lt[t])) * kLn2 : -INFINITY;
    }
    return true;
}

// ---------------------------------------------------------------------------
// Exact path: biases are widened and added on the vector ALUs in base-2
// units (-inf stays -inf), every access is bounds-checked, any L works.  Used
// for biases holding +-inf.  Same lane layout as the fast
// path; K and transposed V are staged through LDS with two barriers per block.
// ---------------------------------------------------------------------------
template <class E, int D>
__device__ void run_exact(const Params& p, const Slice& s, ExactSmem& sm, int tid) {
    using V8 = typename E::v8;
    constexpr int kDHT = (D + 15) / 16;  // 16-wide d tiles of the output; dimensions past D are zero
    constexpr int kDH = (D + 31) / 32;   // 32-wide halves of the contraction over d
    const int64_t L = p.L;
    const int lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;

    V8 qop[kQTiles][kDH];
    for (int t = 0; t < kQTiles; ++t) {
        int64_t i = s.q0 + 16 * t + c;
        if (i >= L) i = L - 1;
        for (int hh = 0; hh < kDH; ++hh) {
            const int d0 = 32 * hh + 8 * g;
            qop[t][hh] = as_v8<E>(d0 < D ? load16(p.q + s.qb + i * s.ql + d0) : uint4{0u, 0u, 0u, 0u});
        }
    }
    f32x4 oacc[kQTiles][kDHT];
    float mrun[kQTiles], lrun[kQTiles];
    for (int t = 0; t < kQTiles; ++t) {
        for (int dh = 0; dh < kDHT; ++dh) oacc[t][dh] = f32x4{0.f, 0.f, 0.f, 0.f};
        mrun[t] = -INFINITY;
        lrun[t] = 0.f;
    }
    const float cq = p.c1;  // log2(e)/sqrt(D)
    const int skey = tid >> 2, sdc = (tid & 3) * 8;

    for (int64_t k0 = 0; k0 < L; k0 += kKB) {
        // each thread stages kDH 16-byte chunks of one key row: d-values 32 hh + sdc .. +7
        uint4 kk[kDH], vv[kDH];
        for (int hh = 0; hh < kDH; ++hh) {
            kk[hh] = vv[hh] = uint4{0u, 0u, 0u, 0u};
            if (k0 + skey < L && 32 * hh + sdc < D) {
                kk[hh] = load16(p.k + s.kb + (k0 + skey) * s.kl + 32 * hh + sdc);
                vv[hh] = load16(p.v + s.vb + (k0 + skey) * s.vl + 32 * hh + sdc);
            }
        }
        __syncthreads();  // previous block's readers are done
        for (int hh = 0; hh < kDH; ++hh) {
            *reinterpret_cast<uint4*>(&sm.k[skey * kKStride + 32 * hh + sdc]) = kk[hh];
            const uint32_t w[4] = {vv[hh].x, vv[hh].y, vv[hh].z, vv[hh].w};
            for (int e = 0; e < 8; ++e)
                sm.vt[(32 * hh + sdc + e) * kVtStride + skey] = (u16)(w[e / 2] >> (16 * (e % 2)));
        }
        __syncthreads();

        f32x4 acc[kQTiles][kKT];
        for (int kt = 0; kt < kKT; ++kt) {
            for (int t = 0; t < kQTiles; ++t) acc[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int hh = 0; hh < kDH; ++hh) {
                const V8 kop =
                    as_v8<E>(*reinterpret_cast<const uint4*>(&sm.k[(16 * kt + c) * kKStride + 32 * hh + 8 * g]));
                for (int t = 0; t < kQTiles; ++t) acc[t][kt] = E::mfma(kop, qop[t][hh], acc[t][kt]);
            }
        }
        for (int kt = 0; kt < kKT; ++kt) {
            const int64_t jb = k0 + 16 * kt + 4 * g;
            for (int t = 0; t < kQTiles; ++t) {
                int64_t i = s.q0 + 16 * t + c;
                if (i >= L) i = L - 1;
                for (int rr = 0; rr < 4; ++rr) {
                    const int64_t j = jb + rr;
                    float bias = 0.f;
                    if (s.mrow && j < L) bias += E::widen(s.mrow[j]);
                    if (s.pbase && j < L) bias += E::widen(s.pbase[i * s.pi + j]);
                    acc[t][kt][rr] = j < L ? fmaf(acc[t][kt][rr], cq, bias * kLog2e) : -INFINITY;
                }
            }
        }
        V8 pmat[kQTiles][2];
        for (int t = 0; t < kQTiles; ++t) {
            float mx = -INFINITY;
            for (int kt = 0; kt < kKT; ++kt)
                for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, acc[t][kt][rr]);
            const float mnew = fmaxf(mrun[t], max_over_groups(mx));
            const float ms = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrun[t] - ms);
            float ls = 0.f;
            for (int kt = 0; kt < kKT; ++kt)
                for (int rr = 0; rr < 4; ++rr) {
                    const float e = __builtin_amdgcn_exp2f(acc[t][kt][rr] - ms);
                    acc[t][kt][rr] = e;
                    ls += e;
                }
            lrun[t] = lrun[t] * alpha + ls;
            mrun[t] = mnew;
            for (int dh = 0; dh < kDHT; ++dh) oacc[t][dh] *= alpha;
            for (int cc = 0; cc < 2; ++cc) {
                const f32x4 a = acc[t][2 * cc], b = acc[t][2 * cc + 1];
                pmat[t][cc] = as_v8<E>(uint4{pack2<E>(a[0], a[1]), pack2<E>(a[2], a[3]), pack2<E>(b[0], b[1]), pack2<E>(b[2], b[3])});
            }
        }
        for (int cc = 0; cc < 2; ++cc)
            for (int dh = 0; dh < kDHT; ++dh) {
                const u16* row = &sm.vt[(16 * dh + c) * kVtStride + 32 * cc + 4 * g];
                const uint2 lo = *reinterpret_cast<const uint2*>(row);
                const uint2 hi = *reinterpret_cast<const uint2*>(row + 16);
                const V8 vop = as_v8<E>(uint4{lo.x, lo.y, hi.x, hi.y});
                for (int t = 0; t < kQTiles; ++t) oacc[t][dh] = E::mfma(vop, pmat[t][cc], oacc[t][dh]);
            }
    }
    for (int t = 0; t < kQTiles; ++t) {
        const float l = sum_over_groups(lrun[t]);
        const int64_t i = s.q0 + 16 * t + c;
        if (i >= L) continue;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        for (int dh = 0; dh < kDHT; ++dh) {
            if (16 * dh + 4 * g >= D) continue;
            u16* dst = p.out + s.ob + i * s.ol + 16 * dh + 4 * g;
            const f32x4 o = oacc[t][dh] * inv;
            *reinterpret_cast<uint2*>(dst) = uint2{pack2<E>(o[0], o[1]), pack2<E>(o[2], o[3])};
        }
        // a row sum of 0 (every key -inf) gives lse = -inf; a NaN one (a NaN bias) stays NaN
        if (s.lrow && g == 0) s.lrow[i] = l > 0.f ? (mrun[t] + __log2f(l)) * kLn2 : (l == 0.f ? -INFINITY : l);
    }
}

// STAGED: the fast path copies the bias tiles through registers.  D <= 32: three workgroups' LDS fit on a CU, and the second
// launch bound keeps the registers within what three waves per SIMD allow
// (168 VGPRs).  D = 64: two workgroups per CU (64 KB of LDS each), 256 VGPRs.
template <class E, int D, bool PAIR, bool MASK, bool STAGED>
__global__ __launch_bounds__(kWaves * 64, D > 32 ? 2 : 3) void fwd_16bit_kernel(Params p) {
    __shared__ __attribute__((aligned(16))) Smem<(D + 31) / 32> sm;

    const uint32_t id = (uint32_t)logical_block(blockIdx.x, p.total);
    const uint32_t r1 = fdiv(id, p.qblocks), r2 = fdiv(r1, p.hd), r3 = fdiv(r2, p.nd);
    const int64_t qb = id - r1 * p.qblocks.d;
    Slice s;
    s.h = r1 - r2 * p.hd.d;
    s.n = r2 - r3 * p.nd.d;
    s.b = r3;
    const Strides& st = p.st;
    s.qb = s.b * st.q[0] + s.n * st.q[1] + s.h * st.q[3];
    s.kb = s.b * st.k[0] + s.n * st.k[1] + s.h * st.k[3];
    s.vb = s.b * st.v[0] + s.n * st.v[1] + s.h * st.v[3];
    s.ob = s.b * st.o[0] + s.n * st.o[1] + s.h * st.o[3];
    s.ql = st.q[2], s.kl = st.k[2], s.vl = st.v[2], s.ol = st.o[2], s.pi = st.pi;
    const int tid = threadIdx.x;
    s.q0 = qb * kBlockQ + (tid >> 6) * kWaveQ;
    s.mrow = p.mask ? p.mask + s.b * st.mb + s.n * st.mn : nullptr;
    s.pbase = p.pair ? p.pair + s.b * st.pb + s.h * st.ph : nullptr;
    s.lrow = p.lse ? p.lse + ((s.b * p.N + s.n) * p.H + s.h) * st.lrow : nullptr;

    if (run_fast<E, D, PAIR, MASK, STAGED>(p, s, sm.f, tid)) return;
    __syncthreads();
    run_exact<E, D>(p, s, sm.e, tid);
}

template <class E, int D, bool PAIR, bool MASK, bool STAGED>
hipError_t launch_variant(Params& p, hipStream_t stream) {
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_16bit_kernel<E, D, PAIR, MASK, STAGED>),
                           dim3((unsigned)p.total), dim3(kWaves * 64), args, 0, stream);
}

// The direct copies of bias rows into LDS need rows that start 16-byte
// aligned (bias strides multiples of 8 elements; the tensors themselves are
// 16-byte aligned), for any L; other rows are staged through registers.  A
// caller with L % 8 != 0 gets the direct copies by passing biases whose rows
// are padded to a multiple of 8 elements.
template <class E, int D, bool PAIR, bool MASK>
hipError_t launch_biases(Params& p, hipStream_t stream) {
    const bool aligned = (!PAIR || (p.st.pb % 8 == 0 && p.st.ph % 8 == 0 && p.st.pi % 8 == 0)) &&
                         (!MASK || (p.st.mb % 8 == 0 && p.st.mn % 8 == 0));
    return aligned ? launch_variant<E, D, PAIR, MASK, false>(p, stream)
                   : launch_variant<E, D, PAIR, MASK, true>(p, stream);
}

template <class E, int D>
hipError_t launch_dim(Params& p, hipStream_t stream) {
    const bool pair = p.pair != nullptr, mask = p.mask != nullptr;
    if (pair && mask) return launch_biases<E, D, true, true>(p, stream);
    if (pair) return launch_biases<E, D, true, false>(p, stream);
    if (mask) return launch_biases<E, D, false, true>(p, stream);
    return launch_biases<E, D, false, false>(p, stream);
}

template <class E>
hipError_t launch_format(Params& p, int64_t d, hipStream_t stream) {
    if (d == 8) return launch_dim<E, 8>(p, stream);
    if (d == 16) return launch_dim<E, 16>(p, stream);
    if (d == 64) return launch_dim<E, 64>(p, stream);
    return launch_dim<E, 32>(p, stream);
}

// x rounded to nearest even in the 16-bit format, as bits
uint16_t bits16_rne(double x, bool f16) {
    if (f16) return __builtin_bit_cast(uint16_t, (_Float16)x);
    const float f = (float)x;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

double widen16(uint16_t b, bool f16) {
    if (f16) return (double)__builtin_bit_cast(_Float16, b);
    const uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

hipError_t launch_fwd_16bit(const FwdArgs& a, hipStream_t stream, bool f16) {
    Params p;
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.mask = static_cast<const u16*>(a.mask);
    p.pair = static_cast<const u16*>(a.pair);
    p.out = static_cast<u16*>(a.out);
    p.lse = a.lse;
    p.st = a.st;
    p.N = a.N;
    p.L = a.L;
    p.H = a.H;
    const int64_t qblocks = (a.L + kBlockQ - 1) / kBlockQ;
    p.total = a.B * a.N * a.H * qblocks;
    if (p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    p.qblocks = make_fastdiv((uint32_t)qblocks);
    p.nd = make_fastdiv((uint32_t)a.N);
    p.hd = make_fastdiv((uint32_t)a.H);
    if (a.D != 8 && a.D != 16 && a.D != 32 && a.D != 64) return hipErrorInvalidValue;
    const double sqd = std::sqrt((double)a.D);
    p.c1 = (float)(1.4426950408889634 / sqd);
    const uint16_t hi = bits16_rne(sqd, f16);
    const uint16_t lo = bits16_rne(sqd - widen16(hi, f16), f16);
    p.sqd = (uint32_t)hi | ((uint32_t)lo << 16);
    return f16 ? launch_format<F16Fmt>(p, a.D, stream) : launch_format<Bf16Fmt>(p, a.D, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) { return launch_fwd_16bit(a, stream, false); }

hipError_t launch_fwd_f16(const FwdArgs& a, hipStream_t stream) { return launch_fwd_16bit(a, stream, true); }

}  // namespace evo
