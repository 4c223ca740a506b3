// Triangle multiplication on the matrix cores (bf16 / f16, fp32 accumulation).
//
// The cubic contraction of the triangle multiplicative update, per channel
// (page "Accelerated molecular modeling with NVIDIA cuEquivariance and NVIDIA
// NIM microservices", open-lab.net, the triangle-operations section names
// it beside triangle attention as the O(N^3) hot spot; the two orientations
// are the plain reading of a product through the third node):
//   outgoing:  x[b,c,i,j] = sum_k a[b,c,i,k] w[b,c,j,k]      (X = A . W^T)
//   incoming:  x[b,c,i,j] = sum_k a[b,c,k,i] w[b,c,k,j]      (X = A^T . W)
// a, w, x are [B, C, L, L]; every (b, c) plane is an independent L x L x L
// matrix product.
//
// Design (v_mfma_f32_16x16x32_{bf16,f16}, wave64):
//  * The product is formed transposed, X^T tile = W-side operand (rows j) x
//    A-side operand (columns i): a 16x16 result leaves j = 4g + 0..3 and
//    i = c in lane c + 16g, so every lane stores 4 consecutive j of one row i
//    (8 bytes).
//  * Workgroup = 8 waves, a 128 x 128 tile of one plane (wave w: j rows
//    64(w%2) .., i columns 32(w/2) ..; 4 x 2 MFMA tiles, 32 accumulators),
//    two workgroups per CU.  Four waves with 64 x 64 each measured 6 % slower:
//    the steps are latency-bound and more waves hide more of it.
//    The result leaves through LDS so that every store is a 16-byte piece of
//    a whole 128-byte row segment, written non-temporally.
//    The contraction runs over k in steps of 64; both operand tiles of a
//    step are copied from global memory straight into LDS one step ahead
//    (double buffered, one barrier per step).
//  * outgoing: the tiles are [row][k] (rows i or j, 8 chunks of 8 k), read
//    as 16-byte row chunks.  incoming: the tiles are [k][column] (16 chunks
//    of 8 columns), read with the transposing ds_read_b64_tr_b16; both
//    operands put k = 32kc + 16(e/4) + 4g + e%4 in element e of lane group g.
//  * Buffer resources of one plane return zeros for rows past L; chunks of k
//    past L get an offset past the range.
//  * L % 8 != 0: rows are no longer 16-byte aligned, so the operand chunks
//    go global -> registers -> LDS (unaligned 16-byte loads, into the slots
//    the direct copies would fill).  A chunk that starts inside the plane's
//    range and ends past it is read element by element; outgoing chunks that
//    cross k = L have their elements past L cleared (they hold the next
//    row); incoming chunks past column L only feed outputs that are not
//    stored.  The epilogue writes the last partial 8-wide piece of each
//    output row element by element.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "evo_attn_launch.h"
#include "gfx950_common.h"

namespace evo {
namespace {

using namespace gfx;

constexpr int kTile = 128;  // output tile (i and j) per workgroup

// x with its 16-bit elements e >= n cleared
__device__ inline uint4 keep_first(uint4 x, int n) {
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
    for (int i = 0; i < 4; ++i) w[i] &= (2 * i < n ? 0xffffu : 0u) | (2 * i + 1 < n ? 0xffff0000u : 0u);
    return uint4{w[0], w[1], w[2], w[3]};
}

struct TmParams {
    const u16* a;
    const u16* w;
    u16* x;
    int64_t L;
    int64_t tdim;   // ceil(L / 128)
    int64_t total;  // planes * tdim^2
};

// LDS per step: one tile of each operand, 128 x KS 16-bit values each.
//   outgoing, [row][k]: CPR = KS/8 chunks of 8 k per row; slot CPR*row + (chunk ^ swz(row)),
//     swz = row & 7 for KS = 64, (row >> 2) & 3 for KS = 32 (rows sharing a bank group differ in slot)
//   incoming, [k][col]: KS rows of k, 16 chunks of 8 columns; slot 16*k + (chunk ^ 2(k & 7))
template <int KS>
struct TmBuf {
    uint4 a[16 * KS];
    uint4 w[16 * KS];
};

template <int KS>
__device__ inline int tm_swz(int row) {
    return KS == 64 ? (row & 7) : ((row >> 2) & 3);
}

constexpr int kNW = 8;  // waves per workgroup
// Two workgroups per CU (64 KB of LDS each), so the launch bound asks for
// four waves per SIMD (at most 128 VGPRs).
template <class E, bool INCOMING, int KS, bool STAGED>
__global__ __launch_bounds__(64 * kNW, 4) void trimul_kernel(TmParams p) {
    using V8 = typename E::v8;
    constexpr int CPR = KS / 8;              // outgoing: 16-byte chunks per tile row
    constexpr int SEG = KS * 4 / 16 / kNW;   // 1 KB copy segments per wave per operand per step
    constexpr int KC = KS / 32;              // 32-wide contraction chunks per step
    constexpr int NT = 2;                    // 16-wide i tiles per wave (j tiles: 4)
    __shared__ __attribute__((aligned(16))) TmBuf<KS> sm[2];

    const int64_t id = logical_block(blockIdx.x, p.total);
    const int64_t per_plane = p.tdim * p.tdim;
    const int64_t plane = id / per_plane, t = id - plane * per_plane;
    const int i0 = (int)(t % p.tdim) * kTile, j0 = (int)(t / p.tdim) * kTile;
    const int L = (int)p.L;
    const int64_t pbase = plane * p.L * p.L;
    const uint32_t range = (uint32_t)L * (uint32_t)L * 2u;
    const Rsrc ra = make_rsrc(p.a + pbase, range), rw = make_rsrc(p.w + pbase, range);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;  // the wave's j rows 64 wm .., i columns 16 NT wn ..
    const int nsteps = (L + KS - 1) / KS;

    // per-lane copy offsets of step 0 (k0 added per step); segment s = SEG wave + q
    uint32_t offa[SEG], offw[SEG];
    int kofs[SEG];  // outgoing: k of this lane's chunk within the step
    for (int q = 0; q < SEG; ++q) {
        const int seg = SEG * wave + q;
        if (!INCOMING) {
            const int row = seg * (64 / CPR) + lane / CPR;
            const int chunk = (lane % CPR) ^ tm_swz<KS>(row);
            kofs[q] = 8 * chunk;
            offa[q] = (uint32_t)(i0 + row) * (uint32_t)L * 2u + 16u * chunk;
            offw[q] = (uint32_t)(j0 + row) * (uint32_t)L * 2u + 16u * chunk;
        } else {
            const int kr = 4 * seg + (lane >> 4);
            const int chunk = (lane & 15) ^ (2 * (kr & 7));
            kofs[q] = 0;
            offa[q] = (uint32_t)kr * (uint32_t)L * 2u + (uint32_t)i0 * 2u + 16u * chunk;
            offw[q] = (uint32_t)kr * (uint32_t)L * 2u + (uint32_t)j0 * 2u + 16u * chunk;
        }
    }
    uint4 sa[SEG], sw[SEG];  // STAGED: chunks between their load and their landing in LDS
    auto copy_step = [&](int st, TmBuf<KS>* __restrict__ dst) {
        const int k0 = st * KS;
        for (int q = 0; q < SEG; ++q) {
            uint32_t oa, ow;
            if (!INCOMING) {
                const bool in = k0 + kofs[q] < L;  // chunks of k past L read zero
                oa = in ? offa[q] + (uint32_t)k0 * 2u : kOOB;
                ow = in ? offw[q] + (uint32_t)k0 * 2u : kOOB;
            } else {
                oa = offa[q] + (uint32_t)k0 * (uint32_t)L * 2u;  // k rows past L start beyond the range
                ow = offw[q] + (uint32_t)k0 * (uint32_t)L * 2u;
            }
            if (!STAGED) {  // untracked: waited for by wait_all() before the step's barrier
                dma16_untracked(ra, &dst->a[64 * (SEG * wave + q)], oa);
                dma16_untracked(rw, &dst->w[64 * (SEG * wave + q)], ow);
            } else {
                sa[q] = bload16_any(ra, oa, range);
                sw[q] = bload16_any(rw, ow, range);
                if (!INCOMING && k0 + KS > L) {  // the step that reaches k = L
                    const int valid = L - (k0 + kofs[q]);
                    if (valid < 8) {
                        sa[q] = keep_first(sa[q], valid);
                        sw[q] = keep_first(sw[q], valid);
                    }
                }
            }
        }
    };
    auto land_step = [&](TmBuf<KS>* __restrict__ dst) {
        if (!STAGED) return;
        for (int q = 0; q < SEG; ++q) {
            dst->a[64 * (SEG * wave + q) + lane] = sa[q];
            dst->w[64 * (SEG * wave + q) + lane] = sw[q];
        }
    };

    f32x4 acc[4][NT];  // [m tile (j)][n tile (i)]
    for (int mt = 0; mt < 4; ++mt)
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    copy_step(0, &sm[0]);
    land_step(&sm[0]);
    wait_all();
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const TmBuf<KS>* __restrict__ cur = &sm[st & 1];
        // direct copies of the next step go first (the other buffer's readers
        // all passed the previous barrier); STAGED loads into registers come
        // after the step's LDS reads, whose registers they reuse
        if (!STAGED && st + 1 < nsteps) copy_step(st + 1, &sm[(st & 1) ^ 1]);
        V8 aop[KC][4], bop[KC][4];  // A operand: w side (rows j); B operand: a side (columns i)
        for (int kc = 0; kc < KC; ++kc)
            for (int q = 0; q < 4; ++q) {
                if (!INCOMING) {
                    const int rj = 64 * wm + 16 * q + c, ri = 16 * NT * wn + 16 * q + c, chunk = 4 * kc + g;
                    aop[kc][q] = as_v8<E>(cur->w[CPR * rj + (chunk ^ tm_swz<KS>(rj))]);
                    if (q < NT) bop[kc][q] = as_v8<E>(cur->a[CPR * ri + (chunk ^ tm_swz<KS>(ri))]);
                } else {
                    // lane c + 16g addresses k row 32kc + 4g + c/4 (and 16 further), columns 4(c%4) .. +3 of
                    // the 16-column group; it receives column c of k rows 32kc + 4g + 0..3 and + 16
                    const int kr = 32 * kc + 4 * g + (c >> 2);
                    const int colj = 64 * wm + 16 * q + 4 * (c & 3), coli = 16 * NT * wn + 16 * q + 4 * (c & 3);
                    const char* bw = reinterpret_cast<const char*>(cur->w);
                    const char* ba = reinterpret_cast<const char*>(cur->a);
                    auto addr = [&](const char* base, int k, int col) {
                        return base + 16 * (16 * k + ((col >> 3) ^ (2 * (k & 7)))) + 2 * (col & 7);
                    };
                    const uint2 wl = ds_read_tr(addr(bw, kr, colj)), wh = ds_read_tr(addr(bw, kr + 16, colj));
                    aop[kc][q] = as_v8<E>(uint4{wl.x, wl.y, wh.x, wh.y});
                    if (q < NT) {
                        const uint2 al = ds_read_tr(addr(ba, kr, coli)), ah = ds_read_tr(addr(ba, kr + 16, coli));
                        bop[kc][q] = as_v8<E>(uint4{al.x, al.y, ah.x, ah.y});
                    }
                }
            }
        if (STAGED && st + 1 < nsteps) copy_step(st + 1, &sm[(st & 1) ^ 1]);
        for (int kc = 0; kc < KC; ++kc)
            for (int mt = 0; mt < 4; ++mt)
                for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = E::mfma(aop[kc][mt], bop[kc][nt], acc[mt][nt]);
        if (st + 1 < nsteps) land_step(&sm[(st & 1) ^ 1]);
        wait_all();
        __syncthreads();
    }

    // Epilogue through LDS: lane c + 16g holds X^T[j = 64 wm + 16 mt + 4g + r][i = 32 wn + 16 nt + c]; each
    // wave writes its 32 (i) x 64 (j) block of x as [i][j] rows (padded to 72 against bank conflicts), then stores
    // whole 128-byte row segments, 16 bytes per lane.  The operand buffers are free (the loop ended with a
    // barrier) and each wave reads back only what it wrote.
    constexpr int kRow = 72;
    static_assert(kNW * 16 * NT * kRow * 2 <= (int)sizeof(sm), "epilogue tile fits the operand buffers");
    u16* tile = reinterpret_cast<u16*>(&sm[0]) + wave * 16 * NT * kRow;
    for (int nt = 0; nt < NT; ++nt)
        for (int mt = 0; mt < 4; ++mt)
            *reinterpret_cast<uint2*>(tile + (16 * nt + c) * kRow + 16 * mt + 4 * g) =
                uint2{pack2<E>(acc[mt][nt][0], acc[mt][nt][1]), pack2<E>(acc[mt][nt][2], acc[mt][nt][3])};
    // x is not read again here: streaming (non-temporal) stores
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const int ib = i0 + 16 * NT * wn, jc = j0 + 64 * wm + 8 * (lane & 7);
    for (int pass = 0; pass < 2 * NT; ++pass) {
        const int row = 8 * pass + (lane >> 3);
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + row * kRow + 8 * (lane & 7));
        if (ib + row < L && jc < L) {
            u16* dst = p.x + pbase + (int64_t)(ib + row) * L + jc;
            if (!STAGED || jc + 8 <= L) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));  // unaligned when STAGED
            } else {
                const u16* e = reinterpret_cast<const u16*>(tile + row * kRow + 8 * (lane & 7));
                for (int q = 0; q < 8; ++q)
                    if (jc + q < L) dst[q] = e[q];
            }
        }
    }
}

constexpr int kKStep = 64;  // contraction step (a 32-wide step with three workgroups per CU measured no faster overall)

template <class E, bool INCOMING>
hipError_t launch(TmParams& p, hipStream_t stream) {
    void* args[] = {&p};
    const void* k = p.L % 8 ? reinterpret_cast<const void*>(&trimul_kernel<E, INCOMING, kKStep, true>)
                            : reinterpret_cast<const void*>(&trimul_kernel<E, INCOMING, kKStep, false>);
    return hipLaunchKernel(k, dim3((unsigned)p.total), dim3(64 * kNW), args, 0, stream);
}

}  // namespace

hipError_t launch_trimul(const void* a, const void* w, void* x, int64_t planes, int64_t L, int incoming, int f16,
                         hipStream_t stream) {
    TmParams p;
    p.a = static_cast<const u16*>(a);
    p.w = static_cast<const u16*>(w);
    p.x = static_cast<u16*>(x);
    p.L = L;
    p.tdim = (L + kTile - 1) / kTile;
    p.total = planes * p.tdim * p.tdim;
    if (p.total >= (int64_t(1) << 31)) return hipErrorInvalidConfiguration;
    if (f16) return incoming ? launch<F16Fmt, true>(p, stream) : launch<F16Fmt, false>(p, stream);
    return incoming ? launch<Bf16Fmt, true>(p, stream) : launch<Bf16Fmt, false>(p, stream);
}

}  // namespace evo
