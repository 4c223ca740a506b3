/*
 * evo_ref.c -- fp64 CPU oracle for the Evoformer biased-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header or constant with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [DSG] "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南" (hmyw.cn/news/91637)
 *         S4   -- the reference attention the unit test compares against:
 *                 softmax(Q.K^T * scale + sum of biases) . V
 *         S5.2 -- layouts: Q/K/V are [*, L, Head, Dim] with L the attended
 *                 axis; bias1 (residue mask) is [B, N, 1, 1, L] and broadcasts
 *                 over heads and queries; bias2 (pair bias) is [B, 1, H, L, L]
 *                 and broadcasts over N; masks are additive large negatives.
 *         S5.3 -- the four variants share this single call form.
 *         S5.4 -- the forward pass also emits an fp32 log-sum-exp per row.
 *
 * What is computed (exactly the definition, in fp64, element by element):
 *   for every b<B, n<N, h<H, i<L:
 *     s_j   = (sum_d q[b,n,i,h,d] k[b,n,j,h,d]) / sqrt(D)
 *             + mask[b,n,0,0,j] + pair[b,0,h,i,j]            (j < L)
 *     m     = max_j s_j
 *     Z     = sum_j exp(s_j - m)
 *     out[b,n,i,h,e] = sum_j exp(s_j - m) / Z * v[b,n,j,h,e]
 *     lse[b,n,h,i]   = m + ln Z
 *
 * Readings where the pages leave a step open:
 *   - scale = 1/sqrt(D), D = Q's last dimension; it multiplies Q.K^T only
 *     and the biases are added after it (the '+' of [DSG] S4 was lost in the
 *     page's extraction).
 *   - pair axis 3 is the query i, axis 4 the key j (the softmax axis), as for
 *     the mask whose last axis is the key axis.
 *   - a missing bias (NULL) contributes zero ([DSG] S5.4: a missing bias is
 *     an empty tensor on the same path).
 *   - lse is natural-log, unpadded, laid out [B, N, H, L].
 *   - a row whose every score is -inf has no defined softmax; the oracle
 *     returns out = 0 and lse = -inf for it.
 *
 * Storage formats: dtype 0 = IEEE binary32, 1 = bfloat16 bit patterns
 * (uint16), 2 = IEEE binary16 bit patterns (uint16).  Every stored value is
 * widened to double exactly before any arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_F32 0
#define REF_BF16 1
#define REF_F16 2

/* bfloat16 is the upper half of a binary32: shift the 16 bits into place. */
static double widen_bf16(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double widen_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);            /* subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(frac | 0x400), expo - 25);  /* 1.frac * 2^(e-15) */
    }
    return sign ? -mag : mag;
}

static double load(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
    case REF_F32: return (double)((const float*)base)[idx];
    case REF_BF16: return widen_bf16(((const uint16_t*)base)[idx]);
    default: return widen_f16(((const uint16_t*)base)[idx]);
    }
}

typedef struct {
    const void *q, *k, *v, *mask, *pair;
    int dtype;
    int64_t B, N, L, H, D;
} ref_args;

/* Element offsets of the [B,N,L,H,D], [B,N,1,1,L] and [B,1,H,L,L] layouts. */
static int64_t off_qkv(const ref_args* a, int64_t b, int64_t n, int64_t l, int64_t h, int64_t d) {
    return (((b * a->N + n) * a->L + l) * a->H + h) * a->D + d;
}
static int64_t off_mask(const ref_args* a, int64_t b, int64_t n, int64_t j) {
    return (b * a->N + n) * a->L + j;
}
static int64_t off_pair(const ref_args* a, int64_t b, int64_t h, int64_t i, int64_t j) {
    return ((b * a->H + h) * a->L + i) * a->L + j;
}

/*
 * One output row (b, n, h, i): the definition above, with the slice's K and
 * V already widened to double ([L][D] each).  s is scratch of L doubles.
 * Writes D values to o_row and returns the row's log-sum-exp.
 */
static double ref_row(const ref_args* a, const double* kd, const double* vd,
                      int64_t b, int64_t n, int64_t h, int64_t i,
                      double* s, double* o_row) {
    const int64_t L = a->L, D = a->D;
    const double scale = 1.0 / sqrt((double)D);
    double qrow[1024];  /* D <= 1024 is checked by the callers */
    for (int64_t d = 0; d < D; ++d) qrow[d] = load(a->q, a->dtype, off_qkv(a, b, n, i, h, d));

    /* scores over the key axis j ([DSG] S4, S5.2) */
    double m = -INFINITY;
    for (int64_t j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qrow[d] * kd[j * D + d];
        double sj = dot * scale;
        if (a->mask) sj += load(a->mask, a->dtype, off_mask(a, b, n, j));
        if (a->pair) sj += load(a->pair, a->dtype, off_pair(a, b, h, i, j));
        s[j] = sj;
        if (sj > m) m = sj;
    }
    if (m == -INFINITY) {  /* every key removed: no softmax exists */
        for (int64_t e = 0; e < D; ++e) o_row[e] = 0.0;
        return -INFINITY;
    }
    /* softmax weights, normaliser and weighted sum of value rows */
    double Z = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        s[j] = exp(s[j] - m);
        Z += s[j];
    }
    for (int64_t e = 0; e < D; ++e) o_row[e] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        double w = s[j] / Z;
        for (int64_t e = 0; e < D; ++e) o_row[e] += w * vd[j * D + e];
    }
    return m + log(Z);  /* [DSG] S5.4: natural-log LSE of the row */
}

/* Widen K and V of slice (b, n, h) to double, [L][D] each. */
static void widen_slice(const ref_args* a, int64_t b, int64_t n, int64_t h, double* kd, double* vd) {
    for (int64_t j = 0; j < a->L; ++j)
        for (int64_t d = 0; d < a->D; ++d) {
            int64_t o = off_qkv(a, b, n, j, h, d);
            kd[j * a->D + d] = load(a->k, a->dtype, o);
            vd[j * a->D + d] = load(a->v, a->dtype, o);
        }
}

static int check_args(const ref_args* a) {
    if (!a->q || !a->k || !a->v) return 1;
    if (a->dtype < REF_F32 || a->dtype > REF_F16) return 2;
    if (a->B < 1 || a->N < 1 || a->L < 1 || a->H < 1 || a->D < 1 || a->D > 1024) return 3;
    return 0;
}

/*
 * Full evaluation.  out: [B,N,L,H,D] doubles, lse: [B,N,H,L] doubles (may be
 * NULL).  Slices (b,n,h) are independent and run on nthreads OpenMP threads.
 * Returns 0, or a nonzero code for a NULL input / bad dtype / bad shape, or
 * 4 when scratch memory cannot be allocated.
 */
int evo_ref_fwd(const void* q, const void* k, const void* v, const void* mask, const void* pair,
                int dtype, int64_t B, int64_t N, int64_t L, int64_t H, int64_t D,
                double* out, double* lse, int nthreads) {
    ref_args a = {q, k, v, mask, pair, dtype, B, N, L, H, D};
    int rc = check_args(&a);
    if (rc) return rc;
    if (!out) return 1;
    const int64_t nslices = B * N * H;
    int failed = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* kd = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* vd = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        double o_row[1024];
        const int ok = kd && vd && s;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
        /* every thread reaches the loop (and its closing barrier); one without
         * scratch memory takes no work */
#pragma omp for schedule(dynamic, 1)
        for (int64_t sl = 0; sl < nslices; ++sl) {
            if (!ok) continue;
            {
                int64_t h = sl % H, n = (sl / H) % N, b = sl / (H * N);
                widen_slice(&a, b, n, h, kd, vd);
                for (int64_t i = 0; i < L; ++i) {
                    double r = ref_row(&a, kd, vd, b, n, h, i, s, o_row);
                    for (int64_t e = 0; e < D; ++e) out[off_qkv(&a, b, n, i, h, e)] = o_row[e];
                    if (lse) lse[((b * N + n) * H + h) * L + i] = r;
                }
            }
        }
        free(kd);
        free(vd);
        free(s);
    }
    return failed ? 4 : 0;
}

/*
 * Selected rows only: rows is nrows x 4 int64 (b, n, h, i); out_rows is
 * nrows x D doubles, lse_rows nrows doubles (may be NULL).  Lets the tests
 * check full-size launches on a sample of outputs.  Returns 5 for an index
 * out of range, otherwise as evo_ref_fwd.
 */
int evo_ref_rows(const void* q, const void* k, const void* v, const void* mask, const void* pair,
                 int dtype, int64_t B, int64_t N, int64_t L, int64_t H, int64_t D,
                 const int64_t* rows, int64_t nrows, double* out_rows, double* lse_rows,
                 int nthreads) {
    ref_args a = {q, k, v, mask, pair, dtype, B, N, L, H, D};
    int rc = check_args(&a);
    if (rc) return rc;
    if (!rows || !out_rows) return 1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t* t = rows + 4 * r;
        if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= N || t[2] < 0 || t[2] >= H || t[3] < 0 || t[3] >= L)
            return 5;
    }
    int failed = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* kd = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* vd = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* s = (double*)malloc(sizeof(double) * (size_t)L);
        const int ok = kd && vd && s;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!ok) continue;
            const int64_t* t = rows + 4 * r;
            widen_slice(&a, t[0], t[1], t[2], kd, vd);
            double lr = ref_row(&a, kd, vd, t[0], t[1], t[2], t[3], s, out_rows + r * D);
            if (lse_rows) lse_rows[r] = lr;
        }
        free(kd);
        free(vd);
        free(s);
    }
    return failed ? 4 : 0;
}

/*
 * Backward pass: the gradients of the forward definition above, in fp64.
 *
 * [DSG] S5.4 states that the forward pass keeps the per-row log-sum-exp for
 * a backward pass and that bias gradients are produced only when asked
 * for; the gradients themselves follow from the definition by the chain
 * rule.  With P_ij = exp(s_ij - lse_i) the softmax weights of row i and dO
 * the incoming gradient of out:
 *   dv_j        = sum_i P_ij dO_i
 *   dP_ij       = dO_i . v_j
 *   delta_i     = sum_e dO_ie out_ie            (= sum_j P_ij dP_ij)
 *   dS_ij       = P_ij (dP_ij - delta_i)        (gradient of the score)
 *   dq_i        = sum_j dS_ij k_j / sqrt(D)
 *   dk_j        = sum_i dS_ij q_i / sqrt(D)
 *   dmask[b,n,j]    = sum_{h,i} dS[b,n,h,i,j]   (the mask broadcasts over h and i)
 *   dpair[b,h,i,j]  = sum_n dS[b,n,h,i,j]       (the pair bias broadcasts over n)
 * out and P are recomputed here from the inputs (not taken from a caller),
 * so the oracle depends on nothing the GPU produced.  A row whose every
 * score is -inf has no softmax and contributes nothing.
 *
 * dout has the inputs' storage format.  dq, dk, dv: [B,N,L,H,D] doubles;
 * dmask: [B,N,L] (may be NULL); dpair: [B,H,L,L] (may be NULL).
 */
static void slice_backward(const ref_args* a, const void* dout, int64_t b, int64_t n, int64_t h,
                           const double* kd, const double* vd, double* P, double* dod, double* od,
                           double* dq, double* dk, double* dv, double* dmask_row, double* dpair_bh) {
    const int64_t L = a->L, D = a->D;
    const double scale = 1.0 / sqrt((double)a->D);
    /* P (row-normalised weights) and out of the slice, through the forward's
     * own row evaluation: it leaves exp(s_j - m) in the row of P */
    for (int64_t i = 0; i < L; ++i) {
        double* Pi = P + i * L;
        const double lse_i = ref_row(a, kd, vd, b, n, h, i, Pi, od + i * D);
        if (lse_i == -INFINITY) {
            for (int64_t j = 0; j < L; ++j) Pi[j] = 0.0;
        } else {
            double Z = 0.0;
            for (int64_t j = 0; j < L; ++j) Z += Pi[j];
            for (int64_t j = 0; j < L; ++j) Pi[j] /= Z;
        }
        for (int64_t e = 0; e < D; ++e) dod[i * D + e] = load(dout, a->dtype, off_qkv(a, b, n, i, h, e));
    }
    /* dv, then dS in place of P (after its use for dv), dq, dk and the bias sums */
    for (int64_t j = 0; j < L; ++j)
        for (int64_t e = 0; e < D; ++e) {
            double g = 0.0;
            for (int64_t i = 0; i < L; ++i) g += P[i * L + j] * dod[i * D + e];
            dv[off_qkv(a, b, n, j, h, e)] = g;
        }
    for (int64_t i = 0; i < L; ++i) {
        double delta = 0.0;
        for (int64_t e = 0; e < D; ++e) delta += dod[i * D + e] * od[i * D + e];
        for (int64_t j = 0; j < L; ++j) {
            double dp = 0.0;
            for (int64_t e = 0; e < D; ++e) dp += dod[i * D + e] * vd[j * D + e];
            P[i * L + j] = P[i * L + j] * (dp - delta); /* now dS_ij */
        }
    }
    for (int64_t i = 0; i < L; ++i)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t j = 0; j < L; ++j) g += P[i * L + j] * kd[j * D + d];
            dq[off_qkv(a, b, n, i, h, d)] = g * scale;
        }
    for (int64_t j = 0; j < L; ++j)
        for (int64_t d = 0; d < D; ++d) {
            double g = 0.0;
            for (int64_t r = 0; r < L; ++r) g += P[r * L + j] * load(a->q, a->dtype, off_qkv(a, b, n, r, h, d));
            dk[off_qkv(a, b, n, j, h, d)] = g * scale;
        }
    if (dmask_row)
        for (int64_t j = 0; j < L; ++j) {
            double g = 0.0;
            for (int64_t i = 0; i < L; ++i) g += P[i * L + j];
            dmask_row[j] += g;
        }
    if (dpair_bh)
        for (int64_t i = 0; i < L; ++i)
            for (int64_t j = 0; j < L; ++j) dpair_bh[i * L + j] += P[i * L + j];
}

int evo_ref_bwd(const void* q, const void* k, const void* v, const void* mask, const void* pair, const void* dout,
                int dtype, int64_t B, int64_t N, int64_t L, int64_t H, int64_t D,
                double* dq, double* dk, double* dv, double* dmask, double* dpair, int nthreads) {
    ref_args a = {q, k, v, mask, pair, dtype, B, N, L, H, D};
    int rc = check_args(&a);
    if (rc) return rc;
    if (!dout || !dq || !dk || !dv) return 1;
    if ((dmask && !mask) || (dpair && !pair)) return 1;
    if (dmask) memset(dmask, 0, sizeof(double) * (size_t)(B * N * L));
    if (dpair) memset(dpair, 0, sizeof(double) * (size_t)(B * H * L * L));
    int failed = 0;
    /* (b, n) pairs in parallel: each owns its dq/dk/dv slices and its mask
     * row; the pair-bias gradient, a sum over n, goes through per-thread
     * partial sums added up at the end */
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double* kd = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* vd = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* P = (double*)malloc(sizeof(double) * (size_t)(L * L));
        double* dod = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* od = (double*)malloc(sizeof(double) * (size_t)(L * D));
        double* part = dpair ? (double*)calloc((size_t)(B * H * L * L), sizeof(double)) : NULL;
        const int ok = kd && vd && P && dod && od && (!dpair || part);
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bn = 0; bn < B * N; ++bn) {
            if (!ok) continue;
            const int64_t b = bn / N, n = bn % N;
            for (int64_t h = 0; h < H; ++h) {
                widen_slice(&a, b, n, h, kd, vd);
                slice_backward(&a, dout, b, n, h, kd, vd, P, dod, od, dq, dk, dv,
                               dmask ? dmask + bn * L : NULL, part ? part + (b * H + h) * L * L : NULL);
            }
        }
        /* the loop's closing barrier has passed: every partial is complete */
#pragma omp critical
        if (ok && part)
            for (int64_t e = 0; e < B * H * L * L; ++e) dpair[e] += part[e];
        free(kd);
        free(vd);
        free(P);
        free(dod);
        free(od);
        free(part);
    }
    return failed ? 4 : 0;
}

/*
 * Triangle multiplication: the cubic contraction at the core of the triangle
 * multiplicative update.  [CUEQ] (the cuEquivariance / NIM article, its
 * "accelerating triangle operations" section) names triangle multiplication
 * beside triangle attention as the O(N^3) hot spot of pair-representation
 * models and motivates it by transitivity: when i is near k and k is near j,
 * i and j are related.  Its formula is not printed there; this is the plain
 * reading of "a product through the third node k", per channel c, in the two
 * orientations (edges leaving or entering i and j):
 *   outgoing (direction 0):  x[b,c,i,j] = sum_k a[b,c,i,k] * w[b,c,j,k]
 *   incoming (direction 1):  x[b,c,i,j] = sum_k a[b,c,k,i] * w[b,c,k,j]
 * a, w and x are [B, C, L, L]; the sums are exact products of the widened
 * stored values accumulated in fp64.  x: [B, C, L, L] doubles.
 * Returns 0, 1 for a NULL pointer, 2 for a bad dtype, 3 for a bad shape or
 * direction.
 */
int evo_ref_trimul(const void* a, const void* w, int dtype, int64_t B, int64_t C, int64_t L, int direction,
                   double* x, int nthreads) {
    if (!a || !w || !x) return 1;
    if (dtype < REF_F32 || dtype > REF_F16) return 2;
    if (B < 1 || C < 1 || L < 1 || (direction != 0 && direction != 1)) return 3;
    const int64_t planes = B * C, LL = L * L;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t bc = 0; bc < planes; ++bc) {
        const int64_t base = bc * LL;
        for (int64_t i = 0; i < L; ++i)
            for (int64_t j = 0; j < L; ++j) {
                double sum = 0.0;
                for (int64_t k = 0; k < L; ++k) {
                    const int64_t ia = direction == 0 ? i * L + k : k * L + i;
                    const int64_t iw = direction == 0 ? j * L + k : k * L + j;
                    sum += load(a, dtype, base + ia) * load(w, dtype, base + iw);
                }
                x[base + i * L + j] = sum;
            }
    }
    return 0;
}
