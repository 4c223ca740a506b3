/*
 * evo_attn.h -- C ABI of the MI355X (gfx950) Evoformer biased-attention
 * forward library, libevoattn.so.
 *
 * Operation.  The page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南"
 * (hmyw.cn/news/91637) defines it: section 4 gives the reference attention
 * softmax(Q.K^T * scale + biases) . V, section 5.2 the layouts and the two
 * optional biases, section 5.3 the four Evoformer variants (MSA row, MSA
 * column, triangle attention around the starting and the ending node) that all
 * use this one call, and section 5.4 the per-row log-sum-exp the forward pass
 * keeps for the backward pass.  For every b<B, n<N, h<H and query i<L:
 *
 *   s_j            = (q[b,n,i,h,:] . k[b,n,j,h,:]) / sqrt(D)
 *                    + mask_bias[b,n,0,0,j] + pair_bias[b,0,h,i,j]      (j < L)
 *   out[b,n,i,h,:] = sum_j softmax_j(s) v[b,n,j,h,:]
 *   lse[b,n,h,i]   = ln sum_j exp(s_j)
 *
 * The [L, L] score matrix is never stored.  The scale is fixed at 1/sqrt(D)
 * and applies to Q.K^T only; the biases are added unscaled.
 *
 * Layout.  Every tensor is dense and row-major (last index fastest):
 *   q, k, v, out  [B, N, L, H, D]   element type `dtype`
 *   mask_bias     [B, N, 1, 1, L]   element type `dtype`, broadcast over H and queries
 *   pair_bias     [B, 1, H, L, L]   element type `dtype`, broadcast over N;
 *                                   axis 3 is the query i, axis 4 the key j
 *   lse           [B, N, H, L]      float32, natural log, no padding of L
 * Variants map onto this as in section 5.3: MSA row attention takes N = MSA
 * sequences and L = residues; MSA column attention N = residues, L = sequences
 * and no pair bias; triangle attention N = L = residues.
 *
 * Ownership.  All pointers are device memory on the calling thread's current
 * HIP device, allocated and freed by the caller.  The library allocates
 * nothing, keeps no mutable global state and never synchronises; calls on
 * different streams may run concurrently from several host threads.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued; on
 * failure the call returns an evo_status_t other than EVO_OK and writes
 * nothing.  EVO_OK from evo_attn_fwd means "validated and enqueued"; the
 * kernel then runs asynchronously and a device fault surfaces at the caller's
 * next synchronisation of `stream`.
 */
#ifndef EVO_ATTN_H
#define EVO_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, out and the biases.  bf16 and f16 follow the
 * guide's fp16 / bf16 inputs (sections 3.3 and 5.1); f32 is an addition of
 * this library for full-precision callers. */
typedef enum {
    EVO_DTYPE_F32 = 0,  /* IEEE binary32 */
    EVO_DTYPE_BF16 = 1, /* bfloat16 */
    EVO_DTYPE_F16 = 2   /* IEEE binary16 */
} evo_dtype_t;

/* Problem size.  B batch, N the broadcast axis of the pair bias (MSA
 * sequences, residues or pair rows), L the attended axis (queries = keys),
 * H heads, D head dimension. */
typedef struct {
    int64_t B, N, L, H, D;
} evo_shape_t;

typedef enum {
    EVO_OK = 0,
    EVO_ERR_NULL_POINTER = 1, /* q, k, v, out or shape is NULL                              */
    EVO_ERR_BAD_SHAPE = 2,    /* a size < 1, or a tensor of more than 2^62 bytes            */
    EVO_ERR_BAD_DTYPE = 3,    /* dtype is not an evo_dtype_t value                          */
    EVO_ERR_MISALIGNED = 4,   /* a tensor pointer is not 16-byte aligned                    */
    EVO_ERR_ALIASING = 5,     /* out or lse overlaps an input, or out overlaps lse          */
    EVO_ERR_UNSUPPORTED = 6,  /* valid but not implemented (dtype / head dimension)         */
    EVO_ERR_HIP = 7           /* the HIP runtime reported an error at launch                */
} evo_status_t;

/*
 * Enqueue the forward pass on `stream` (a hipStream_t; NULL = the default
 * stream of the current device).
 *   q, k, v     inputs, [B,N,L,H,D]
 *   mask_bias   [B,N,1,1,L] or NULL (no mask: all zero)
 *   pair_bias   [B,1,H,L,L] or NULL (no pair bias: all zero)
 *   out         output, [B,N,L,H,D], same dtype as q
 *   lse         output, [B,N,H,L] float32, or NULL to skip it
 * Supported today: dtype BF16 or F16 with D in {8, 16, 32} (MFMA path; also
 * needs L * H * D * 2 < 2^31 and L * L * 2 < 2^31, i.e. L <= 32767) and
 * dtype F32 with D in {8, 16, 32, 64}; any B, N, H >= 1 and any L >= 1.
 * Other valid combinations return EVO_ERR_UNSUPPORTED.
 * A query row whose every score is -inf gets out = 0 and lse = -inf.  In
 * F16 a large negative mask value such as -1e9 is -inf, which is how such
 * masks arrive in that format; a -inf bias gives its key exactly zero weight.
 */
evo_status_t evo_attn_fwd(const void* q, const void* k, const void* v, const void* mask_bias,
                          const void* pair_bias, void* out, float* lse, const evo_shape_t* shape,
                          evo_dtype_t dtype, void* stream);

/*
 * The validation of evo_attn_fwd alone, with the same arguments minus the
 * stream.  Pure host code: makes no HIP call and never dereferences a tensor
 * pointer, so it also runs on machines without a GPU.
 */
evo_status_t evo_attn_check(const void* q, const void* k, const void* v, const void* mask_bias,
                            const void* pair_bias, const void* out, const float* lse,
                            const evo_shape_t* shape, evo_dtype_t dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* evo_status_string(evo_status_t status);

/*
 * The hipError_t (as an int) that made the calling thread's most recent
 * evo_attn_fwd return EVO_ERR_HIP, or 0 if none has.  Thread-local; never
 * reset by successful calls.  Lets a caller report the runtime's own reason.
 */
int evo_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EVO_ATTN_H */
