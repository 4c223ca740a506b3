/*
 * evo_attn.h -- C ABI of the MI355X (gfx950) Evoformer biased-attention
 * library, libevoattn.so: the forward pass and its gradients.
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

#include <stddef.h>
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
    EVO_ERR_NULL_POINTER = 1, /* a required pointer (see each call) is NULL                 */
    EVO_ERR_BAD_SHAPE = 2,    /* a size < 1, or a tensor of more than 2^62 bytes            */
    EVO_ERR_BAD_DTYPE = 3,    /* dtype is not an evo_dtype_t value                          */
    EVO_ERR_MISALIGNED = 4,   /* a tensor pointer is not 16-byte aligned                    */
    EVO_ERR_ALIASING = 5,     /* an output overlaps an input or another output              */
    EVO_ERR_UNSUPPORTED = 6,  /* valid but not implemented (dtype / head dimension)         */
    EVO_ERR_HIP = 7,          /* the HIP runtime reported an error at launch                */
    EVO_ERR_NO_BIAS = 8,      /* evo_attn_bwd: a bias gradient requested for an absent bias  */
    EVO_ERR_SCRATCH = 9       /* evo_attn_bwd_noalloc: not even two chunks of the pair
                                 gradient's partial sums fit the library's static buffer    */
} evo_status_t;

/*
 * Enqueue the forward pass on `stream` (a hipStream_t; NULL = the default
 * stream of the current device).
 *   q, k, v     inputs, [B,N,L,H,D]
 *   mask_bias   [B,N,1,1,L] or NULL (no mask: all zero)
 *   pair_bias   [B,1,H,L,L] or NULL (no pair bias: all zero)
 *   out         output, [B,N,L,H,D], same dtype as q
 *   lse         output, [B,N,H,L] float32, or NULL to skip it
 * Supported today: dtype BF16 or F16 with D in {8, 16, 32, 64} (MFMA path; it
 * addresses one head's rows of a slice and the rows of a pair matrix with
 * 32-bit byte offsets, so it needs (L - 1) * H * D * 2 + 2 D < 2^31 and
 * rows up to L + 128 below 2^32, (L + 128) * H * D * 2 < 2^32, and, when a
 * pair bias is given, (L - 1) * L * 2 + 2 L < 2^31 (L <= 32767) and
 * (L + 128) * L * 2 < 2^32) and dtype F32 with D in {8, 16, 32, 64}; any
 * B, N, H >= 1 and any L >= 1.
 * Other valid combinations return EVO_ERR_UNSUPPORTED.
 * A query row whose every score is -inf gets out = 0 and lse = -inf.  In
 * F16 a large negative mask value such as -1e9 is -inf, which is how such
 * masks arrive in that format; a -inf bias gives its key exactly zero weight.
 */
evo_status_t evo_attn_fwd(const void* q, const void* k, const void* v, const void* mask_bias,
                          const void* pair_bias, void* out, float* lse, const evo_shape_t* shape,
                          evo_dtype_t dtype, void* stream);

/*
 * Element strides of every tensor, for callers whose tensors are views (a
 * transposed pair representation, an MSA tensor read column-wise, a padded
 * LSE).  Section 5.3 of the guide: triangle attention around the ending node
 * and MSA column attention attend along the other axis of the same tensor as
 * their row-wise counterparts; with these strides they read it in place.
 *   q, k, v, out   strides of the b, n, l and h axes of [B,N,L,H,D]; the d
 *                  axis is contiguous (stride 1).  Example: Q of ending-node
 *                  attention as a view of X[B, L_i, L_j, H, D] (n = j, l = i):
 *                  {L*L*H*D, H*D, L*H*D, D}.
 *   mask_b, mask_n strides of mask_bias [B,N,1,1,L]; keys contiguous
 *   pair_b, pair_h, pair_i
 *                  strides of pair_bias [B,1,H,L,L] (pair_i: between query
 *                  rows, >= L); keys contiguous
 *   lse_row        elements between the lse rows of consecutive (b, n, h),
 *                  >= L (the guide's padded layout is ceil(L/32)*32, section 5.4)
 * The strides of q, k, v and out must be multiples of 16 bytes
 * (EVO_ERR_MISALIGNED); every stride must be non-negative (EVO_ERR_BAD_SHAPE);
 * out's strides must give distinct elements distinct addresses
 * (EVO_ERR_ALIASING).  Bias strides may take any value.  Bias rows that start
 * 16-byte aligned (mask and pair strides multiples of 8 elements) are copied
 * straight into on-chip memory, for any L; other rows (such as dense biases
 * with L % 8 != 0) take a slower staged copy.  A caller with L % 8 != 0 can
 * keep the fast copies by padding the bias rows to a multiple of 8 elements:
 * the padding is read (as keys past L, never weighted) but not written, and
 * padding that holds NaN or inf only sends the affected work to the exact
 * path.
 */
typedef struct {
    int64_t q[4], k[4], v[4], out[4];
    int64_t mask_b, mask_n;
    int64_t pair_b, pair_h, pair_i;
    int64_t lse_row;
} evo_layout_t;

/* Fill *layout with the dense layout of *shape (what evo_attn_fwd assumes). */
void evo_attn_dense_layout(const evo_shape_t* shape, evo_layout_t* layout);

/*
 * evo_attn_fwd with explicit strides (see evo_layout_t); every other rule is
 * that of evo_attn_fwd.  Extents for the aliasing check run from each
 * pointer to its tensor's last element.  For bf16 and f16 the row strides of
 * q, k, v and (when given) the pair bias must also keep (L + 128) rows below
 * 2^32 bytes (else EVO_ERR_UNSUPPORTED).
 */
evo_status_t evo_attn_fwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, void* out, float* lse, const evo_layout_t* layout,
                                  const evo_shape_t* shape, evo_dtype_t dtype, void* stream);

/* The validation of evo_attn_fwd_strided alone; host-only. */
evo_status_t evo_attn_check_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                    const void* pair_bias, const void* out, const float* lse,
                                    const evo_layout_t* layout, const evo_shape_t* shape, evo_dtype_t dtype);

/*
 * The validation of evo_attn_fwd alone, with the same arguments minus the
 * stream.  Pure host code: makes no HIP call and never dereferences a tensor
 * pointer, so it also runs on machines without a GPU.
 */
evo_status_t evo_attn_check(const void* q, const void* k, const void* v, const void* mask_bias,
                            const void* pair_bias, const void* out, const float* lse,
                            const evo_shape_t* shape, evo_dtype_t dtype);

/*
 * Enqueue the backward pass on `stream`: the gradients of a scalar loss with
 * respect to q, k, v and, on request, each bias, given dout = d loss / d out.
 * Section 5.4 of the guide describes this pass: it recomputes the attention
 * weights from q, k, the biases and the forward pass's log-sum-exp instead of
 * keeping the [L, L] matrix, uses the per-row quantity delta_i = dout_i . out_i,
 * and computes a bias gradient only when the caller asks for it.  With
 * P_ij = exp(s_ij - lse_i) the forward weights and dS_ij = P_ij (dout_i . v_j
 * - delta_i):
 *   dq_i = sum_j dS_ij k_j / sqrt(D)        dk_j = sum_i dS_ij q_i / sqrt(D)
 *   dv_j = sum_i P_ij dout_i
 *   dmask_bias[b,n,0,0,j] = sum over h and i of dS[b,n,h,i,j]
 *   dpair_bias[b,0,h,i,j] = sum over n of dS[b,n,h,i,j]
 * (each bias gradient summed over the axes along which that bias broadcasts).
 *
 *   q, k, v, mask_bias, pair_bias   the forward pass's inputs, as for evo_attn_fwd
 *   out, lse     the forward pass's outputs for those inputs (evo_attn_fwd with
 *                a non-NULL lse); both required
 *   dout         [B,N,L,H,D] incoming gradient, element type `dtype`
 *   dq, dk, dv   [B,N,L,H,D] outputs, element type `dtype`
 *   dmask_bias   [B,N,1,1,L] output of type `dtype`, or NULL to skip it; only
 *                with a mask_bias (else EVO_ERR_NO_BIAS)
 *   dpair_bias   [B,1,H,L,L] output of type `dtype`, or NULL to skip it (and
 *                its kernel); only with a pair_bias (else EVO_ERR_NO_BIAS)
 *   delta        [B,N,H,L] float32, written with dout_i . out_i (the saved
 *                intermediate of section 5.4); required, owned by the caller
 *   workspace, workspace_bytes
 *                optional device scratch for the pair gradient: the pass may
 *                split the N axis of that sum over more workgroups and keep
 *                the partial sums there (fp32; they are added in a fixed
 *                order, so results stay deterministic).  Query the size with
 *                evo_attn_bwd_workspace_size.  NULL (or fewer bytes than one
 *                split needs) runs the pass without it, more slowly for small
 *                B*H*L^2.  Owned by the caller, contents undefined after the
 *                call; calls that share a workspace must not overlap in time.
 * Every output is overwritten, never accumulated into.  All arithmetic is
 * fp32; results are rounded to nearest-even into `dtype` once, at the end.
 * Sums are formed in a fixed order: the same inputs give bit-identical
 * gradients on every call.  A row with lse = -inf (every key -inf) receives
 * and passes on no gradient.
 * Supported today: every dtype with D in {8, 16, 32, 64} (the guide's limit
 * for this pass is D <= 64), any B, N, H, L >= 1.  Other valid combinations
 * return EVO_ERR_UNSUPPORTED.  Required pointers: q, k, v, out, lse, dout, dq,
 * dk, dv, delta, shape.  Pointer, ownership, alignment, aliasing and error
 * rules are those of evo_attn_fwd; the outputs (dq, dk, dv, dmask_bias,
 * dpair_bias, delta) and the workspace may overlap neither an input nor one
 * another.  workspace_bytes above 2^62 is EVO_ERR_BAD_SHAPE.
 */
evo_status_t evo_attn_bwd(const void* q, const void* k, const void* v, const void* mask_bias,
                          const void* pair_bias, const void* out, const float* lse, const void* dout,
                          void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias, float* delta,
                          void* workspace, size_t workspace_bytes, const evo_shape_t* shape, evo_dtype_t dtype,
                          void* stream);

/*
 * Bytes of workspace with which evo_attn_bwd runs fastest for this shape and
 * dtype (0: it uses none), for the dense layout; a strided call uses as much
 * of it as its layout allows.  Host-only; returns 0 for an invalid shape.
 */
size_t evo_attn_bwd_workspace_size(const evo_shape_t* shape, evo_dtype_t dtype);

/*
 * The validation of evo_attn_bwd alone (same arguments minus the stream).
 * Host-only, like evo_attn_check.
 */
evo_status_t evo_attn_bwd_check(const void* q, const void* k, const void* v, const void* mask_bias,
                                const void* pair_bias, const void* out, const float* lse, const void* dout,
                                const void* dq, const void* dk, const void* dv, const void* dmask_bias,
                                const void* dpair_bias, const float* delta, const void* workspace,
                                size_t workspace_bytes, const evo_shape_t* shape, evo_dtype_t dtype);

/*
 * evo_attn_bwd on strided views (see evo_layout_t): training of ending-node
 * triangle attention and MSA column attention in place, without transposed
 * copies (section 5.3 of the guide).  Every gradient has the layout of the
 * tensor it belongs to: dout and out share layout->out, dq, dk and dv share
 * layout->q, ->k and ->v, dmask_bias shares the mask strides, dpair_bias the
 * pair strides, and delta the lse row stride (rows of layout->lse_row floats,
 * >= L).  Every other rule is that of evo_attn_bwd, plus: q, k, v and out
 * strides multiples of 16 bytes (EVO_ERR_MISALIGNED); each written gradient's
 * strides giving distinct elements distinct addresses, and the extents (first
 * to last element) of outputs, workspace and inputs pairwise disjoint
 * (EVO_ERR_ALIASING).  Layouts the matrix-core kernels cannot address with
 * 32-bit offsets, or whose rows do not span every head, run on the vector-ALU
 * kernels: slower, same results.  Bias rows at any stride stay on the matrix
 * cores.
 */
evo_status_t evo_attn_bwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias, float* delta,
                                  void* workspace, size_t workspace_bytes, const evo_layout_t* layout,
                                  const evo_shape_t* shape, evo_dtype_t dtype, void* stream);

/* The validation of evo_attn_bwd_strided alone; host-only. */
evo_status_t evo_attn_bwd_check_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                        const void* pair_bias, const void* out, const float* lse, const void* dout,
                                        const void* dq, const void* dk, const void* dv, const void* dmask_bias,
                                        const void* dpair_bias, const float* delta, const void* workspace,
                                        size_t workspace_bytes, const evo_layout_t* layout,
                                        const evo_shape_t* shape, evo_dtype_t dtype);

/*
 * Triangle multiplication: the cubic contraction of the triangle
 * multiplicative update, per channel c.  The page "Accelerated molecular
 * modeling with NVIDIA cuEquivariance and NVIDIA NIM microservices"
 * (open-lab.net), in its section on triangle operations, names it with
 * triangle attention as the O(N^3) hot spot of pair-representation models,
 * motivated by transitivity (i near k and k near j relate i and j); the
 * formula below is the plain reading of a product through the third node k,
 * in its two orientations:
 *   EVO_TRIMUL_OUTGOING:  x[b,c,i,j] = sum_k a[b,c,i,k] * w[b,c,j,k]
 *   EVO_TRIMUL_INCOMING:  x[b,c,i,j] = sum_k a[b,c,k,i] * w[b,c,k,j]
 * a, w and x are dense [B, C, L, L] tensors of `dtype` (channel-major: each
 * (b, c) plane is an L x L row-major matrix), device memory owned by the
 * caller; x may overlap neither input.  Products are accumulated in fp32 and
 * x is rounded to nearest-even once.  The layer normalisations, projections
 * and gates around this contraction in a model are O(L^2) per channel and
 * not part of this call.
 * Supported today: BF16 and F16 with L <= 32767 and (L + 128) * L * 2 <
 * 2^32; any B, C >= 1.  Other valid calls return
 * EVO_ERR_UNSUPPORTED.  Errors as for evo_attn_fwd (a bad direction is
 * EVO_ERR_BAD_SHAPE); nothing is written on error.
 */
typedef enum { EVO_TRIMUL_OUTGOING = 0, EVO_TRIMUL_INCOMING = 1 } evo_trimul_direction_t;

typedef struct {
    int64_t B, C, L;
} evo_trimul_shape_t;

evo_status_t evo_trimul(const void* a, const void* w, void* x, const evo_trimul_shape_t* shape,
                        evo_trimul_direction_t direction, evo_dtype_t dtype, void* stream);

/* The validation of evo_trimul alone; host-only. */
evo_status_t evo_trimul_check(const void* a, const void* w, const void* x, const evo_trimul_shape_t* shape,
                              evo_trimul_direction_t direction, evo_dtype_t dtype);

/*
 * evo_attn_bwd without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments are
 * those of evo_attn_bwd; the pair gradient's partial sums go to a static
 * device array of the library instead of a caller workspace, of
 * evo_attn_bwd_noalloc_scratch_bytes() bytes (40 MiB) on every GPU the library
 * runs on, held until the process ends.  The pass splits N into as many of
 * the recommended chunks (evo_attn_bwd_workspace_size) as fit in the array:
 * results are bit-identical to evo_attn_bwd's with the recommended workspace
 * when that fits in 40 MiB, and otherwise to evo_attn_bwd's with a workspace
 * of the largest whole number of chunks that fits.  A shape (with a pair
 * gradient requested) of which not even two chunks fit (B * H * L * L above
 * about 5.2 million) returns EVO_ERR_SCRATCH before anything is enqueued;
 * use evo_attn_bwd with a workspace of your own there.  The call makes no
 * hipMalloc or hipFree; its first call on a device looks up that device's
 * array address (hipGetSymbolAddress).  Calls on one GPU share its array:
 * calls that overlap in time on one GPU race on it.
 */
evo_status_t evo_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias, float* delta,
                                  const evo_shape_t* shape, evo_dtype_t dtype, void* stream);

/* Size in bytes of the static scratch array evo_attn_bwd_noalloc uses on each GPU. */
size_t evo_attn_bwd_noalloc_scratch_bytes(void);

/* The hipError_t (as an int) of the calling thread's last evo_attn_bwd_noalloc
 * failure in its own set-up (the scratch address lookup), or 0. */
int evo_attn_bwd_noalloc_last_hip_error(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* evo_status_string(evo_status_t status);

/*
 * The hipError_t (as an int) that made the calling thread's most recent
 * evo_attn_fwd or evo_attn_bwd return EVO_ERR_HIP, or 0 if none has.  Thread-local; never
 * reset by successful calls.  Lets a caller report the runtime's own reason.
 */
int evo_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EVO_ATTN_H */
