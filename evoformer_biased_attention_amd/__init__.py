"""Python binding of libevoattn.so, the MI355X Evoformer biased-attention library (forward and backward).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/evo_attn.h.  The functions keep
the C names (`evo_attn_fwd`, `evo_attn_bwd`, their `*_check` validators,
`evo_status_string`) and take
either raw device addresses (int) or torch tensors, whose `data_ptr()` is
passed through; PyTorch is used for device memory and streams only.

The library must be built first (`python evoformer_biased_attention_amd/build.py`
or `__graft_entry__.build()`); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libevoattn.so")

EVO_DTYPE_F32, EVO_DTYPE_BF16, EVO_DTYPE_F16 = 0, 1, 2
(EVO_OK, EVO_ERR_NULL_POINTER, EVO_ERR_BAD_SHAPE, EVO_ERR_BAD_DTYPE, EVO_ERR_MISALIGNED, EVO_ERR_ALIASING,
 EVO_ERR_UNSUPPORTED, EVO_ERR_HIP, EVO_ERR_NO_BIAS, EVO_ERR_SCRATCH) = range(10)

# Symbols declared in include/evo_attn.h.
EXPORTED = ("evo_attn_fwd", "evo_attn_check", "evo_attn_fwd_strided", "evo_attn_check_strided",
            "evo_attn_dense_layout", "evo_attn_bwd", "evo_attn_bwd_check", "evo_attn_bwd_workspace_size",
            "evo_attn_bwd_strided", "evo_attn_bwd_check_strided",
            "evo_trimul", "evo_trimul_check", "evo_status_string", "evo_attn_last_hip_error",
            "evo_attn_bwd_noalloc", "evo_attn_bwd_noalloc_scratch_bytes", "evo_attn_bwd_noalloc_last_hip_error")
EVO_TRIMUL_OUTGOING, EVO_TRIMUL_INCOMING = 0, 1


class EvoShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("N", ctypes.c_int64), ("L", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64)]


class EvoLayout(ctypes.Structure):
    """evo_layout_t: element strides (q, k, v, out: b, n, l, h; biases; lse rows)."""
    _fields_ = [("q", ctypes.c_int64 * 4), ("k", ctypes.c_int64 * 4), ("v", ctypes.c_int64 * 4),
                ("out", ctypes.c_int64 * 4), ("mask_b", ctypes.c_int64), ("mask_n", ctypes.c_int64),
                ("pair_b", ctypes.c_int64), ("pair_h", ctypes.c_int64), ("pair_i", ctypes.c_int64),
                ("lse_row", ctypes.c_int64)]


class EvoTrimulShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("C", ctypes.c_int64), ("L", ctypes.c_int64)]


class EvoAttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = f"evo_attn status {status}: {evo_status_string(status)}"
        if status == EVO_ERR_HIP:
            msg += f" (hipError_t {evo_attn_last_hip_error()})"
        super().__init__(msg)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python evoformer_biased_attention_amd/build.py`")
    # One HIP runtime per process.  PyTorch ships its own libamdhip64 (same
    # soname, libamdhip64.so.7); loading torch first makes the dynamic loader
    # bind this library to that runtime instead of mapping a second copy from
    # /opt/rocm, whose device pointers and streams torch's would not know.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.evo_attn_fwd.restype = ctypes.c_int
    lib.evo_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(EvoShape), ctypes.c_int, vp]
    lib.evo_attn_check.restype = ctypes.c_int
    lib.evo_attn_check.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(EvoShape), ctypes.c_int]
    lib.evo_attn_fwd_strided.restype = ctypes.c_int
    lib.evo_attn_fwd_strided.argtypes = [vp] * 7 + [ctypes.POINTER(EvoLayout), ctypes.POINTER(EvoShape), ctypes.c_int,
                                                    vp]
    lib.evo_attn_check_strided.restype = ctypes.c_int
    lib.evo_attn_check_strided.argtypes = [vp] * 7 + [ctypes.POINTER(EvoLayout), ctypes.POINTER(EvoShape), ctypes.c_int]
    lib.evo_attn_dense_layout.restype = None
    lib.evo_attn_dense_layout.argtypes = [ctypes.POINTER(EvoShape), ctypes.POINTER(EvoLayout)]
    lib.evo_attn_bwd.restype = ctypes.c_int
    lib.evo_attn_bwd.argtypes = [vp] * 15 + [ctypes.c_size_t, ctypes.POINTER(EvoShape), ctypes.c_int, vp]
    lib.evo_attn_bwd_check.restype = ctypes.c_int
    lib.evo_attn_bwd_check.argtypes = [vp] * 15 + [ctypes.c_size_t, ctypes.POINTER(EvoShape), ctypes.c_int]
    lib.evo_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.evo_attn_bwd_workspace_size.argtypes = [ctypes.POINTER(EvoShape), ctypes.c_int]
    lib.evo_attn_bwd_strided.restype = ctypes.c_int
    lib.evo_attn_bwd_strided.argtypes = [vp] * 15 + [ctypes.c_size_t, ctypes.POINTER(EvoLayout),
                                                     ctypes.POINTER(EvoShape), ctypes.c_int, vp]
    lib.evo_attn_bwd_check_strided.restype = ctypes.c_int
    lib.evo_attn_bwd_check_strided.argtypes = [vp] * 15 + [ctypes.c_size_t, ctypes.POINTER(EvoLayout),
                                                           ctypes.POINTER(EvoShape), ctypes.c_int]
    lib.evo_trimul.restype = ctypes.c_int
    lib.evo_trimul.argtypes = [vp, vp, vp, ctypes.POINTER(EvoTrimulShape), ctypes.c_int, ctypes.c_int, vp]
    lib.evo_trimul_check.restype = ctypes.c_int
    lib.evo_trimul_check.argtypes = [vp, vp, vp, ctypes.POINTER(EvoTrimulShape), ctypes.c_int, ctypes.c_int]
    lib.evo_status_string.restype = ctypes.c_char_p
    lib.evo_status_string.argtypes = [ctypes.c_int]
    lib.evo_attn_last_hip_error.restype = ctypes.c_int
    lib.evo_attn_last_hip_error.argtypes = []
    lib.evo_attn_bwd_noalloc.restype = ctypes.c_int
    lib.evo_attn_bwd_noalloc.argtypes = [vp] * 14 + [ctypes.POINTER(EvoShape), ctypes.c_int, vp]
    lib.evo_attn_bwd_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.evo_attn_bwd_noalloc_scratch_bytes.argtypes = []
    lib.evo_attn_bwd_noalloc_last_hip_error.restype = ctypes.c_int
    lib.evo_attn_bwd_noalloc_last_hip_error.argtypes = []
    return lib


_lib = _load()


def _addr(x):
    """None -> NULL, int -> itself, tensor -> data_ptr()."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _shape(shape):
    if isinstance(shape, EvoShape):
        return shape
    return EvoShape(*[int(s) for s in shape])


def evo_status_string(status: int) -> str:
    return _lib.evo_status_string(int(status)).decode()


def evo_attn_last_hip_error() -> int:
    """hipError_t of this thread's last launch failure (0 if none)."""
    return _lib.evo_attn_last_hip_error()


def evo_attn_check(q, k, v, mask_bias, pair_bias, out, lse, shape, dtype) -> int:
    """Host-only validation; returns the status code (no HIP call is made)."""
    return _lib.evo_attn_check(_addr(q), _addr(k), _addr(v), _addr(mask_bias), _addr(pair_bias), _addr(out),
                               _addr(lse), ctypes.byref(_shape(shape)), int(dtype))


def evo_attn_fwd(q, k, v, mask_bias, pair_bias, out, lse, shape, dtype, stream=None) -> int:
    """Enqueue the forward pass; returns the status code.

    `stream` is a hipStream_t as an int (e.g. torch.cuda.current_stream().cuda_stream)
    or None for the default stream.
    """
    return _lib.evo_attn_fwd(_addr(q), _addr(k), _addr(v), _addr(mask_bias), _addr(pair_bias), _addr(out),
                             _addr(lse), ctypes.byref(_shape(shape)), int(dtype), stream)


def evo_attn_bwd_check(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, delta,
                       shape, dtype, workspace=None, workspace_bytes=0) -> int:
    """Host-only validation of the backward call; returns the status code."""
    return _lib.evo_attn_bwd_check(*[_addr(x) for x in (q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                                       dmask_bias, dpair_bias, delta, workspace)],
                                   int(workspace_bytes), ctypes.byref(_shape(shape)), int(dtype))


def evo_attn_bwd_workspace_size(shape, dtype) -> int:
    """Bytes of workspace for the fastest backward on this shape (0: none used)."""
    return int(_lib.evo_attn_bwd_workspace_size(ctypes.byref(_shape(shape)), int(dtype)))


def evo_attn_bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, delta,
                 shape, dtype, stream=None, workspace=None, workspace_bytes=0) -> int:
    """Enqueue the backward pass; returns the status code (arguments as in include/evo_attn.h)."""
    return _lib.evo_attn_bwd(*[_addr(x) for x in (q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                                 dmask_bias, dpair_bias, delta, workspace)],
                             int(workspace_bytes), ctypes.byref(_shape(shape)), int(dtype), stream)


def evo_attn_bwd_noalloc(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, delta,
                         shape, dtype, stream=None) -> int:
    """Enqueue the backward pass with the library's static scratch instead of a workspace (no allocation);
    returns the status code (EVO_ERR_SCRATCH when the shape needs more than the static buffer holds)."""
    return _lib.evo_attn_bwd_noalloc(*[_addr(x) for x in (q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                                         dmask_bias, dpair_bias, delta)],
                                     ctypes.byref(_shape(shape)), int(dtype), stream)


def evo_attn_bwd_noalloc_scratch_bytes() -> int:
    """Bytes of the static scratch array evo_attn_bwd_noalloc uses on each GPU."""
    return int(_lib.evo_attn_bwd_noalloc_scratch_bytes())


def evo_attn_bwd_check_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias,
                               delta, layout, shape, dtype, workspace=None, workspace_bytes=0) -> int:
    """Host-only validation of the strided backward call; returns the status code."""
    return _lib.evo_attn_bwd_check_strided(*[_addr(x) for x in (q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk,
                                                               dv, dmask_bias, dpair_bias, delta, workspace)],
                                           int(workspace_bytes), ctypes.byref(layout), ctypes.byref(_shape(shape)),
                                           int(dtype))


def evo_attn_bwd_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, delta,
                         layout, shape, dtype, stream=None, workspace=None, workspace_bytes=0) -> int:
    """Enqueue the backward pass on strided tensors; each gradient has its tensor's layout."""
    return _lib.evo_attn_bwd_strided(*[_addr(x) for x in (q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv,
                                                         dmask_bias, dpair_bias, delta, workspace)],
                                     int(workspace_bytes), ctypes.byref(layout), ctypes.byref(_shape(shape)),
                                     int(dtype), stream)


def evo_attn_dense_layout(shape) -> EvoLayout:
    """The dense layout of `shape` (what evo_attn_fwd assumes)."""
    lay = EvoLayout()
    _lib.evo_attn_dense_layout(ctypes.byref(_shape(shape)), ctypes.byref(lay))
    return lay


def evo_attn_check_strided(q, k, v, mask_bias, pair_bias, out, lse, layout, shape, dtype) -> int:
    """Host-only validation of the strided call; returns the status code."""
    return _lib.evo_attn_check_strided(_addr(q), _addr(k), _addr(v), _addr(mask_bias), _addr(pair_bias), _addr(out),
                                       _addr(lse), ctypes.byref(layout), ctypes.byref(_shape(shape)), int(dtype))


def evo_attn_fwd_strided(q, k, v, mask_bias, pair_bias, out, lse, layout, shape, dtype, stream=None) -> int:
    """Enqueue the forward pass on strided tensors; returns the status code."""
    return _lib.evo_attn_fwd_strided(_addr(q), _addr(k), _addr(v), _addr(mask_bias), _addr(pair_bias), _addr(out),
                                     _addr(lse), ctypes.byref(layout), ctypes.byref(_shape(shape)), int(dtype), stream)


def layout_of(q, k, v, out, mask_bias=None, pair_bias=None, lse_row=None) -> EvoLayout:
    """evo_layout_t from torch tensors viewed as [B,N,L,H,D] (d contiguous), [B,N,1,1,L] and [B,1,H,L,L]
    (keys contiguous); lse_row defaults to L."""
    lay = EvoLayout()
    L = q.shape[2]
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.stride(4) != 1:
            raise ValueError(f"{name}: the head dimension must be contiguous")
        getattr(lay, name)[:] = [t.stride(0), t.stride(1), t.stride(2), t.stride(3)]
    if mask_bias is not None:
        if mask_bias.stride(4) != 1:
            raise ValueError("mask_bias: keys must be contiguous")
        lay.mask_b, lay.mask_n = mask_bias.stride(0), mask_bias.stride(1)
    if pair_bias is not None:
        if pair_bias.stride(4) != 1:
            raise ValueError("pair_bias: keys must be contiguous")
        lay.pair_b, lay.pair_h, lay.pair_i = pair_bias.stride(0), pair_bias.stride(2), pair_bias.stride(3)
    else:
        lay.pair_i = L
    lay.lse_row = L if lse_row is None else int(lse_row)
    return lay


def torch_dtype_code(dt) -> int:
    import torch
    return {torch.float32: EVO_DTYPE_F32, torch.bfloat16: EVO_DTYPE_BF16, torch.float16: EVO_DTYPE_F16}[dt]


def fwd(q, k, v, mask_bias=None, pair_bias=None, out=None, lse=True, stream=None):
    """torch convenience wrapper: allocates out (and lse) with torch, then calls evo_attn_fwd.

    q, k, v: [B,N,L,H,D] contiguous device tensors; mask_bias [B,N,1,1,L] and
    pair_bias [B,1,H,L,L] of the same dtype, or None.  Returns (out, lse or None).
    Raises EvoAttnError for any status other than EVO_OK.
    """
    import torch
    B, N, L, H, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("mask_bias", mask_bias), ("pair_bias", pair_bias)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is None:
        out = torch.empty_like(q)
    if lse is True:
        lse_t = torch.empty((B, N, H, L), dtype=torch.float32, device=q.device)
    elif lse is False or lse is None:
        lse_t = None
    else:
        lse_t = lse
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = evo_attn_fwd(q, k, v, mask_bias, pair_bias, out, lse_t, (B, N, L, H, D), torch_dtype_code(q.dtype),
                      stream)
    if st != EVO_OK:
        raise EvoAttnError(st)
    return out, lse_t


def _lse_row(lse, B, N, H, L):
    """Row stride of an lse-like tensor [B,N,H,L] whose (b, n, h) rows are equally spaced."""
    if tuple(lse.shape) != (B, N, H, L) or lse.stride(3) != 1:
        raise ValueError("lse must be [B,N,H,L] with contiguous rows")
    # size-1 axes have arbitrary strides: take the row step from the first axis that moves
    row = lse.stride(2) if H > 1 else lse.stride(1) if N > 1 else lse.stride(0) if B > 1 else L
    if (N > 1 and lse.stride(1) != H * row) or (B > 1 and lse.stride(0) != N * H * row):
        raise ValueError("lse rows must be equally spaced")
    return row


def _self_overlapping(t) -> bool:
    """Whether two distinct indices of t share an address (a broadcast view such as expand()'s stride 0)."""
    axes = sorted((st, n) for st, n in zip(t.stride(), t.shape) if n > 1)
    reach = 1
    for st, n in axes:
        if st < reach:
            return True
        reach += (n - 1) * st
    return False


def bwd(q, k, v, mask_bias, pair_bias, out, lse, dout, want_dmask=True, want_dpair=True, stream=None,
        workspace=True):
    """torch convenience wrapper around evo_attn_bwd_strided: allocates the gradients (each with the
    strides of its tensor, so views such as the transposed tensors of ending-node or column attention
    get gradients in the same views), delta (with lse's row stride) and, unless workspace=False, the
    recommended workspace, with torch.

    out and lse are the forward pass's results for the same inputs; dout must have out's strides.
    Returns (dq, dk, dv, dmask_bias or None, dpair_bias or None, delta); a bias gradient is computed
    only when that bias is given and wanted.  A wanted bias gradient needs a bias whose elements have
    distinct addresses (a broadcast view's gradient would collide with itself): ValueError otherwise.
    Raises EvoAttnError for any status other than EVO_OK.
    """
    import torch
    B, N, L, H, D = q.shape
    for name, t, want in (("mask_bias", mask_bias, want_dmask), ("pair_bias", pair_bias, want_dpair)):
        if t is not None and want and _self_overlapping(t):
            raise ValueError(f"{name} is a broadcast view: its gradient needs a bias with distinct elements")
    if tuple(dout.stride()) != tuple(out.stride()):
        raise ValueError("dout must have the strides of out")
    row = _lse_row(lse, B, N, H, L)
    lay = layout_of(q, k, v, out, mask_bias, pair_bias, lse_row=row)
    like = lambda t: torch.empty_strided(t.size(), t.stride(), dtype=t.dtype, device=t.device)
    dq, dk, dv = like(q), like(k), like(v)
    dmask = like(mask_bias) if (mask_bias is not None and want_dmask) else None
    dpair = like(pair_bias) if (pair_bias is not None and want_dpair) else None
    delta = torch.empty((B, N, H, row), dtype=torch.float32, device=q.device)[..., :L]
    code = torch_dtype_code(q.dtype)
    ws, ws_bytes = None, 0
    if workspace and dpair is not None:
        ws_bytes = evo_attn_bwd_workspace_size((B, N, L, H, D), code)
        if ws_bytes:
            ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = evo_attn_bwd_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask, dpair, delta, lay,
                              (B, N, L, H, D), code, stream, workspace=ws, workspace_bytes=ws_bytes)
    if st != EVO_OK:
        raise EvoAttnError(st)
    return dq, dk, dv, dmask, dpair, delta


# ---------------------------------------------------------------------------
# Differentiable call.  The pages' interface takes Q, K, V and a list of at
# most two biases (None where a bias is absent), the first broadcast like
# [B, N, 1, 1, L] (one key mask per sequence), the second like
# [B, 1, H, L, L] (one pair bias per head), and returns O; gradients flow to
# Q, K, V and to each bias that requires one.  Both passes are the C ABI's
# (evo_attn_fwd_strided, evo_attn_bwd_strided), so views such as the
# transposed tensors of ending-node or column attention need no copies.
# ---------------------------------------------------------------------------
def _check_biases(q, biases):
    """(mask_bias, pair_bias) from the bias list; raises ValueError for a list of more than two or a bias of
    the wrong shape, dtype or device, before anything is launched."""
    biases = list(biases) if biases is not None else []
    if len(biases) > 2:
        raise ValueError("at most two biases: [mask_bias [B,N,1,1,L], pair_bias [B,1,H,L,L]]")
    biases += [None] * (2 - len(biases))
    B, N, L, H, D = q.shape
    want = {0: (B, N, 1, 1, L), 1: (B, 1, H, L, L)}
    for i, b in enumerate(biases):
        if b is None:
            continue
        if tuple(b.shape) != want[i]:
            raise ValueError(f"bias {i} must have shape {want[i]}, not {tuple(b.shape)}")
        if b.dtype != q.dtype or b.device != q.device:
            raise ValueError(f"bias {i} must have q's dtype and device")
        if b.stride(4) != 1:
            raise ValueError(f"bias {i}: keys must be contiguous")
    return biases[0], biases[1]


_FN = None


def _function():
    """The torch.autograd.Function (built on first use, so that importing this package needs no torch)."""
    global _FN
    if _FN is not None:
        return _FN
    import torch

    class EvoformerAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, mask_bias, pair_bias):
            B, N, L, H, D = q.shape
            out = torch.empty_like(q)  # q's strides when q is dense, else contiguous
            if out.stride(4) != 1:
                out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
            lse = torch.empty((B, N, H, L), dtype=torch.float32, device=q.device)
            lay = layout_of(q, k, v, out, mask_bias, pair_bias)
            st = evo_attn_fwd_strided(q, k, v, mask_bias, pair_bias, out, lse, lay, (B, N, L, H, D),
                                      torch_dtype_code(q.dtype), torch.cuda.current_stream(q.device).cuda_stream)
            if st != EVO_OK:
                raise EvoAttnError(st)
            ctx.save_for_backward(q, k, v, mask_bias, pair_bias, out, lse)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, mask_bias, pair_bias, out, lse = ctx.saved_tensors
            if tuple(dout.stride()) != tuple(out.stride()):
                d = torch.empty_strided(out.size(), out.stride(), dtype=out.dtype, device=out.device)
                d.copy_(dout)
                dout = d
            need = ctx.needs_input_grad
            dq, dk, dv, dm, dp, _ = bwd(q, k, v, mask_bias, pair_bias, out, lse, dout,
                                        want_dmask=mask_bias is not None and need[3],
                                        want_dpair=pair_bias is not None and need[4])
            return dq, dk, dv, dm, dp

    _FN = EvoformerAttentionFn
    return _FN


def evoformer_attention(q, k, v, biases=()):
    """O = softmax(Q K^T / sqrt(D) + mask_bias + pair_bias) V over the keys of each (b, n, h), differentiable.

    q, k, v: [B, N, L, H, D] device tensors (head dimension contiguous; any other strides, e.g. a
    transposed view); biases: a list of at most two tensors or None, [mask_bias [B,N,1,1,L],
    pair_bias [B,1,H,L,L]], of q's dtype (keys contiguous).  Returns O, [B,N,L,H,D], in q's dtype.
    Gradients reach q, k, v and every bias with requires_grad; a bias gradient is computed only then.
    Raises ValueError for a bad bias list and EvoAttnError for a status other than EVO_OK.
    """
    mask_bias, pair_bias = _check_biases(q, biases)
    # A broadcast bias (e.g. a mask expand()ed over N) that needs a gradient is
    # materialised first: its gradient then has one element per position, and
    # autograd sums it back over the broadcast axes.
    if mask_bias is not None and mask_bias.requires_grad and _self_overlapping(mask_bias):
        mask_bias = mask_bias.contiguous()
    if pair_bias is not None and pair_bias.requires_grad and _self_overlapping(pair_bias):
        pair_bias = pair_bias.contiguous()
    return _function().apply(q, k, v, mask_bias, pair_bias)


def evo_trimul_check(a, w, x, shape, direction, dtype) -> int:
    """Host-only validation of the triangle multiplication; shape is (B, C, L)."""
    return _lib.evo_trimul_check(_addr(a), _addr(w), _addr(x), ctypes.byref(EvoTrimulShape(*[int(v) for v in shape])),
                                 int(direction), int(dtype))


def evo_trimul(a, w, x, shape, direction, dtype, stream=None) -> int:
    """Enqueue the triangle multiplication (include/evo_attn.h); returns the status code."""
    return _lib.evo_trimul(_addr(a), _addr(w), _addr(x), ctypes.byref(EvoTrimulShape(*[int(v) for v in shape])),
                           int(direction), int(dtype), stream)


def trimul(a, w, direction="outgoing", out=None, stream=None):
    """torch wrapper: a, w contiguous [B, C, L, L] device tensors; returns x of the same shape and dtype."""
    import torch
    for name, t in (("a", a), ("w", w)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    x = torch.empty_like(a) if out is None else out
    B, C, L, _ = a.shape
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    d = {"outgoing": EVO_TRIMUL_OUTGOING, "incoming": EVO_TRIMUL_INCOMING}[direction]
    st = evo_trimul(a, w, x, (B, C, L), d, torch_dtype_code(a.dtype), stream)
    if st != EVO_OK:
        raise EvoAttnError(st)
    return x
