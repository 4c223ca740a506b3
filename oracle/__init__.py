"""fp64 CPU oracle for the Evoformer biased-attention forward and backward passes.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library: the arithmetic lives in ``evo_ref.c``
(plain loops in double precision), loaded here through ctypes.

The operation (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南",
hmyw.cn, sections 4, 5.2 and 5.4):

    s_j  = q_i . k_j / sqrt(D) + mask[b,n,0,0,j] + pair[b,0,h,i,j]
    out_i = sum_j softmax_j(s) v_j,      lse_i = ln sum_j exp(s_j)

Triangle multiplication (``trimul``) is the second operation: per channel,
a product through the third node of a [B, C, L, L] pair tensor (see
``evo_ref_trimul`` in evo_ref.c for the reading and its source).

The backward pass (section 5.4: the gradients the training path needs,
bias gradients only on request) is the chain rule applied to the same
definition: ``bwd`` returns dq, dk, dv and, when asked, the mask and pair
gradients, each summed over the axes that bias broadcasts along.

Inputs are numpy arrays holding the stored values: ``float32`` arrays for
dtype "f32", ``uint16`` bit patterns for "bf16" and "f16".  Outputs are
float64 arrays, ``out`` shaped [B,N,L,H,D] and ``lse`` shaped [B,N,H,L].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "evo_ref.c")
_LIB = os.path.join(_HERE, "libevoref.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}


GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """gcc one C source into a shared library at `out` (atomic replace)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile evo_ref.c into libevoref.so (OpenMP, IEEE double, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def load_library(path: str):
    """ctypes handle for another build of the oracle source (used by the tests)."""
    return _bind(path)


def _bind(path):
    lib = ctypes.CDLL(path)
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.evo_ref_fwd.restype = ctypes.c_int
    lib.evo_ref_fwd.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, dp, dp,
                                ctypes.c_int]
    lib.evo_ref_bwd.restype = ctypes.c_int
    lib.evo_ref_bwd.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64,
                                dp, dp, dp, dp, dp, ctypes.c_int]
    lib.evo_ref_trimul.restype = ctypes.c_int
    lib.evo_ref_trimul.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, dp, ctypes.c_int]
    lib.evo_ref_rows.restype = ctypes.c_int
    lib.evo_ref_rows.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int, i64, i64, i64, i64, i64, vp, i64,
                                 dp, dp, ctypes.c_int]
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(_LIB)
    return _lib


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def _prep(q, k, v, mask, pair, dtype):
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
    st = _STORAGE[dtype]
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    if q.ndim != 5:
        raise ValueError("q must be [B,N,L,H,D]")
    B, N, L, H, D = q.shape
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype != st or x.shape != (B, N, L, H, D):
            raise ValueError(f"{name}: expected {st.__name__} {(B, N, L, H, D)}, got {x.dtype} {x.shape}")
    if mask is not None:
        mask = np.ascontiguousarray(mask)
        if mask.dtype != st or mask.shape != (B, N, 1, 1, L):
            raise ValueError(f"mask: expected {st.__name__} {(B, N, 1, 1, L)}")
    if pair is not None:
        pair = np.ascontiguousarray(pair)
        if pair.dtype != st or pair.shape != (B, 1, H, L, L):
            raise ValueError(f"pair: expected {st.__name__} {(B, 1, H, L, L)}")
    return q, k, v, mask, pair, (B, N, L, H, D)


def _ptr(x):
    return None if x is None else x.ctypes.data


def fwd(q, k, v, mask=None, pair=None, dtype="bf16", nthreads=None, lib=None):
    """Full evaluation; returns (out [B,N,L,H,D] float64, lse [B,N,H,L] float64).

    `lib` selects another build of evo_ref.c (the tests load deliberately
    broken copies to show that the pins catch them); default: libevoref.so.
    """
    q, k, v, mask, pair, (B, N, L, H, D) = _prep(q, k, v, mask, pair, dtype)
    out = np.empty((B, N, L, H, D), np.float64)
    lse = np.empty((B, N, H, L), np.float64)
    rc = (lib or _load()).evo_ref_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(pair), DTYPES[dtype],
                             B, N, L, H, D, out.ctypes.data, lse.ctypes.data,
                             nthreads or default_threads())
    if rc:
        raise RuntimeError(f"evo_ref_fwd failed with code {rc}")
    return out, lse


def rows(q, k, v, mask=None, pair=None, dtype="bf16", idx=None, nthreads=None, lib=None):
    """Selected rows; idx is an int array [R,4] of (b, n, h, i).

    Returns (out_rows [R,D] float64, lse_rows [R] float64).
    """
    q, k, v, mask, pair, (B, N, L, H, D) = _prep(q, k, v, mask, pair, dtype)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 4))
    out = np.empty((idx.shape[0], D), np.float64)
    lse = np.empty((idx.shape[0],), np.float64)
    rc = (lib or _load()).evo_ref_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(pair), DTYPES[dtype],
                              B, N, L, H, D, idx.ctypes.data, idx.shape[0], out.ctypes.data,
                              lse.ctypes.data, nthreads or default_threads())
    if rc:
        raise RuntimeError(f"evo_ref_rows failed with code {rc}")
    return out, lse


def bwd(q, k, v, mask=None, pair=None, dout=None, dtype="bf16", want_dmask=True, want_dpair=True,
        nthreads=None, lib=None):
    """Gradients of sum(out * dout) with respect to q, k, v and the biases.

    dout has the inputs' storage format and shape [B,N,L,H,D].  Returns
    (dq, dk, dv, dmask, dpair) as float64 arrays: dq/dk/dv [B,N,L,H,D], dmask
    [B,N,1,1,L] (None unless a mask is given and want_dmask), dpair
    [B,1,H,L,L] (None unless a pair bias is given and want_dpair).
    """
    q, k, v, mask, pair, (B, N, L, H, D) = _prep(q, k, v, mask, pair, dtype)
    dout = np.ascontiguousarray(dout)
    if dout.dtype != _STORAGE[dtype] or dout.shape != (B, N, L, H, D):
        raise ValueError(f"dout: expected {_STORAGE[dtype].__name__} {(B, N, L, H, D)}")
    dq, dk, dv = (np.empty((B, N, L, H, D), np.float64) for _ in range(3))
    dmask = np.empty((B, N, 1, 1, L), np.float64) if (mask is not None and want_dmask) else None
    dpair = np.empty((B, 1, H, L, L), np.float64) if (pair is not None and want_dpair) else None
    rc = (lib or _load()).evo_ref_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(pair), _ptr(dout),
                                      DTYPES[dtype], B, N, L, H, D, dq.ctypes.data, dk.ctypes.data,
                                      dv.ctypes.data, _ptr(dmask), _ptr(dpair),
                                      nthreads or default_threads())
    if rc:
        raise RuntimeError(f"evo_ref_bwd failed with code {rc}")
    return dq, dk, dv, dmask, dpair


TRIMUL_DIRECTIONS = {"outgoing": 0, "incoming": 1}


def trimul(a, w, dtype="bf16", direction="outgoing", nthreads=None, lib=None):
    """x[b,c,i,j] = sum_k a[b,c,i,k] w[b,c,j,k] (outgoing) or sum_k a[b,c,k,i] w[b,c,k,j] (incoming).

    a, w: [B, C, L, L] storage arrays; returns x [B, C, L, L] float64.
    """
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {sorted(DTYPES)}")
    st = _STORAGE[dtype]
    a, w = np.ascontiguousarray(a), np.ascontiguousarray(w)
    if a.ndim != 4 or a.shape[2] != a.shape[3] or a.shape != w.shape or a.dtype != st or w.dtype != st:
        raise ValueError(f"a, w: expected {st.__name__} [B, C, L, L] of one shape")
    B, C, L, _ = a.shape
    x = np.empty((B, C, L, L), np.float64)
    rc = (lib or _load()).evo_ref_trimul(a.ctypes.data, w.ctypes.data, DTYPES[dtype], B, C, L,
                                         TRIMUL_DIRECTIONS[direction], x.ctypes.data, nthreads or default_threads())
    if rc:
        raise RuntimeError(f"evo_ref_trimul failed with code {rc}")
    return x
