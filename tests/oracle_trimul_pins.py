"""Pins for the oracle's triangle multiplication (evo_ref_trimul).

Every check takes `tref(a, w, dtype, direction) -> x` so that the same checks
run against the real oracle and against deliberately broken builds.  The
references are numpy's einsum in float64 (a library routine), a pure-Python
brute force with exactly rounded sums, closed forms and invariants of the
contraction:
  outgoing: x[b,c,i,j] = sum_k a[b,c,i,k] w[b,c,j,k]
  incoming: x[b,c,i,j] = sum_k a[b,c,k,i] w[b,c,k,j]
"""
from __future__ import annotations

import math

import numpy as np

from synthetic import storage_to_f32, to_storage

DIRS = ("outgoing", "incoming")


def _rand(shape, dtype, seed, scale=1.0):
    x = (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)
    return to_storage(x, dtype)


def _f64(x, dtype):
    return storage_to_f32(x, dtype).astype(np.float64)


def pin_trimul_einsum(tref):
    for t, shape in enumerate([(1, 1, 1, 1), (1, 3, 7, 7), (2, 2, 16, 16), (1, 4, 33, 33)]):
        for dtype in ("f32", "bf16"):
            a, w = _rand(shape, dtype, 10 + t), _rand(shape, dtype, 20 + t)
            af, wf = _f64(a, dtype), _f64(w, dtype)
            np.testing.assert_allclose(tref(a, w, dtype, "outgoing"), np.einsum("bcik,bcjk->bcij", af, wf),
                                       rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(tref(a, w, dtype, "incoming"), np.einsum("bcki,bckj->bcij", af, wf),
                                       rtol=1e-12, atol=1e-12)


def pin_trimul_brute_force(tref):
    shape = (2, 2, 4, 4)
    a, w = _rand(shape, "f32", 1), _rand(shape, "f32", 2)
    af, wf = _f64(a, "f32"), _f64(w, "f32")
    out = tref(a, w, "f32", "outgoing")
    inc = tref(a, w, "f32", "incoming")
    B, C, L, _ = shape
    for b in range(B):
        for c in range(C):
            for i in range(L):
                for j in range(L):
                    assert abs(out[b, c, i, j] - math.fsum(af[b, c, i, k] * wf[b, c, j, k] for k in range(L))) < 1e-13
                    assert abs(inc[b, c, i, j] - math.fsum(af[b, c, k, i] * wf[b, c, k, j] for k in range(L))) < 1e-13


def pin_trimul_identity(tref):
    """a = I in every channel: outgoing gives w transposed, incoming gives w."""
    B, C, L = 1, 3, 9
    eye = np.broadcast_to(np.eye(L, dtype=np.float32), (B, C, L, L)).copy()
    for dtype in ("f32", "bf16", "f16"):
        w = _rand((B, C, L, L), dtype, 3)
        wf = _f64(w, dtype)
        np.testing.assert_array_equal(tref(to_storage(eye, dtype), w, dtype, "outgoing"), wf.transpose(0, 1, 3, 2))
        np.testing.assert_array_equal(tref(to_storage(eye, dtype), w, dtype, "incoming"), wf)


def pin_trimul_ones(tref):
    """a = w = 1: every entry is L, in both orientations."""
    ones = to_storage(np.ones((2, 2, 13, 13), np.float32), "bf16")
    for d in DIRS:
        assert np.all(tref(ones, ones, "bf16", d) == 13.0)


def pin_trimul_transpose_relation(tref):
    """incoming(a, w) = outgoing(a^T, w^T), the transpose over the two node axes."""
    a, w = _rand((1, 3, 11, 11), "bf16", 4), _rand((1, 3, 11, 11), "bf16", 5)
    tT = lambda x: np.ascontiguousarray(x.transpose(0, 1, 3, 2))
    np.testing.assert_allclose(tref(a, w, "bf16", "incoming"), tref(tT(a), tT(w), "bf16", "outgoing"),
                               rtol=1e-13, atol=1e-13)


def pin_trimul_operand_swap(tref):
    """Swapping the operands transposes the result; with w = a the result is symmetric."""
    a, w = _rand((2, 2, 10, 10), "bf16", 6), _rand((2, 2, 10, 10), "bf16", 7)
    for d in DIRS:
        np.testing.assert_allclose(tref(w, a, "bf16", d), tref(a, w, "bf16", d).transpose(0, 1, 3, 2),
                                   rtol=1e-13, atol=1e-13)
        x = tref(a, a, "bf16", d)
        np.testing.assert_allclose(x, x.transpose(0, 1, 3, 2), rtol=1e-13, atol=1e-13)


def pin_trimul_channels_independent(tref):
    a, w = _rand((2, 3, 8, 8), "bf16", 8), _rand((2, 3, 8, 8), "bf16", 9)
    for d in DIRS:
        x = tref(a, w, "bf16", d)
        a2 = a.copy()
        a2[:, 1] = _rand((2, 8, 8), "bf16", 10)
        x2 = tref(a2, w, "bf16", d)
        np.testing.assert_array_equal(x2[:, [0, 2]], x[:, [0, 2]])
        assert not np.array_equal(x2[:, 1], x[:, 1])


def pin_trimul_dtype_widening(tref):
    """Values exact in all three formats give identical results in all three."""
    rng = np.random.default_rng(11)
    a = rng.integers(-16, 16, (1, 2, 6, 6)).astype(np.float32) / 8
    w = rng.integers(-16, 16, (1, 2, 6, 6)).astype(np.float32) / 8
    for d in DIRS:
        res = [tref(to_storage(a, dt), to_storage(w, dt), dt, d) for dt in ("f32", "bf16", "f16")]
        for r in res[1:]:
            np.testing.assert_array_equal(r, res[0])


ALL_TRIMUL_PINS = [pin_trimul_identity, pin_trimul_ones, pin_trimul_einsum, pin_trimul_brute_force,
                   pin_trimul_transpose_relation, pin_trimul_operand_swap, pin_trimul_channels_independent,
                   pin_trimul_dtype_widening]
