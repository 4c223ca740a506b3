"""Pins for the fp64 oracle's backward pass: facts fixed by mathematics.

Every check takes `gref(q, k, v, mask, pair, dout, dtype) -> (dq, dk, dv,
dmask, dpair)` so that the same checks run against the real oracle build and
against deliberately broken builds (which they must reject).  None of them
retypes the oracle's gradient formulas: the references are automatic
differentiation of the forward definition (torch, float64), central finite
differences of the already pinned forward oracle, closed forms worked out by
hand, and invariants of the softmax Jacobian.

Operation (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南", hmyw.cn,
sections 4 and 5.4): out = softmax(Q.K^T / sqrt(D) + mask + pair) . V; the
backward pass returns the gradients of a scalar loss sum(out * dO) with
respect to q, k, v and each bias, a bias gradient summed over the axes along
which that bias broadcasts (mask: heads and queries; pair: the N axis).
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from synthetic import MASK_NEG, random_dout, random_problem, storage_to_f32, to_storage

NEG = MASK_NEG


def _st(x, dtype):
    return to_storage(np.asarray(x, np.float32), dtype)


def _f64(x, dtype):
    return storage_to_f32(x, dtype).astype(np.float64)


def _call(gref, w, dout):
    return gref(w.q, w.k, w.v, w.mask, w.pair, dout, w.dtype)


# ---------------------------------------------------------------------------
# Automatic differentiation of the forward definition (torch, float64, CPU).
# ---------------------------------------------------------------------------
def torch_grads(q, k, v, mask, pair, dout):
    """float64 arrays in [B,N,L,H,D] / [B,N,1,1,L] / [B,1,H,L,L]; returns autograd gradients."""
    import torch
    t = {n: None if x is None else torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for n, x in (("q", q), ("k", k), ("v", v), ("mask", mask), ("pair", pair))}
    D = q.shape[-1]
    qh, kh, vh = (t[n].permute(0, 1, 3, 2, 4) for n in ("q", "k", "v"))  # [B,N,H,L,D]
    s = torch.matmul(qh, kh.transpose(-1, -2).contiguous()) / math.sqrt(D)
    if t["mask"] is not None:
        s = s + t["mask"]            # [B,N,1,1,L] broadcasts over heads and queries
    if t["pair"] is not None:
        s = s + t["pair"]            # [B,1,H,L,L] broadcasts over N
    o = torch.matmul(torch.softmax(s, dim=-1), vh).permute(0, 1, 3, 2, 4)
    (o * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    g = lambda n: None if t[n] is None else t[n].grad.numpy()
    return g("q"), g("k"), g("v"), g("mask"), g("pair")


def pin_bwd_torch_autograd(gref, shapes=((1, 2, 9, 2, 8), (2, 3, 17, 2, 16), (1, 2, 33, 3, 32))):
    for t, (B, N, L, H, D) in enumerate(shapes):
        for dtype in ("f32", "bf16"):
            w = random_problem(B, N, L, H, D, dtype=dtype, seed=500 + t, mask="random", pair="normal",
                               mask_frac=0.2, bias_scale=1.5)
            dout = random_dout(w.shape, dtype, seed=600 + t)
            got = _call(gref, w, dout)
            want = torch_grads(*(_f64(x, dtype) for x in (w.q, w.k, w.v, w.mask, w.pair, dout)))
            for name, a, b in zip(("dq", "dk", "dv", "dmask", "dpair"), got, want):
                np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12, err_msg=name)
            # one bias at a time, and none
            for m, p in ((w.mask, None), (None, w.pair), (None, None)):
                got = gref(w.q, w.k, w.v, m, p, dout, dtype)
                want = torch_grads(*(None if x is None else _f64(x, dtype) for x in (w.q, w.k, w.v, m, p, dout)))
                for name, a, b in zip(("dq", "dk", "dv", "dmask", "dpair"), got, want):
                    assert (a is None) == (b is None), name
                    if a is not None:
                        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12, err_msg=name)


# ---------------------------------------------------------------------------
# Central finite differences of the (separately pinned) forward oracle.
# ---------------------------------------------------------------------------
def pin_bwd_finite_differences(gref):
    """f32 storage, inputs on a 2^-8 grid so that x +- 2^-14 is exact; loss = sum(out * dO).

    The central difference has truncation error ~h^2 * f''' (about 1e-8 here),
    far below the effect of any wrong term in a gradient.
    """
    B, N, L, H, D = 1, 2, 5, 2, 4
    rng = np.random.default_rng(77)
    grid = lambda shape, lim: (rng.integers(-lim, lim, shape).astype(np.float32) / 256)
    q, k, v = (grid((B, N, L, H, D), 384) for _ in range(3))
    mask = grid((B, N, 1, 1, L), 512)
    pair = grid((B, 1, H, L, L), 512)
    dout = grid((B, N, L, H, D), 256)
    dof = dout.astype(np.float64)
    h = 2.0 ** -14

    def loss(xs):
        o, _ = oracle.fwd(*xs, dtype="f32", nthreads=1)
        return math.fsum((o * dof).ravel())

    base = [q, k, v, mask, pair]
    got = gref(q, k, v, mask, pair, dout, "f32")
    for which, name in enumerate(("dq", "dk", "dv", "dmask", "dpair")):
        fd = np.zeros(base[which].shape)
        for idx in np.ndindex(base[which].shape):
            up = [x.copy() for x in base]
            dn = [x.copy() for x in base]
            up[which][idx] += np.float32(h)
            dn[which][idx] -= np.float32(h)
            assert up[which][idx] - base[which][idx] == np.float32(h)  # the step is exact
            fd[idx] = (loss(up) - loss(dn)) / (2 * h)
        np.testing.assert_allclose(got[which], fd, rtol=0, atol=2e-6, err_msg=name)


# ---------------------------------------------------------------------------
# Closed form: two keys and a zero query, where the softmax is a sigmoid.
# ---------------------------------------------------------------------------
def pin_bwd_two_keys_closed_form(gref):
    """L=2, D=4 (scale 1/2), q=0, k_j=e_j, v_j=e_j, pair rows (0, 1), dO=(1, 2, 0, 0).

    P = (1, e)/(1+e) for every query; with g = dO.(v0 - v1) = -1 and
    c = e/(1+e)^2 = P0 P1: dS = (c g, -c g) = (-c, c).  Then
    dpair[i] = (-c, c); dmask = sum over the two queries = (-2c, 2c);
    dq_i = (dS0 k0 + dS1 k1)/2 = (-c/2, c/2, 0, 0); dk_j = dS_j q / 2 = 0;
    dv_j = sum_i P_j dO = 2 P_j (1, 2, 0, 0).
    """
    E = math.e
    c = E / (1 + E) ** 2
    P = np.array([1 / (1 + E), E / (1 + E)])
    for dtype in ("f32", "bf16", "f16"):
        q = np.zeros((1, 1, 2, 1, 4), np.float32)
        k = np.zeros_like(q)
        v = np.zeros_like(q)
        for j in range(2):
            k[0, 0, j, 0, j] = 1
            v[0, 0, j, 0, j] = 1
        dout = np.zeros_like(q)
        dout[0, 0, :, 0, 0] = 1
        dout[0, 0, :, 0, 1] = 2
        mask = np.zeros((1, 1, 1, 1, 2), np.float32)
        pair = np.array([[0, 1], [0, 1]], np.float32).reshape(1, 1, 1, 2, 2)
        dq, dk, dv, dmask, dpair = gref(*(_st(x, dtype) for x in (q, k, v, mask, pair, dout)), dtype)
        for i in range(2):
            np.testing.assert_allclose(dpair[0, 0, 0, i], [-c, c], rtol=1e-14)
            np.testing.assert_allclose(dq[0, 0, i, 0], [-c / 2, c / 2, 0, 0], rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(dmask[0, 0, 0, 0], [-2 * c, 2 * c], rtol=1e-14)
        assert np.all(dk == 0.0)
        for j in range(2):
            np.testing.assert_allclose(dv[0, 0, j, 0], [2 * P[j], 4 * P[j], 0, 0], rtol=1e-14)


# ---------------------------------------------------------------------------
# Special cases.
# ---------------------------------------------------------------------------
def pin_bwd_zero_dout(gref):
    """dO = 0 gives exactly zero gradients."""
    w = random_problem(2, 2, 11, 2, 8, dtype="bf16", seed=41, mask="tail", pair="normal", mask_frac=0.3)
    dq, dk, dv, dm, dp = _call(gref, w, np.zeros_like(w.q))
    for g in (dq, dk, dv, dm, dp):
        assert np.all(g == 0.0)


def pin_bwd_single_key(gref):
    """L = 1: the weight is 1 whatever the score, so dq = dk = 0, bias gradients are 0 and dv = dO."""
    w = random_problem(2, 3, 1, 2, 16, dtype="bf16", seed=42, mask="normal", pair="normal")
    dout = random_dout(w.shape, "bf16", seed=43)
    dq, dk, dv, dm, dp = _call(gref, w, dout)
    for g in (dq, dk, dm, dp):
        assert np.all(g == 0.0)
    np.testing.assert_array_equal(dv, _f64(dout, "bf16"))


def pin_bwd_uniform_values(gref):
    """All value rows of a slice equal: out does not depend on the weights, so
    every score gradient vanishes (dq = dk = dmask = dpair = 0 up to rounding)
    while dv_j = sum_i P_ij dO_i still sums over j to sum_i dO_i."""
    B, N, L, H, D = 1, 2, 13, 2, 8
    w = random_problem(B, N, L, H, D, dtype="bf16", seed=44, mask="normal", pair="normal", bias_scale=2.0)
    v = w.v.copy()
    v[:] = v[:, :, :1]  # broadcast value row 0 over the key axis
    dout = random_dout(w.shape, "bf16", seed=45)
    dq, dk, dv, dm, dp = gref(w.q, w.k, v, w.mask, w.pair, dout, "bf16")
    for g in (dq, dk, dm, dp):
        assert np.max(np.abs(g)) < 1e-13
    np.testing.assert_allclose(dv.sum(axis=2), _f64(dout, "bf16").sum(axis=2), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Invariants of the softmax Jacobian.
# ---------------------------------------------------------------------------
def pin_bwd_zero_sums(gref):
    """Each row of the score gradient sums to zero over keys, hence
    sum_j dpair[.,j] = 0, sum_j dmask[.,j] = 0 and sum_j dk_j = 0; and the
    weights of a row sum to one, hence sum_j dv_j = sum_i dO_i."""
    w = random_problem(2, 3, 21, 2, 16, dtype="bf16", seed=46, mask="tail", pair="normal", mask_frac=0.3,
                       bias_scale=2.0)
    dout = random_dout(w.shape, "bf16", seed=47)
    dq, dk, dv, dm, dp = _call(gref, w, dout)
    scale = max(np.max(np.abs(dp)), np.max(np.abs(dm)), np.max(np.abs(dk)))
    assert scale > 1e-3  # the check is not vacuous
    assert np.max(np.abs(dp.sum(axis=-1))) < 1e-13 * scale * w.shape[2]
    assert np.max(np.abs(dm.sum(axis=-1))) < 1e-13 * scale * w.shape[2]
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-13 * scale * w.shape[2]
    np.testing.assert_allclose(dv.sum(axis=2), _f64(dout, "bf16").sum(axis=2), rtol=1e-12, atol=1e-12)


def pin_bwd_mask_is_pair_summed(gref):
    """With N = 1 both biases receive the same score gradient, so the mask
    gradient equals the pair gradient summed over heads and queries."""
    w = random_problem(2, 1, 15, 3, 8, dtype="bf16", seed=48, mask="normal", pair="normal", bias_scale=2.0)
    dout = random_dout(w.shape, "bf16", seed=49)
    _, _, _, dm, dp = _call(gref, w, dout)
    np.testing.assert_allclose(dm[:, 0, 0, 0, :], dp[:, 0].sum(axis=(1, 2)), rtol=1e-12, atol=1e-14)


def pin_bwd_replicated_n(gref):
    """Three identical copies of one (b, n) slice along N: dq, dk, dv and dmask
    repeat the single-copy values and dpair is three times the single-copy one."""
    w = random_problem(1, 1, 12, 2, 8, dtype="bf16", seed=50, mask="normal", pair="normal", bias_scale=2.0)
    dout = random_dout(w.shape, "bf16", seed=51)
    one = _call(gref, w, dout)
    rep = lambda x: np.repeat(x, 3, axis=1)
    three = gref(rep(w.q), rep(w.k), rep(w.v), rep(w.mask), w.pair, rep(dout), "bf16")
    for a, b in zip(three[:4], one[:4]):
        for n in range(3):
            np.testing.assert_array_equal(a[:, n], b[:, 0])
    np.testing.assert_allclose(three[4], 3 * one[4], rtol=1e-14, atol=1e-16)


def pin_bwd_replicated_heads(gref):
    """Two identical heads (same q, k, v, pair and dO): every per-head gradient
    repeats, and the mask gradient (a sum over heads) doubles."""
    w = random_problem(2, 2, 10, 1, 8, dtype="bf16", seed=52, mask="normal", pair="normal", bias_scale=2.0)
    dout = random_dout(w.shape, "bf16", seed=53)
    one = _call(gref, w, dout)
    rep = lambda x: np.repeat(x, 2, axis=3)
    two = gref(rep(w.q), rep(w.k), rep(w.v), w.mask, np.repeat(w.pair, 2, axis=2), rep(dout), "bf16")
    for a, b in zip(two[:3], one[:3]):
        for h in range(2):
            np.testing.assert_array_equal(a[:, :, :, h], b[:, :, :, 0])
    for h in range(2):
        np.testing.assert_array_equal(two[4][:, :, h], one[4][:, :, 0])
    np.testing.assert_allclose(two[3], 2 * one[3], rtol=1e-14, atol=1e-16)


def pin_bwd_permute_keys(gref):
    """Permuting the keys (k, v rows, mask entries, pair columns) permutes dk, dv,
    dmask and the pair gradient's columns and leaves dq unchanged."""
    w = random_problem(1, 2, 14, 2, 8, dtype="bf16", seed=54, mask="normal", pair="normal", bias_scale=2.0)
    dout = random_dout(w.shape, "bf16", seed=55)
    dq, dk, dv, dm, dp = _call(gref, w, dout)
    p = np.random.default_rng(56).permutation(w.shape[2])
    g = gref(w.q, w.k[:, :, p], w.v[:, :, p], w.mask[..., p], w.pair[..., p], dout, "bf16")
    np.testing.assert_allclose(g[0], dq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[1], dk[:, :, p], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[2], dv[:, :, p], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[3], dm[..., p], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g[4], dp[..., p], rtol=1e-12, atol=1e-14)


def pin_bwd_neg_inf_slice(gref):
    """f16 storage turns the -1e9 mask into -inf.  A (b, n) whose every key is
    -inf has no softmax and contributes nothing: its dq, dk, dv and dmask are
    zero and the pair gradient equals that of the problem without it."""
    w = random_problem(1, 3, 9, 2, 8, dtype="f16", seed=57, mask="normal", pair="normal")
    dout = random_dout(w.shape, "f16", seed=58)
    mask = w.mask.copy()
    mask[0, 1] = _st(np.full((1, 1, 9), NEG, np.float32), "f16")
    dq, dk, dv, dm, dp = gref(w.q, w.k, w.v, mask, w.pair, dout, "f16")
    for g in (dq, dk, dv):
        assert np.all(g[0, 1] == 0.0)
    assert np.all(dm[0, 1] == 0.0)
    keep = [0, 2]
    sub = gref(w.q[:, keep], w.k[:, keep], w.v[:, keep], mask[:, keep], w.pair, dout[:, keep], "f16")
    for a, b in zip((dq, dk, dv, dm), sub[:4]):
        np.testing.assert_array_equal(a[:, keep], b)
    np.testing.assert_allclose(dp, sub[4], rtol=1e-14, atol=1e-16)


ALL_BWD_PINS = [
    pin_bwd_two_keys_closed_form, pin_bwd_torch_autograd, pin_bwd_finite_differences, pin_bwd_zero_dout,
    pin_bwd_single_key, pin_bwd_uniform_values, pin_bwd_zero_sums, pin_bwd_mask_is_pair_summed,
    pin_bwd_replicated_n, pin_bwd_replicated_heads, pin_bwd_permute_keys, pin_bwd_neg_inf_slice,
]
