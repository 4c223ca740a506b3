"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Every check takes `ref(q, k, v, mask, pair, dtype) -> (out, lse)` so that the
same checks run against the real oracle build and against deliberately broken
builds (which they must reject).  None of them retypes the oracle's formula:
each compares with a closed form, an invariant, a library routine, or a
brute-force evaluation written in a different style (explicit score matrix,
exactly rounded sums).

Operation (page "DeepSpeed DS4Sci_EvoformerAttention 内核实战指南", hmyw.cn):
softmax(Q.K^T * scale + mask + pair) . V with the per-row log-sum-exp
(sections 4, 5.2, 5.4); scale = 1/sqrt(D).
"""
from __future__ import annotations

import math

import numpy as np

from synthetic import MASK_NEG, random_problem, storage_to_f32, to_storage

NEG = MASK_NEG


def _st(x, dtype):
    return to_storage(np.asarray(x, np.float32), dtype)


def _f64(x, dtype):
    return storage_to_f32(x, dtype).astype(np.float64)


# ---------------------------------------------------------------------------
# Brute force: explicit [L, L] score matrix, exactly rounded sums (math.fsum).
# ---------------------------------------------------------------------------
def brute_force(w):
    q, k, v = (_f64(x, w.dtype) for x in (w.q, w.k, w.v))
    B, N, L, H, D = w.shape
    mask = None if w.mask is None else _f64(w.mask, w.dtype)
    pair = None if w.pair is None else _f64(w.pair, w.dtype)
    out = np.zeros((B, N, L, H, D))
    lse = np.zeros((B, N, H, L))
    inv = 1.0 / math.sqrt(D)
    for b in range(B):
        for n in range(N):
            for h in range(H):
                Q, K, V = q[b, n, :, h, :], k[b, n, :, h, :], v[b, n, :, h, :]
                S = np.array([[math.fsum(Q[i] * K[j]) * inv for j in range(L)] for i in range(L)])
                if mask is not None:
                    S = S + mask[b, n, 0, 0][None, :]
                if pair is not None:
                    S = S + pair[b, 0, h]
                for i in range(L):
                    top = S[i].max()
                    e = np.exp(S[i] - top)
                    Z = math.fsum(e)
                    P = e / Z
                    out[b, n, i, h, :] = [math.fsum(P * V[:, d]) for d in range(D)]
                    lse[b, n, h, i] = top + math.log(Z)
    return out, lse


def pin_brute_force(ref, shapes=((1, 1, 1, 1, 1), (1, 2, 3, 2, 8), (2, 1, 5, 3, 32), (1, 3, 17, 1, 8),
                                 (3, 2, 2, 2, 1))):
    for t, (B, N, L, H, D) in enumerate(shapes):
        for dtype in ("f32", "bf16"):
            w = random_problem(B, N, L, H, D, dtype=dtype, seed=100 + t, mask="normal", pair="normal")
            o, l = ref(w.q, w.k, w.v, w.mask, w.pair, dtype)
            bo, bl = brute_force(w)
            np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l, bl, rtol=1e-12, atol=1e-13)
            # one-sided biases
            w2 = random_problem(B, N, L, H, D, dtype=dtype, seed=200 + t, mask="tail", pair=None,
                                mask_frac=0.5)
            o, l = ref(w2.q, w2.k, w2.v, w2.mask, None, dtype)
            bo, bl = brute_force(w2)
            np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l, bl, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Library routine: torch scaled_dot_product_attention in float64 on the CPU,
# attn_mask = mask + pair broadcast to [B, N, H, L, L]; LSE via logsumexp.
# ---------------------------------------------------------------------------
def pin_torch_sdpa(ref, shapes=((1, 3, 40, 4, 32), (2, 2, 33, 3, 16))):
    import torch
    import torch.nn.functional as F
    for t, (B, N, L, H, D) in enumerate(shapes):
        w = random_problem(B, N, L, H, D, dtype="bf16", seed=300 + t, mask="random", pair="normal",
                           mask_frac=0.2, bias_scale=2.0)
        o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
        q, k, v = (torch.from_numpy(_f64(x, "bf16")).permute(0, 1, 3, 2, 4) for x in (w.q, w.k, w.v))
        bias = torch.from_numpy(_f64(w.mask, "bf16")) + torch.from_numpy(_f64(w.pair, "bf16"))
        bias = bias.expand(B, N, H, L, L)
        to = F.scaled_dot_product_attention(q, k, v, attn_mask=bias)  # [B,N,H,L,D]
        np.testing.assert_allclose(o, to.permute(0, 1, 3, 2, 4).numpy(), rtol=1e-11, atol=1e-12)
        scores = torch.matmul(q, k.transpose(-1, -2)) / math.sqrt(D) + bias
        np.testing.assert_allclose(l, torch.logsumexp(scores, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------
def pin_hand_worked(ref):
    """L=3, D=4 (scale 1/2), integer inputs; weights worked out by hand.

    keys k0=e0, k1=e1, k2=e0+e1; values v_j = e_j; key 2 masked by -1e9.
      query 0: q=2e0, pair row (0,2,0): s=(1, 2, .) -> w=(1, e)/(1+e), lse=1+ln(1+e)
      query 1: q=0,  pair row (-1,0,3): s=(-1,0,.) -> w=(1, e)/(1+e), lse=ln(1+1/e)
      query 2: q=4e1, pair row (0,0,0): s=(0, 2, .) -> w=(1,e^2)/(1+e^2), lse=ln(1+e^2)
    """
    E = math.e
    for dtype in ("f32", "bf16", "f16"):
        q = np.zeros((1, 1, 3, 1, 4), np.float32)
        k = np.zeros_like(q)
        v = np.zeros_like(q)
        q[0, 0, 0, 0, 0] = 2
        q[0, 0, 2, 0, 1] = 4
        k[0, 0, 0, 0, 0] = 1
        k[0, 0, 1, 0, 1] = 1
        k[0, 0, 2, 0, :2] = 1
        for j in range(3):
            v[0, 0, j, 0, j] = 1
        mask = np.array([0, 0, NEG], np.float32).reshape(1, 1, 1, 1, 3)
        pair = np.array([[0, 2, 0], [-1, 0, 3], [0, 0, 0]], np.float32).reshape(1, 1, 1, 3, 3)
        o, l = ref(_st(q, dtype), _st(k, dtype), _st(v, dtype), _st(mask, dtype), _st(pair, dtype), dtype)
        want = np.array([[1 / (1 + E), E / (1 + E), 0, 0],
                         [1 / (1 + E), E / (1 + E), 0, 0],
                         [1 / (1 + E * E), E * E / (1 + E * E), 0, 0]])
        np.testing.assert_allclose(o[0, 0, :, 0, :], want, rtol=1e-14, atol=1e-15)
        assert np.all(o[0, 0, :, 0, 2] == 0.0)  # the masked key's value never leaks
        np.testing.assert_allclose(l[0, 0, 0], [1 + math.log(1 + E), math.log(1 + 1 / E), math.log(1 + E * E)],
                                   rtol=1e-14)


def pin_zero_query_mean(ref):
    """Q = 0, no pair, m masked keys: out = mean of the kept value rows, lse = ln(L - m)."""
    B, N, L, H, D = 1, 3, 37, 2, 8
    w = random_problem(B, N, L, H, D, dtype="bf16", seed=5, mask="tail", pair=None, mask_frac=0.4)
    q0 = np.zeros_like(w.q)
    o, l = ref(q0, w.k, w.v, w.mask, None, "bf16")
    vf = _f64(w.v, "bf16")
    mf = _f64(w.mask, "bf16")
    for n in range(N):
        keep = mf[0, n, 0, 0] == 0
        m = L - keep.sum()
        for h in range(H):
            np.testing.assert_allclose(o[0, n, :, h, :], np.broadcast_to(vf[0, n, keep, h, :].mean(0), (L, D)),
                                       rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(l[0, n, h], math.log(L - m), rtol=1e-14)


def pin_single_key(ref):
    """L = 1: out = v_0; lse = the only score, with q = k = e_0 (dot 1)."""
    D = 16
    for dtype in ("f32", "bf16"):
        q = np.zeros((1, 2, 1, 3, D), np.float32)
        q[..., 0] = 1
        rng = np.random.default_rng(9)
        v = rng.standard_normal(q.shape).astype(np.float32)
        mask = np.array([0.5, -2.0], np.float32).reshape(1, 2, 1, 1, 1)
        pair = np.array([1.0, 0.25, -3.0], np.float32).reshape(1, 1, 3, 1, 1)
        o, l = ref(_st(q, dtype), _st(q, dtype), _st(v, dtype), _st(mask, dtype), _st(pair, dtype), dtype)
        np.testing.assert_array_equal(o, _f64(_st(v, dtype), dtype))
        for n in range(2):
            for h in range(3):
                np.testing.assert_allclose(l[0, n, h, 0], 1 / math.sqrt(D) + mask.flat[n] + pair.flat[h],
                                           rtol=1e-15)


def pin_uniform_values(ref):
    """Every value row equal to c: out = c for every query, whatever the scores."""
    w = random_problem(2, 2, 19, 3, 8, dtype="bf16", seed=6, mask="random", pair="normal", mask_frac=0.3,
                       bias_scale=3.0)
    c = np.linspace(-2, 2, 8).astype(np.float32)
    v = _st(np.broadcast_to(c, w.v.shape), "bf16")
    o, _ = ref(w.q, w.k, v, w.mask, w.pair, "bf16")
    np.testing.assert_allclose(o, np.broadcast_to(_f64(_st(c, "bf16"), "bf16"), o.shape), rtol=1e-14, atol=1e-15)


def pin_one_boosted_key(ref):
    """Q = 0 and pair +beta on key j* of query row i only: closed-form weights."""
    B, N, L, H, D = 1, 2, 11, 2, 4
    beta, jstar, istar = 1.5, 7, 3
    rng = np.random.default_rng(11)
    v = rng.standard_normal((B, N, L, H, D)).astype(np.float32)
    pair = np.zeros((B, 1, H, L, L), np.float32)
    pair[0, 0, 1, istar, jstar] = beta
    z = np.zeros((B, N, L, H, D), np.float32)
    o, l = ref(_st(z, "f32"), _st(z, "f32"), v, None, pair, "f32")
    vd = v.astype(np.float64)
    for n in range(N):
        want = (math.exp(beta) * vd[0, n, jstar, 1] + vd[0, n, :, 1].sum(0) - vd[0, n, jstar, 1]) / (
            math.exp(beta) + L - 1)
        np.testing.assert_allclose(o[0, n, istar, 1], want, rtol=1e-13)
        np.testing.assert_allclose(l[0, n, 1, istar], math.log(math.exp(beta) + L - 1), rtol=1e-14)
        # every other (head, query) row is a plain mean with lse = ln L
        np.testing.assert_allclose(o[0, n, istar, 0], vd[0, n, :, 0].mean(0), rtol=1e-13)
        np.testing.assert_allclose(l[0, n, 0, istar], math.log(L), rtol=1e-14)


def pin_two_keys_sigmoid(ref):
    """Two keys: weight of key 0 = sigmoid(s0 - s1), with dots fixed by choice of q, k."""
    D = 4
    q = np.zeros((1, 1, 2, 1, D), np.float32)
    k = np.zeros_like(q)
    q[0, 0, 0, 0, :] = [1, 1, 0, 0]
    q[0, 0, 1, 0, :] = [0, 0, 2, 0]
    k[0, 0, 0, 0, :] = [3, 0, 0, 0]  # dots: q0.k0 = 3, q0.k1 = 1, q1.k0 = 0, q1.k1 = 2
    k[0, 0, 1, 0, :] = [0, 1, 1, 0]
    v = np.zeros_like(q)
    v[0, 0, 0, 0, 0] = 1
    v[0, 0, 1, 0, 1] = 1
    mask = np.array([0.25, -0.5], np.float32).reshape(1, 1, 1, 1, 2)
    pair = np.array([[0.0, 1.0], [-1.0, 0.5]], np.float32).reshape(1, 1, 1, 2, 2)
    o, _ = ref(q, k, v, mask, pair, "f32")
    s = [[3 / 2 + 0.25 + 0.0, 1 / 2 - 0.5 + 1.0], [0 / 2 + 0.25 - 1.0, 2 / 2 - 0.5 + 0.5]]
    for i in range(2):
        p0 = 1 / (1 + math.exp(s[i][1] - s[i][0]))
        np.testing.assert_allclose(o[0, 0, i, 0, :2], [p0, 1 - p0], rtol=1e-14)


def pin_weights_via_onehot_values(ref):
    """With v_j = e_j (D = L) the output row is the weight row: it sums to 1,
    is nonnegative and holds exact zeros at keys masked by -1e9."""
    B, N, L, H = 1, 2, 24, 2
    w = random_problem(B, N, L, H, L, dtype="bf16", seed=12, mask="random", pair="normal", mask_frac=0.25,
                       bias_scale=2.0)
    eye = np.zeros((B, N, L, H, L), np.float32)
    for j in range(L):
        eye[:, :, j, :, j] = 1
    o, _ = ref(w.q, w.k, _st(eye, "bf16"), w.mask, w.pair, "bf16")
    np.testing.assert_allclose(o.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert (o >= 0).all()
    masked = _f64(w.mask, "bf16")[:, :, 0, 0, :] < -1e8  # [B, N, L]
    for n in range(N):
        assert np.all(o[0, n][:, :, masked[0, n]] == 0.0)
        assert np.all(o[0, n][:, :, ~masked[0, n]] > 0.0)


def pin_zero_bias_is_plain_attention(ref):
    """All-zero biases give exactly the no-bias result (plain scaled dot-product attention)."""
    w = random_problem(1, 2, 21, 2, 8, dtype="bf16", seed=13, mask="zero", pair="zero")
    o1, l1 = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    o2, l2 = ref(w.q, w.k, w.v, None, None, "bf16")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------------------
# Invariants.
# ---------------------------------------------------------------------------
def _pb(B=2, N=3, L=13, H=2, D=8, seed=21):
    return random_problem(B, N, L, H, D, dtype="bf16", seed=seed, mask="normal", pair="normal", bias_scale=2.0)


def pin_permute_n(ref):
    """Permuting the N axis of q, k, v and mask permutes out and lse the same way."""
    w = _pb()
    o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    p = np.array([2, 0, 1])
    o2, l2 = ref(w.q[:, p], w.k[:, p], w.v[:, p], w.mask[:, p], w.pair, "bf16")
    np.testing.assert_allclose(o2, o[:, p], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l2, l[:, p], rtol=1e-14, atol=1e-15)


def pin_permute_keys(ref):
    """Permuting keys (k, v rows, mask entries, pair columns) leaves out and lse unchanged."""
    w = _pb()
    o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    p = np.random.default_rng(3).permutation(w.shape[2])
    o2, l2 = ref(w.q, w.k[:, :, p], w.v[:, :, p], w.mask[..., p], w.pair[..., p], "bf16")
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l, rtol=1e-13, atol=1e-14)


def pin_permute_queries(ref):
    """Permuting queries (q rows and pair rows) permutes out and lse."""
    w = _pb()
    o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    p = np.random.default_rng(4).permutation(w.shape[2])
    o2, l2 = ref(w.q[:, :, p], w.k, w.v, w.mask, w.pair[:, :, :, p, :], "bf16")
    np.testing.assert_allclose(o2, o[:, :, p], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l2, l[..., p], rtol=1e-14, atol=1e-15)


def pin_row_shift(ref):
    """Adding c to every pair entry of one (h, i) row leaves out unchanged and adds c to lse."""
    w = _pb()
    o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    pf = storage_to_f32(w.pair, "bf16").copy()
    pf[0, 0, 1, 5, :] += np.float32(4.0)  # exact in bf16 for these magnitudes? checked below
    shifted = to_storage(pf, "bf16")
    exact = np.array_equal(storage_to_f32(shifted, "bf16")[0, 0, 1, 5] - 4.0, storage_to_f32(w.pair, "bf16")[0, 0, 1, 5])
    o2, l2 = ref(w.q, w.k, w.v, w.mask, shifted, "bf16")
    if exact:
        np.testing.assert_allclose(o2[0, :, 5, 1], o[0, :, 5, 1], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l2[0, :, 1, 5], l[0, :, 1, 5] + 4.0, rtol=1e-13)
    # rows other than (h=1, i=5) do not move at all
    keep = np.ones(o.shape, bool)
    keep[0, :, 5, 1] = False
    np.testing.assert_array_equal(o2[keep], o[keep])
    # f32 storage: any shift is exact enough to check
    wf = random_problem(1, 2, 9, 2, 4, dtype="f32", seed=22, mask="normal", pair="normal")
    o, l = ref(wf.q, wf.k, wf.v, wf.mask, wf.pair, "f32")
    p2 = wf.pair.copy()
    p2[0, 0, 0, 2, :] += np.float32(0.75)
    o2, l2 = ref(wf.q, wf.k, wf.v, wf.mask, p2, "f32")
    np.testing.assert_allclose(o2[0, :, 2, 0], o[0, :, 2, 0], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(l2[0, :, 0, 2], l[0, :, 0, 2] + 0.75, rtol=1e-6)


def pin_all_keys_finite_mask(ref):
    """Every key of a sequence masked by the same finite -1e9 (stored exactly: f32, and bf16's nearest
    value): softmax is invariant under a constant shift, so out equals the unmasked result and lse moves
    by exactly the mask value (fp64 keeps the score differences next to 1e9 to ~1e-7)."""
    for dtype in ("f32", "bf16"):
        w = random_problem(1, 3, 11, 2, 8, dtype=dtype, seed=31, mask="zero", pair="normal")
        o0, l0 = ref(w.q, w.k, w.v, w.mask, w.pair, dtype)
        mf = np.zeros(storage_to_f32(w.mask, dtype).shape, np.float32)
        mf[0, 1] = -1e9
        masked = to_storage(mf, dtype)
        c = float(storage_to_f32(masked, dtype)[0, 1, 0, 0, 0])  # the stored value of -1e9
        o1, l1 = ref(w.q, w.k, w.v, masked, w.pair, dtype)
        np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-6)
        np.testing.assert_allclose(l1[0, 1], l0[0, 1] + c, rtol=0, atol=1e-6)
        np.testing.assert_array_equal(l1[0, [0, 2]], l0[0, [0, 2]])


def pin_heads_independent(ref):
    """Changing head 0's inputs leaves head 1's outputs bit-identical."""
    w = _pb()
    o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    q, k, v, p = (x.copy() for x in (w.q, w.k, w.v, w.pair))
    rng = np.random.default_rng(5)
    for x in (q, k, v):
        x[:, :, :, 0, :] = rng.integers(0, 0x3F00, x[:, :, :, 0, :].shape, dtype=np.uint16)
    p[:, :, 0] = rng.integers(0, 0x3F00, p[:, :, 0].shape, dtype=np.uint16)
    o2, l2 = ref(q, k, v, w.mask, p, "bf16")
    np.testing.assert_array_equal(o2[:, :, :, 1], o[:, :, :, 1])
    np.testing.assert_array_equal(l2[:, :, 1], l[:, :, 1])
    assert not np.array_equal(o2[:, :, :, 0], o[:, :, :, 0])


def pin_split_batch(ref):
    """Evaluating B and N slices separately gives the same result as one call."""
    w = _pb()
    o, l = ref(w.q, w.k, w.v, w.mask, w.pair, "bf16")
    for b in range(w.shape[0]):
        for n in range(w.shape[1]):
            o1, l1 = ref(w.q[b:b + 1, n:n + 1], w.k[b:b + 1, n:n + 1], w.v[b:b + 1, n:n + 1],
                         w.mask[b:b + 1, n:n + 1], w.pair[b:b + 1], "bf16")
            np.testing.assert_array_equal(o1[0, 0], o[b, n])
            np.testing.assert_array_equal(l1[0, 0], l[b, n])


def pin_dtype_widening(ref):
    """Values exactly representable in bf16 and f16 give identical results in all storage types."""
    rng = np.random.default_rng(14)
    shape = (1, 2, 10, 2, 8)
    # multiples of 1/8 in [-4, 4): exact in bf16, f16 and f32
    q, k, v = (rng.integers(-32, 32, shape).astype(np.float32) / 8 for _ in range(3))
    mask = rng.integers(-16, 16, (1, 2, 1, 1, 10)).astype(np.float32) / 8
    pair = rng.integers(-16, 16, (1, 1, 2, 10, 10)).astype(np.float32) / 8
    res = [ref(*(_st(x, dt) for x in (q, k, v, mask, pair)), dt) for dt in ("f32", "bf16", "f16")]
    for o, l in res[1:]:
        np.testing.assert_array_equal(o, res[0][0])
        np.testing.assert_array_equal(l, res[0][1])
    # subnormal, large and negative f16 values decode to their exact values
    vals = np.array([2.0 ** -24, -3 * 2.0 ** -20, 65504.0, -0.0, 1.5, -1024.0], np.float32)
    vv = np.zeros((1, 1, 1, 1, 6), np.float32)
    vv[0, 0, 0, 0] = vals
    o, _ = ref(_st(np.zeros_like(vv), "f16"), _st(np.zeros_like(vv), "f16"), _st(vv, "f16"), None, None, "f16")
    np.testing.assert_array_equal(o[0, 0, 0, 0], vals.astype(np.float64))


def pin_all_keys_neg_inf(ref):
    """A row whose every key is -inf (f16 storage of -1e9 overflows to -inf) returns out = 0, lse = -inf;
    rows with one finite key are unaffected."""
    L = 4
    q = np.zeros((1, 2, L, 1, 4), np.float32)
    v = np.ones_like(q)
    mask = np.full((1, 2, 1, 1, L), NEG, np.float32)
    mask[0, 1, 0, 0, 2] = 0
    o, l = ref(_st(q, "f16"), _st(q, "f16"), _st(v, "f16"), _st(mask, "f16"), None, "f16")
    assert np.all(o[0, 0] == 0) and np.all(np.isneginf(l[0, 0]))
    np.testing.assert_array_equal(o[0, 1], 1.0)
    np.testing.assert_array_equal(l[0, 1], 0.0)


ALL_PINS = [
    pin_hand_worked, pin_brute_force, pin_torch_sdpa, pin_zero_query_mean, pin_single_key,
    pin_uniform_values, pin_one_boosted_key, pin_two_keys_sigmoid, pin_weights_via_onehot_values,
    pin_zero_bias_is_plain_attention, pin_permute_n, pin_permute_keys, pin_permute_queries,
    pin_row_shift, pin_heads_independent, pin_split_batch, pin_dtype_widening, pin_all_keys_neg_inf,
    pin_all_keys_finite_mask,
]
