"""The differentiable call evoformer_attention(q, k, v, [mask_bias, pair_bias]) against the fp64 oracle.

Forward output and every gradient (through torch.autograd, loss = sum(out * dout)) are compared with
oracle.fwd and oracle.bwd under the tolerances of the forward and backward parity tests.  A bias that
does not require a gradient gets none (and its kernel work is skipped); a missing bias behaves as no
bias; views such as the transposed tensors of ending-node attention are used in place.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from test_gpu_bwd_parity import THREADS, compare_grads, f64, to_dev
from test_gpu_parity import compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401
    return torch


def leaf(torch, x, dtype, grad=True):
    if x is None:
        return None
    return to_dev(torch, x, dtype).requires_grad_(grad)


def run(torch, w, dout, grad_mask=True, grad_pair=True):
    """Forward and backward through evoformer_attention; returns (out, [dq, dk, dv, dmask, dpair]) as
    float64 numpy (None for a gradient that was not requested)."""
    import evoformer_biased_attention_amd as E
    q, k, v = (leaf(torch, x, w.dtype) for x in (w.q, w.k, w.v))
    mask = leaf(torch, w.mask, w.dtype, grad_mask)
    pair = leaf(torch, w.pair, w.dtype, grad_pair)
    out = E.evoformer_attention(q, k, v, [mask, pair])
    (out.float() * to_dev(torch, dout, w.dtype).float()).sum().backward()
    torch.cuda.synchronize()
    grads = [q.grad, k.grad, v.grad, mask.grad if mask is not None else None,
             pair.grad if pair is not None else None]
    return f64(out.detach()), [f64(g) for g in grads]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("L", [64, 77])
@pytest.mark.parametrize("D", [32, 64])
def test_autograd_matches_oracle(torch_dev, D, L, dtype):
    """D = 64 chains the 16-bit forward (two 32-wide halves) into the matrix-core backward."""
    w = S.random_problem(1, 4, L, 2, D, dtype=dtype, seed=L + 500 + D, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, dtype, seed=L + 501)
    o, grads = run(torch_dev, w, dout)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, None, ro, None, dtype, f"autograd forward L={L} D={D}")
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(grads, list(want), dtype, f"autograd L={L} D={D}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_broadcast_mask(torch_dev, dtype):
    """A mask given once per batch element and expand()ed over N (stride 0), requiring a gradient: the call
    materialises it, and the gradient that reaches the [B,1,1,1,L] leaf is the oracle's mask gradient
    summed over N."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = 1, 5, 72, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=540, mask=None, pair="normal")
    mf = np.zeros((B, 1, 1, 1, L), np.float32)
    mf[..., L - 9:] = -1e9
    mf[..., :5] = np.float32(0.75)
    base = S.to_storage(mf, dtype)
    w.mask = np.ascontiguousarray(np.broadcast_to(base, (B, N, 1, 1, L)))
    dout = S.random_dout(w.shape, dtype, seed=541)
    q, k, v = (leaf(torch, x, dtype) for x in (w.q, w.k, w.v))
    mleaf = leaf(torch, base, dtype)
    pair = leaf(torch, w.pair, dtype, False)
    out = E.evoformer_attention(q, k, v, [mleaf.expand(B, N, 1, 1, L), pair])
    (out.float() * to_dev(torch, dout, dtype).float()).sum().backward()
    torch.cuda.synchronize()
    ro, _ = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(f64(out.detach()), None, ro, None, dtype, "broadcast mask, forward")
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    got = [f64(q.grad), f64(k.grad), f64(v.grad), f64(mleaf.grad)]
    compare_grads(got, [want[0], want[1], want[2], want[3].sum(axis=1, keepdims=True)], dtype,
                  "broadcast mask")
    # the low-level wrapper refuses to write a gradient into a broadcast view
    with pytest.raises(ValueError):
        E.bwd(q.detach(), k.detach(), v.detach(), mleaf.detach().expand(B, N, 1, 1, L), None, out.detach(),
              torch.zeros((B, N, H, L), dtype=torch.float32, device="cuda"), to_dev(torch, dout, dtype))


def test_autograd_bias_gradients_only_on_request(torch_dev):
    w = S.random_problem(1, 3, 80, 2, 32, dtype="bf16", seed=510, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=511)
    _, all_grads = run(torch_dev, w, dout)
    _, some = run(torch_dev, w, dout, grad_mask=False, grad_pair=False)
    assert some[3] is None and some[4] is None
    for a, b in zip(all_grads[:3], some[:3]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("which", ["mask", "pair", "none"])
def test_autograd_missing_biases(torch_dev, which):
    """A bias given as None (or left out of the list) is no bias."""
    w = S.random_problem(1, 3, 48, 2, 16, dtype="f16", seed=520 + len(which), mask="tail" if which == "mask" else None,
                         pair="normal" if which == "pair" else None)
    dout = S.random_dout(w.shape, "f16", seed=521)
    o, grads = run(torch_dev, w, dout)
    ro, _ = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="f16", nthreads=THREADS)
    compare(o, None, ro, None, "f16", f"no {which} bias")
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="f16", nthreads=THREADS)
    compare_grads(grads, list(want), "f16", f"autograd without {which}")


def test_autograd_transposed_views(torch_dev):
    """Ending-node attention: q, k, v and dO are permuted views of X[B, L, N, H, D]; out and the gradients
    come back in the same layout, with no copies, and match the oracle on dense transposed copies."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = 1, 40, 56, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=530, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=531)
    X = {n: np.ascontiguousarray(getattr(w, n).transpose(0, 2, 1, 3, 4)) for n in ("q", "k", "v")}
    xq, xk, xv = (to_dev(torch, X[n], "bf16").requires_grad_(True) for n in ("q", "k", "v"))
    perm = lambda t: t.permute(0, 2, 1, 3, 4)
    mask, pair = leaf(torch, w.mask, "bf16"), leaf(torch, w.pair, "bf16")
    out = E.evoformer_attention(perm(xq), perm(xk), perm(xv), [mask, pair])
    assert out.stride() == perm(xq).stride()  # written in place of the view's layout
    do = perm(to_dev(torch, np.ascontiguousarray(dout.transpose(0, 2, 1, 3, 4)), "bf16"))
    (out.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    grads = [f64(perm(t.grad)) for t in (xq, xk, xv)] + [f64(mask.grad), f64(pair.grad)]
    ro, _ = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    compare(f64(out.detach()), None, ro, None, "bf16", "transposed views, forward")
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="bf16", nthreads=THREADS)
    compare_grads(grads, list(want), "bf16", "transposed views")
