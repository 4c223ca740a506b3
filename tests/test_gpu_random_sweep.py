"""A seeded sweep of random problems through both passes, against the full oracles.

Each case draws a dtype, a head dimension, B, N, L, H, the bias subset and the kind of mask (tail padding,
random keys, or N(0, s^2) values) and a bias scale, then checks the forward (out and lse) and the backward
(every gradient and delta) element by element at the same tolerances as the fixed-shape tests.  The cases
cross the kernel families' boundaries: 16-bit and fp32 matrix-core kernels (D = 8 padded with zero columns on
both), aligned and staged bias rows (L % 8 and L % 4), partial 64-key blocks, and the pair gradient's
workspace split over N when N is large enough.  A sequence whose every key would carry the finite -1e9 mask
(no parity claim for such rows) gets its first key unmasked.

The bias gradients are sums of dS over heads and queries (mask) or over N (pair), and can be small against the
terms they sum (few keys, few heads).  delta is formed from the forward's stored, rounded out rather than the
exact O (reading B3), which moves every dS of row (b, n, h, i) by P * dO . (O - out); for those two gradients the
allowed error therefore adds that shift, bounded with P <= 1 and summed over the same axes, to the usual bound:
sum over (h, i) of |dO . (O - out)| for dmask, sum over n for dpair, with O the oracle's and out the kernel's.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from test_gpu_bwd_parity import NAMES, THREADS, TOL as BWD_TOL, compare_delta, run_bwd
from test_gpu_parity import parity_full, say

pytestmark = pytest.mark.gpu

CASES = 100


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch


def draw(i):
    rng = np.random.default_rng(9000 + i)
    dtype = ["f32", "bf16", "f16"][rng.integers(3)]
    D = int(rng.choice([8, 16, 32, 64]))
    L = int(rng.choice([rng.integers(1, 20), rng.integers(20, 140), 64 * rng.integers(1, 4) + rng.integers(-1, 2),
                        rng.integers(140, 300)]))
    L = max(L, 1)
    B = int(rng.integers(1, 3))
    N = int(rng.choice([rng.integers(1, 7), rng.integers(16, 26)]))
    H = int(rng.integers(1, 5))
    mask = [None, "tail", "random", "normal"][rng.integers(4)]
    pair = [None, "normal"][rng.integers(2)]
    frac = float(rng.uniform(0.05, 0.4))
    scale = float(rng.choice([1.0, 4.0]))
    return dict(shape=(B, N, L, H, D), dtype=dtype, mask=mask, pair=pair, frac=frac, scale=scale, seed=9100 + i)


def problem(c):
    B, N, L, H, D = c["shape"]
    w = S.random_problem(B, N, L, H, D, dtype=c["dtype"], seed=c["seed"], mask=c["mask"], pair=c["pair"],
                         mask_frac=c["frac"], bias_scale=c["scale"])
    if w.mask is not None and c["mask"] in ("tail", "random"):
        mf = S.storage_to_f32(w.mask, c["dtype"]).copy()
        dead = np.all(mf <= -1e9, axis=-1)  # [B, N, 1, 1]
        if dead.any():
            mf[..., 0][dead] = 0.0
            w.mask = S.to_storage(mf, c["dtype"])
    w.name = f"sweep{c['seed']}"
    return w


def compare_bwd(got, want, out_used, w, dout):
    """Every gradient against the oracle's; the bias gradients with the delta shift added to their bound."""
    tol = BWD_TOL[w.dtype]
    ro, _ = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=w.dtype, nthreads=THREADS)
    dof = S.storage_to_f32(dout, w.dtype).astype(np.float64)
    shift = np.abs(np.einsum("bnlhd,bnlhd->bnhl", dof, ro - out_used))  # |dO . (O - out)| per row
    extra = {"dmask": shift.sum(axis=(2, 3))[:, :, None, None, None],        # [B, N, 1, 1, 1]
             "dpair": shift.sum(axis=1)[:, None, :, :, None]}                # [B, 1, H, L, 1]
    for name, g, r in zip(NAMES, got, want):
        assert (g is None) == (r is None), f"{w.name} {name}: presence differs"
        if g is None:
            continue
        assert np.isfinite(g).all(), f"{w.name} {name}: non-finite values"
        scale = max(np.abs(r).max(), 1e-30)
        bound = tol["max"] * scale + extra.get(name, 0.0)
        err = np.abs(g - r)
        msg = (f"{w.name} {name}: max|d|/max|ref|={err.max() / scale:.3e} mean={err.mean() / scale:.3e}, "
               f"delta shift up to {np.max(extra.get(name, 0.0)) / scale:.3e} of max|ref|")
        say("  " + msg)
        assert (err <= bound).all(), msg
        assert err.mean() <= tol["mean"] * scale + np.mean(np.broadcast_to(extra.get(name, 0.0), err.shape)), msg


@pytest.mark.parametrize("i", range(CASES))
def test_random_problem_both_passes(torch_dev, i):
    c = draw(i)
    say(f"case {i}: {c}")
    w = problem(c)
    parity_full(torch_dev, w)
    if c["shape"][2] > 1:  # one key: the gradients other than dv vanish (covered by the fixed-shape tests)
        dout = S.random_dout(w.shape, c["dtype"], seed=c["seed"] + 1)
        got, delta, out_used = run_bwd(torch_dev, w, dout)
        want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=w.dtype, nthreads=THREADS)
        compare_bwd(got, list(want), out_used, w, dout)
        compare_delta(delta, w, dout, w.name)
