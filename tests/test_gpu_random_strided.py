"""A seeded sweep of random memory layouts through both strided entry points, against the oracles on dense
copies of the same values.

Each case draws a problem as in the dense sweep and a layout for it: Q, K, V, dO (and so out, dQ, dK, dV)
dense, transposed (X[B,L,N,H,D], the ending-node and column variants) or with padded rows (H*D plus a
16-byte multiple between rows); mask rows and pair rows and matrices padded by random amounts, aligned or not;
the LSE and delta rows padded; with or without the pair gradient's workspace.  out is checked against the
oracle's forward, the gradients and delta as in the dense sweep (the bias gradients with the delta shift of
reading B3 added to their bound), and the pair gradient's padding must stay NaN.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from test_gpu_bwd_parity import THREADS, compare_delta, f64, say, to_dev
from test_gpu_bwd_strided import strided_bwd
from test_gpu_parity import compare as compare_fwd
from test_gpu_random_sweep import compare_bwd, draw, problem

pytestmark = pytest.mark.gpu

CASES = 80


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch


def rows_view(torch, x, dtype, mode, pad):
    """x: [B,N,L,H,D] storage -> a device view in the given layout with the same values."""
    B, N, L, H, D = x.shape
    if mode == "dense":
        return to_dev(torch, x, dtype)
    if mode == "transposed":
        return to_dev(torch, np.ascontiguousarray(x.transpose(0, 2, 1, 3, 4)), dtype).permute(0, 2, 1, 3, 4)
    buf = np.zeros((B, N, L, H * D + pad), x.dtype)
    buf[..., : H * D] = x.reshape(B, N, L, H * D)
    return to_dev(torch, buf, dtype)[..., : H * D].view(B, N, L, H, D)


def layout_case(i, c):
    rng = np.random.default_rng(7700 + i)
    es = 4 if c["dtype"] == "f32" else 2
    mode = ["dense", "transposed", "padded"][rng.integers(3)]
    return dict(mode=mode, row_pad=int(rng.integers(1, 4)) * 16 // es, mask_pad=int(rng.choice([0, 1, 3, 8])),
                pair_pad_i=int(rng.choice([0, 1, 3, 8])), pair_pad_l=int(rng.choice([0, 2, 5])),
                lse_pad=int(rng.choice([0, 3, 32])), use_ws=bool(rng.integers(2)))


@pytest.mark.parametrize("i", range(CASES))
def test_random_layout_both_passes(torch_dev, i):
    torch = torch_dev
    c = draw(500 + i)
    B, N, L, H, D = c["shape"]
    if L == 1:
        c["shape"] = (B, N, 2, H, D)  # one key: the gradients other than dv vanish
        B, N, L, H, D = c["shape"]
    lay = layout_case(i, c)
    say(f"case {i}: {c} layout {lay}")
    w = problem(c)
    dtype = w.dtype
    dout = S.random_dout(w.shape, dtype, seed=c["seed"] + 1)
    q, k, v, do = (rows_view(torch, x, dtype, lay["mode"], lay["row_pad"]) for x in (w.q, w.k, w.v, dout))
    mask = None
    if w.mask is not None:
        wide = np.zeros((B, N, 1, 1, L + lay["mask_pad"]), w.mask.dtype)
        wide[..., :L] = w.mask
        mask = to_dev(torch, wide, dtype)[..., :L]
    pair, pair_store, pl, pi = None, None, L + lay["pair_pad_l"], L + lay["pair_pad_i"]
    if w.pair is not None:
        wide = np.zeros((B, 1, H, pl, pi), w.pair.dtype)
        wide[..., :L, :L] = w.pair
        full = to_dev(torch, wide, dtype)
        pair = full[..., :L, :L]
        pair_store = torch.empty_like(full).reshape(-1)
    got, delta, raw = strided_bwd(torch, q, k, v, mask, pair, do, lse_row=L + lay["lse_pad"], use_ws=lay["use_ws"],
                                  pair_storage=pair_store)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    out_used = f64(raw[6])
    compare_fwd(out_used, None, ro, None, dtype, f"{w.name} out")
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_bwd(got, list(want), out_used, w, dout)
    compare_delta(delta, w, dout, w.name)
    if pair_store is not None:
        padded = pair_store.view(B, 1, H, pl, pi).float()
        assert torch.isnan(padded[..., L:, :]).all() and torch.isnan(padded[..., :L, L:]).all(), "dpair padding"
