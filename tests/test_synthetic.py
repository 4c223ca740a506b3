"""Seeded input generators: rounding, determinism and the workload recipes."""
import numpy as np
import pytest
import torch

import synthetic as S


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1e9, -1e9, 3.0e38, np.inf, -np.inf], np.float32)]).astype(np.float32)
    ours = S.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert S.bf16_bits_to_f32(S.f32_to_bf16_bits(np.float32([-1e9])))[0] == -998244352.0


def test_f16_storage_roundtrip():
    x = np.array([1.0, -2.5, 65504.0, 2.0 ** -24, -1e9], np.float32)
    back = S.storage_to_f32(S.to_storage(x, "f16"), "f16")
    np.testing.assert_array_equal(back[:4], x[:4])
    assert back[4] == -np.inf


def test_deterministic():
    a = S.random_problem(1, 2, 9, 2, 8, seed=4)
    b = S.random_problem(1, 2, 9, 2, 8, seed=4)
    for x, y in zip((a.q, a.k, a.v, a.mask, a.pair), (b.q, b.k, b.v, b.mask, b.pair)):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_int8_pair_bias_is_exact(dtype):
    w = S.random_problem(2, 1, 37, 3, 8, dtype=dtype, seed=11, pair="int8")
    pf = S.storage_to_f32(w.pair, dtype).astype(np.float64)
    k = pf * 32
    np.testing.assert_array_equal(k, np.round(k))          # every value is k / 32 exactly
    assert k.min() >= -128 and k.max() <= 127
    assert len(np.unique(k)) > 200                          # and the int8 range is used
    np.testing.assert_array_equal(w.pair, S.random_problem(2, 1, 37, 3, 8, dtype=dtype, seed=11, pair="int8").pair)


@pytest.mark.parametrize("c", [1, 2, 4])
def test_workload_recipes(c):
    w = S.workload(c)
    B, N, L, H, D = w.shape
    assert w.q.shape == (B, N, L, H, D)
    mf = None if w.mask is None else S.storage_to_f32(w.mask, w.dtype)
    if c == 1:
        assert w.dtype == "f32" and (mf[..., 56:] == -1e9).all() and (mf[..., :56] == 0).all()
        assert w.pair.shape == (1, 1, 8, 64, 64)
    if c == 2:
        t = w.meta["tails"]
        assert t.min() >= 0 and t.max() <= 25
        for n in range(N):
            assert (mf[0, n, 0, 0, L - t[n]:] < -9e8).all() and (mf[0, n, 0, 0, :L - t[n]] == 0).all()
    if c == 4:
        assert (mf[..., 368:] < -9e8).all() and (mf[..., :368] == 0).all()
        pf = S.storage_to_f32(w.pair, "bf16")
        assert pf.shape == (1, 1, 4, 384, 384)
        assert 0.8 < pf.std() < 1.2  # z ~ N(0,1) projected by W ~ N(0, 1/128): unit variance
        assert not np.allclose(pf[0, 0, 0], pf[0, 0, 0].T)  # asymmetric: a transposed read shows


def test_workload_5_is_transposed_projection():
    """Ending-node pair bias is the starting-node projection with i and j swapped."""
    L, H = 24, 2
    import numpy as np
    r = [np.random.default_rng(s) for s in np.random.SeedSequence(3).spawn(2)]
    start = S._projected_pair(*r, L, H, transpose=False)
    r = [np.random.default_rng(s) for s in np.random.SeedSequence(3).spawn(2)]
    end = S._projected_pair(*r, L, H, transpose=True)
    np.testing.assert_array_equal(end[0, 0], start[0, 0].transpose(0, 2, 1))


def test_sample_rows():
    idx = S.sample_rows((2, 3, 10, 4, 8), 50, seed=1)
    assert idx.shape[1] == 4
    assert len({tuple(r) for r in idx}) == len(idx)
    assert (idx.min(0) >= 0).all() and (idx.max(0) < np.array([2, 3, 4, 10])).all()
