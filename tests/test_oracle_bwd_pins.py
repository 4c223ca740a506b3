"""The fp64 oracle's backward pass against its pins (CPU only)."""
import pytest

import oracle_bwd_pins


@pytest.fixture(scope="module")
def gref(oracle_lib):
    def _gref(q, k, v, mask, pair, dout, dtype):
        return oracle_lib.bwd(q, k, v, mask, pair, dout, dtype=dtype, nthreads=4)
    return _gref


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_oracle_bwd_pin(gref, pin):
    pin(gref)


def test_bwd_threads_agree(oracle_lib):
    """The pair gradient's per-thread partial sums give the same result for any thread count."""
    import numpy as np
    from synthetic import random_dout, random_problem
    w = random_problem(2, 5, 19, 2, 8, dtype="bf16", seed=61, mask="tail", pair="normal", mask_frac=0.3)
    dout = random_dout(w.shape, "bf16", seed=62)
    one = oracle_lib.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="bf16", nthreads=1)
    many = oracle_lib.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="bf16", nthreads=6)
    for a, b in zip(one[:4], many[:4]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(many[4], one[4], rtol=1e-13, atol=1e-15)


def test_bwd_rejects_bias_gradient_without_bias(oracle_lib):
    import ctypes
    import numpy as np
    from synthetic import random_dout, random_problem
    w = random_problem(1, 1, 5, 1, 4, dtype="f32", seed=1, mask=None, pair=None)
    dout = random_dout(w.shape, "f32", seed=2)
    buf = [np.zeros(w.shape) for _ in range(3)]
    dm = np.zeros((1, 1, 1, 1, 5))
    lib = oracle_lib._load()
    rc = lib.evo_ref_bwd(w.q.ctypes.data, w.k.ctypes.data, w.v.ctypes.data, None, None, dout.ctypes.data,
                         0, 1, 1, 5, 1, 4, buf[0].ctypes.data, buf[1].ctypes.data, buf[2].ctypes.data,
                         dm.ctypes.data, None, 1)
    assert rc != 0
