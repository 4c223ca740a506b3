"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle_pins


@pytest.fixture(scope="module")
def ref(oracle_lib):
    def _ref(q, k, v, mask, pair, dtype):
        return oracle_lib.fwd(q, k, v, mask, pair, dtype=dtype, nthreads=4)
    return _ref


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(ref, pin):
    pin(ref)


def test_rows_match_full(oracle_lib):
    """The sampled-row entry point returns the same rows as the full evaluation."""
    import numpy as np
    from synthetic import random_problem, sample_rows
    w = random_problem(2, 3, 29, 2, 16, dtype="bf16", seed=31, mask="tail", pair="normal", mask_frac=0.3)
    o, l = oracle_lib.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=2)
    idx = sample_rows(w.shape, 40, seed=3)
    ro, rl = oracle_lib.rows(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", idx=idx, nthreads=2)
    b, n, h, i = idx.T
    np.testing.assert_array_equal(ro, o[b, n, i, h, :])
    np.testing.assert_array_equal(rl, l[b, n, h, i])


def test_rows_rejects_out_of_range(oracle_lib):
    import numpy as np
    from synthetic import random_problem
    w = random_problem(1, 1, 5, 1, 4, dtype="f32", seed=1, mask=None, pair=None)
    with pytest.raises(RuntimeError):
        oracle_lib.rows(w.q, w.k, w.v, None, None, dtype="f32", idx=np.array([[0, 0, 0, 5]]))


def test_guide_facts_fixture():
    """The page facts the tests rely on are present in the golden fixture."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "ds4sci_guide_facts.json")) as f:
        facts = json.load(f)
    assert [1, 256, 256, 4, 32] in facts["unit_test"]["shapes_B_N_L_H_D"]
    assert facts["unit_test"]["tolerance"]["bfloat16"] == 5e-2
    assert facts["layouts"]["pair_bias"] == "[B, 1, H, L, L]"
