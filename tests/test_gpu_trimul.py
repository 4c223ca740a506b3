"""Triangle multiplication: HIP kernel vs the fp64 oracle, element by element, through the C ABI.

Tolerances, as errors normalised by max|x_ref| of each test: bf16 max <= 8e-3,
mean <= 2e-3; f16 max <= 2e-3, mean <= 5e-4.  The kernel multiplies the
stored values exactly and accumulates in fp32 (relative error ~L * 2^-24 of
sum |a w|, below 1e-4 here); the budget is the single rounding of x to the
storage format (half an ulp: 2^-9 relative in bf16, 2^-12 in f16), allowed
twice.  Outputs are poisoned with NaN first.
"""
import numpy as np
import pytest

import oracle
import synthetic as S

pytestmark = pytest.mark.gpu

TOL = {"bf16": (8e-3, 2e-3), "f16": (2e-3, 5e-4)}
THREADS = min(16, oracle.default_threads())


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401
    return torch


def dev(torch, x, dtype, extra=0):
    t = torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    if not extra:
        return t.to("cuda")
    buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device="cuda")
    buf[: t.numel()] = t.reshape(-1).to("cuda")
    return buf[: t.numel()].view(t.shape)


def compare(x, ref, dtype, what):
    assert np.isfinite(x).all(), f"{what}: non-finite output"
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(x - ref) / scale
    print(f"  {what}: max={err.max():.3e} mean={err.mean():.3e} (max|ref| {scale:.3g})", flush=True)
    assert err.max() <= TOL[dtype][0] and err.mean() <= TOL[dtype][1], what


def run(torch, a, w, dtype, direction, extra=0):
    import evoformer_biased_attention_amd as E
    ta, tw = dev(torch, a, dtype, extra), dev(torch, w, dtype, extra)
    x = torch.full_like(ta, float("nan"))
    print(f"  trimul {a.shape} {dtype} {direction}", flush=True)
    E.trimul(ta, tw, direction, out=x)
    torch.cuda.synchronize()
    return x.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("L", [1, 3, 8, 16, 31, 64, 72, 99, 128, 130, 136, 200, 257, 264])
def test_trimul_ragged(torch_dev, L, direction, dtype):
    """L % 8 != 0 (1, 3, 31, 99, 130, 257) stages the operands through registers."""
    a, w = S.trimul_problem(2, 3, L, dtype, seed=L)
    compare(run(torch_dev, a, w, dtype, direction), oracle.trimul(a, w, dtype, direction, nthreads=THREADS), dtype,
            f"L={L} {direction}")


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_trimul_workload_sampled_channels(torch_dev, direction):
    """The named size (B=1, C=128, L=384) in one launch; the oracle evaluates channels 0, 37 and 127."""
    c = S.TRIMUL_WORKLOAD
    a, w = S.trimul_problem(c["B"], c["C"], c["L"], c["dtype"], seed=384)
    x = run(torch_dev, a, w, c["dtype"], direction)
    for ch in (0, 37, 127):
        ref = oracle.trimul(a[:, ch:ch + 1], w[:, ch:ch + 1], c["dtype"], direction, nthreads=THREADS)
        compare(x[:, ch:ch + 1], ref, c["dtype"], f"{c['name']} channel {ch} {direction}")


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("L", [72, 77])
def test_trimul_rows_past_L_read_as_zero(torch_dev, direction, L):
    """NaN right after both inputs, L = 72 (partial 128 tile and partial 64 contraction step) and L = 77
    (staged copies: the last chunk of the plane crosses the end of the range)."""
    a, w = S.trimul_problem(1, 2, L, "bf16", seed=5)
    x = run(torch_dev, a, w, "bf16", direction, extra=256 * L)
    compare(x, oracle.trimul(a, w, "bf16", direction, nthreads=THREADS), "bf16", f"NaN tail {direction}")


def test_trimul_same_operand(torch_dev):
    """a and w may be one tensor; outgoing(a, a) is symmetric."""
    a, _ = S.trimul_problem(1, 2, 64, "bf16", seed=6)
    x = run(torch_dev, a, a, "bf16", "outgoing")
    compare(x, oracle.trimul(a, a, "bf16", "outgoing", nthreads=THREADS), "bf16", "a = w")
    np.testing.assert_array_equal(x, x.transpose(0, 1, 3, 2))


def test_trimul_errors_write_nothing(torch_dev):
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    a = torch.zeros((1, 2, 100, 100), dtype=torch.float32, device="cuda")
    x = torch.full_like(a, 7.0)
    assert E.evo_trimul(a, a, x, (1, 2, 100), 0, E.EVO_DTYPE_F32) == E.EVO_ERR_UNSUPPORTED
    assert E.evo_trimul(a, a, a, (1, 2, 100), 0, E.EVO_DTYPE_F32) == E.EVO_ERR_ALIASING
    torch.cuda.synchronize()
    assert bool((x == 7.0).all())
