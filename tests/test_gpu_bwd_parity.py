"""Backward pass: HIP path vs the fp64 oracle, element by element, through the C ABI.

The HIP backward takes the forward pass's out and lse, from the HIP forward
(the pipeline a caller runs) unless a test asks for the oracle's, rounded to
the storage format.  The oracle recomputes everything from q, k, v, the biases
and dO in fp64 and never sees a GPU value.  Every comparison prints its
normalised errors, and the largest per dtype and gradient is printed when the
module ends (the measured margin under each bound).

Tolerances, per gradient tensor G, as errors normalised by max|G_ref|:
  f32:  max <= 1e-4, mean <= 1e-5
  bf16: max <= 1.6e-2, mean <= 2e-3
  f16:  max <= 4e-3, mean <= 5e-4
The backward arithmetic is fp32; the 16-bit budgets come from rounding each
gradient to the storage format once (half an ulp: 2^-9 relative in bf16,
2^-12 in f16) and from delta = dO . out using the stored (rounded) out, whose
error moves every dS_ij of a row by P_ij times that row's delta error.  The
max bounds allow four ulps of the largest value (bf16 ulp 2^-8, f16 2^-10):
two for the final rounding and two for delta.  The delta term is the larger
one where the softmax is peaked (biases of scale 8): one key takes almost all
the weight, dS_ij = P_ij dO_i . (v_j - out_i) becomes a small difference and
the rounding of out reaches it undiminished.  The guide's own unit test
accepts 5e-2 (bf16) and 1e-2 (fp16) on the gradients (section 4).  The mean of the rounding
error alone reaches a quarter ulp (2^-10 for bf16) when most values sit near
the maximum, as in a tensor of a few elements, so the mean bounds are twice
that: the forward's 2e-3 for bf16, and 5e-4 for f16.
With a single key (L = 1), P = 1 and dS = dO . v - dO . out with out = v, so
dq, dk and both bias gradients vanish identically; those are checked against
the fp32 error bound of that cancellation instead (single_key_bound).
delta = dO . out is computed from the out the backward is given, which
carries the forward pass's own error (bounded by the forward tolerances:
max |d out| <= 1e-4 / 2e-2 / 1e-2 for f32 / bf16 / f16); so it is compared
with dO . out_ref within that bound times sum_e |dO_e|.

Outputs are poisoned with NaN before every launch.
"""
import sys

import numpy as np
import pytest

import oracle
import synthetic as S

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max=1e-4, mean=1e-5, out=1e-4),
       "bf16": dict(max=1.6e-2, mean=2e-3, out=2e-2),
       "f16": dict(max=4e-3, mean=5e-4, out=1e-2)}
THREADS = min(16, oracle.default_threads())
NAMES = ("dq", "dk", "dv", "dmask", "dpair")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch


def to_dev(torch, x, dtype):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    elif dtype == "f16":
        t = t.view(torch.float16)
    return t.to("cuda")


def f64(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def fwd_supported(dtype, D):
    return D in (8, 16, 32, 64)


# largest normalised error seen per (dtype, gradient), printed when the module ends
WORST = {}


@pytest.fixture(scope="module", autouse=True)
def report_worst():
    yield
    for (dtype, name), (mx, mean, what) in sorted(WORST.items()):
        say(f"largest {dtype} {name}: max|d|/max|ref|={mx:.3e} (bound {TOL[dtype]['max']:.1e}, {what}); "
            f"largest mean {mean:.3e} (bound {TOL[dtype]['mean']:.1e})")


def run_bwd(torch, w, dout, want_dmask=True, want_dpair=True, fwd_from_oracle=False, stream=None, use_ws=True):
    """Forward (HIP, or the oracle where the HIP forward lacks the shape), then the HIP backward, with the
    recommended workspace (NaN-filled) unless use_ws is False.

    Returns (grads as float64 numpy [dq, dk, dv, dmask|None, dpair|None], delta, out).
    """
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = w.shape
    q, k, v = (to_dev(torch, x, w.dtype) for x in (w.q, w.k, w.v))
    mask, pair = to_dev(torch, w.mask, w.dtype), to_dev(torch, w.pair, w.dtype)
    do = to_dev(torch, dout, w.dtype)
    if fwd_from_oracle or not fwd_supported(w.dtype, D):
        ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=w.dtype, nthreads=THREADS)
        out = to_dev(torch, S.to_storage(ro.astype(np.float32), w.dtype), w.dtype)
        lse = torch.from_numpy(rl.astype(np.float32)).to("cuda")
    else:
        out, lse = E.fwd(q, k, v, mask, pair)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    dmask = torch.full_like(mask, float("nan")) if (mask is not None and want_dmask) else None
    dpair = torch.full_like(pair, float("nan")) if (pair is not None and want_dpair) else None
    delta = torch.full((B, N, H, L), float("nan"), dtype=torch.float32, device="cuda")
    code = E.torch_dtype_code(q.dtype)
    ws_bytes = E.evo_attn_bwd_workspace_size(w.shape, code) if use_ws else 0
    ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device="cuda") if ws_bytes else None
    say(f"  bwd {w.name} shape={w.shape} dtype={w.dtype} mask={mask is not None} pair={pair is not None} "
        f"dmask={dmask is not None} dpair={dpair is not None} workspace={ws_bytes}")
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = E.evo_attn_bwd(q, k, v, mask, pair, out, lse, do, dq, dk, dv, dmask, dpair, delta, w.shape, code, stream,
                        workspace=ws, workspace_bytes=ws_bytes)
    assert st == E.EVO_OK, E.evo_status_string(st)
    torch.cuda.synchronize()
    return [f64(x) for x in (dq, dk, dv, dmask, dpair)], f64(delta), f64(out)


def compare_grads(got, want, dtype, what):
    tol = TOL[dtype]
    for name, g, r in zip(NAMES, got, want):
        assert (g is None) == (r is None), f"{what} {name}: presence differs"
        if g is None:
            continue
        assert np.isfinite(g).all(), f"{what} {name}: non-finite values"
        scale = max(np.abs(r).max(), 1e-30)
        err = np.abs(g - r) / scale
        msg = f"{what} {name}: max|d|/max|ref|={err.max():.3e} mean={err.mean():.3e} (max|ref|={scale:.3e})"
        say("  " + msg)
        prev = WORST.get((dtype, name), (0.0, 0.0, ""))
        WORST[(dtype, name)] = (max(prev[0], err.max()), max(prev[1], err.mean()),
                                what if err.max() > prev[0] else prev[2])
        assert err.max() <= tol["max"], msg
        assert err.mean() <= tol["mean"], msg


def compare_delta(delta, w, dout, what):
    """delta = dO . out, checked against the oracle's out."""
    ro, _ = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=w.dtype, nthreads=THREADS)
    dof = S.storage_to_f32(dout, w.dtype).astype(np.float64)
    want = np.einsum("bnlhd,bnlhd->bnhl", dof, ro)
    bound = TOL[w.dtype]["out"] * np.abs(dof).sum(axis=-1).transpose(0, 1, 3, 2) + 1e-6
    assert (np.abs(delta - want) <= bound).all(), f"{what}: delta off by {np.abs(delta - want).max():.3e}"


def parity(torch, w, dout, want_dmask=True, want_dpair=True, **kw):
    """HIP backward vs the oracle's; returns the HIP gradients."""
    got, delta, _ = run_bwd(torch, w, dout, want_dmask, want_dpair, **kw)
    want = list(oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=w.dtype, want_dmask=want_dmask,
                           want_dpair=want_dpair, nthreads=THREADS))
    compare_grads(got, want, w.dtype, w.name)
    compare_delta(delta, w, dout, w.name)
    return got


# ---------------------------------------------------------------------------
# Ragged shapes: several 64-row tiles and a partial one, every dtype and head
# dimension, every bias combination.
# ---------------------------------------------------------------------------
SHAPES = [(1, 1, 1, 1), (1, 2, 5, 3), (2, 3, 17, 2), (1, 2, 64, 2), (1, 2, 77, 3), (2, 2, 130, 2)]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [8, 16, 32, 64])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_ragged(torch_dev, shape, d, dtype):
    B, N, L, H = shape
    w = S.random_problem(B, N, L, H, d, dtype=dtype, seed=B * 1000 + N * 100 + L + H + d, mask="tail",
                         pair="normal", mask_frac=0.3)
    dout = S.random_dout(w.shape, dtype, seed=L + d)
    if L == 1:
        single_key(torch_dev, w, dout)
    else:
        parity(torch_dev, w, dout)


# fp32 inputs with 16-byte aligned bias rows (L % 4 == 0 in the dense layout):
# every stage runs on the fp32 matrix-core kernels, D = 8 as D = 16 with
# zero-padded chunks (N is too small here for the pair gradient's workspace:
# one range of n per tile).
# Every bias combination, bias gradients on and off, against the full backward
# oracle.
# The dk/dv stage loads the next head's K and V rows during the current
# head's last query step (aligned bias rows), and every stage issues the next
# step's copies at the top of the step.  Heads with one query step (L <= 64:
# that step is both the head's first and its last) and with two, four heads,
# against the oracle.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L,D", [(8, 32), (64, 32), (64, 64), (128, 16), (128, 32)])
def test_bwd_next_head_rows_loaded_early(torch_dev, dtype, L, D):
    w = S.random_problem(1, 3, L, 4, D, dtype=dtype, seed=L * 10 + D, mask="tail", pair="normal", mask_frac=0.2)
    dout = S.random_dout(w.shape, dtype, seed=L + D)
    say(f"next-head rows {dtype} L={L} D={D}")
    parity(torch_dev, w, dout)


F32_MFMA_BWD = [(1, 2, 4, 2, 16), (1, 3, 20, 2, 32), (2, 2, 68, 3, 32), (1, 2, 132, 2, 16), (1, 1, 192, 4, 32),
                (1, 2, 36, 2, 64), (2, 2, 100, 3, 64), (1, 1, 132, 2, 64), (1, 2, 4, 2, 8), (2, 2, 132, 3, 8)]


@pytest.mark.parametrize("shape", F32_MFMA_BWD, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("bias", ["both", "mask", "pair", "none"])
def test_bwd_f32_matrix_core_path(torch_dev, shape, bias):
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=sum(shape) * 7 + len(bias),
                         mask="tail" if bias in ("both", "mask") else None,
                         pair="normal" if bias in ("both", "pair") else None, mask_frac=0.3)
    dout = S.random_dout(w.shape, "f32", seed=L + D + len(bias))
    parity(torch_dev, w, dout)
    if bias == "both":
        parity(torch_dev, w, dout, want_dmask=False, want_dpair=False)


F32_STAGED_BWD = [(1, 2, 5, 2, 16), (1, 3, 17, 2, 32), (2, 2, 65, 3, 32), (1, 2, 99, 2, 64), (1, 24, 130, 2, 32),
                  (1, 20, 77, 2, 8)]


@pytest.mark.parametrize("shape", F32_STAGED_BWD, ids=lambda s: "x".join(map(str, s)))
def test_bwd_f32_matrix_core_unaligned_bias_rows(torch_dev, shape):
    """L % 4 != 0: the dense bias rows start at every 4-byte alignment, so the fp32 matrix-core kernels read
    the pair rows with unaligned loads over their exact range, stage the mask row through registers and write
    the pair gradient element by element (through the workspace reduction for N = 24).  Large biases sit on
    the last element of every pair and mask row."""
    B, N, L, H, D = shape
    w = with_edge_biases(S.random_problem(B, N, L, H, D, dtype="f32", seed=sum(shape) * 11, mask="tail",
                                          pair="normal", mask_frac=0.3))
    dout = S.random_dout(w.shape, "f32", seed=L + 5 * D)
    parity(torch_dev, w, dout)
    if N >= 16:
        parity(torch_dev, w, dout, use_ws=False)


@pytest.mark.parametrize("D", [32, 8])
def test_bwd_f32_matrix_core_masked_rows(torch_dev, D):
    """fp32 backward with -inf masks on part of a row and on a whole row (no gradient passes through it),
    and a peaked softmax (bias scale 8), on the matrix-core path (D = 8 zero-padded to 16)."""
    B, N, L, H = 1, 4, 96, 2
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=321, mask="zero", pair="normal", bias_scale=8.0)
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., 10:50] = -np.inf
    mf[0, 1] = -np.inf
    mf[0, 2, ..., 60:] = -1e9
    w.mask = mf
    dout = S.random_dout(w.shape, "f32", seed=322)
    parity(torch_dev, w, dout)


def single_key(torch, w, dout):
    """L = 1: dv = dO (P = 1) is compared as usual.  dq, dk, dmask and dpair vanish identically (the oracle
    returns exact zeros); the kernel's dS is the fp32 difference of two evaluations of the same D-term dot
    product dO . v, so |dS| <= 2 gamma_D sum_d |dO_d v_d| with gamma_D = D u / (1 - D u), u = 2^-24.  Each
    gradient multiplies that by its fan-in: |k| / sqrt(D) per element for dq, |q| / sqrt(D) for dk, the H
    heads for dmask and the N sequences for dpair; rounding to the storage format cannot enlarge a bound
    that is representable."""
    got, delta, _ = run_bwd(torch, w, dout)
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=w.dtype, nthreads=THREADS)
    B, N, L, H, D = w.shape
    for name, r in zip(NAMES, want):
        if name != "dv":
            assert r is None or not r.any(), f"oracle {name} is not identically zero for one key"
    compare_grads([None, None, got[2], None, None], [None, None, want[2], None, None], w.dtype, w.name)
    f = lambda x: S.storage_to_f32(x, w.dtype).astype(np.float64)
    u = 2.0 ** -24
    gamma = D * u / (1 - D * u)
    ds = 2 * gamma * np.abs(f(dout) * f(w.v)).sum(axis=-1)        # [B,N,1,H] bound on |dS|
    bounds = {"dq": ds[..., None] * np.abs(f(w.k)) / np.sqrt(D),
              "dk": ds[..., None] * np.abs(f(w.q)) / np.sqrt(D),
              "dmask": ds.sum(axis=-1).reshape(B, N, 1, 1, 1),
              "dpair": ds.sum(axis=1).reshape(B, 1, H, 1, 1)}
    for name, g in zip(NAMES, got):
        if name in bounds and g is not None:
            excess = np.abs(g) - bounds[name]
            say(f"  {w.name} {name}: max|g|={np.abs(g).max():.3e} within the cancellation bound: {(excess <= 0).all()}")
            assert (excess <= 0).all(), f"{w.name} {name}: exceeds the cancellation bound by {excess.max():.3e}"
    compare_delta(delta, w, dout, w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bias", ["mask", "pair", "none"])
def test_bwd_bias_subsets(torch_dev, dtype, bias):
    w = S.random_problem(1, 3, 90, 2, 32, dtype=dtype, seed=len(bias) * 13, mask="tail" if bias == "mask" else None,
                         pair="normal" if bias == "pair" else None, mask_frac=0.3)
    dout = S.random_dout(w.shape, dtype, seed=5)
    parity(torch_dev, w, dout)


def test_bwd_bias_gradients_on_request(torch_dev):
    """Without dmask/dpair the other gradients are unchanged (and the pair kernel does not run)."""
    w = S.random_problem(1, 2, 70, 2, 32, dtype="bf16", seed=21, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=22)
    full = parity(torch_dev, w, dout)
    part = parity(torch_dev, w, dout, want_dmask=False, want_dpair=False)
    assert part[3] is None and part[4] is None
    for a, b in zip(full[:3], part[:3]):
        np.testing.assert_array_equal(a, b)


def test_bwd_deterministic(torch_dev):
    """Sums are formed in a fixed order: two calls agree bit for bit."""
    w = S.random_problem(1, 5, 100, 2, 32, dtype="bf16", seed=23, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=24)
    a, da, _ = run_bwd(torch_dev, w, dout)
    b, db, _ = run_bwd(torch_dev, w, dout)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(da, db)


def test_bwd_large_biases_random_masks(torch_dev):
    w = S.random_problem(1, 4, 150, 2, 32, dtype="bf16", seed=25, mask="random", pair="normal", mask_frac=0.5,
                         bias_scale=8.0)
    parity(torch_dev, w, S.random_dout(w.shape, "bf16", seed=26))


@pytest.mark.parametrize("L", [40, 96])
def test_bwd_f16_fully_masked_sequence(torch_dev, L):
    """f16 turns -1e9 into -inf: a sequence with every key removed gets and passes on no gradient."""
    B, N, H, D = 1, 3, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="f16", seed=27 + L, mask="zero", pair="normal")
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., 10:30] = -1e9
    mf[0, 1] = -1e9
    w.mask = S.to_storage(mf, "f16")
    dout = S.random_dout(w.shape, "f16", seed=28)
    got = parity(torch_dev, w, dout)
    for g in got[:4]:
        assert np.all(g[0, 1] == 0)


def test_bwd_oracle_forward_inputs(torch_dev):
    """The backward accepts out/lse from any forward: oracle values give the same gradients to the bound."""
    w = S.random_problem(1, 2, 80, 2, 32, dtype="bf16", seed=29, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=30)
    parity(torch_dev, w, dout, fwd_from_oracle=True)


def test_bwd_non_default_stream(torch_dev):
    torch = torch_dev
    w = S.random_problem(1, 2, 96, 2, 32, dtype="bf16", seed=31, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got, _, _ = run_bwd(torch, w, dout, stream=s.cuda_stream)
    want = list(oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="bf16", nthreads=THREADS))
    compare_grads(got, want, "bf16", "side stream")


def test_bwd_errors_write_nothing(torch_dev):
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    shp = (1, 1, 32, 1, 24)
    q = torch.zeros(shp, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 1, 32), dtype=torch.float32, device="cuda")
    outs = [torch.full_like(q, 7.0) for _ in range(3)]
    delta = torch.full_like(lse, 7.0)
    st = E.evo_attn_bwd(q, q, q, None, None, q, lse, q, *outs, None, None, delta, shp, E.EVO_DTYPE_BF16, None)
    assert st == E.EVO_ERR_UNSUPPORTED
    st = E.evo_attn_bwd(q, q, q, None, q, q, lse, q, *outs, None, outs[0], delta, (1, 1, 32, 1, 32),
                        E.EVO_DTYPE_BF16, None)
    assert st != E.EVO_OK
    torch.cuda.synchronize()
    assert all(bool((o == 7.0).all()) for o in outs) and bool((delta == 7.0).all())


# ---------------------------------------------------------------------------
# Named workloads at full size (the oracle's full backward finishes in seconds
# for these): the guide's unit-test shape and the triangle-attention problem.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("c", [1, 2, 4])
def test_bwd_workload_full(torch_dev, c):
    w = S.workload(c)
    say(f"workload {c} backward: full oracle comparison")
    parity(torch_dev, w, S.random_dout(w.shape, w.dtype, seed=100 + c))


@pytest.mark.parametrize("L", [4096, 4093])
def test_bwd_long_rows(torch_dev, L):
    """Rows of 64 blocks of keys: L = 4096 (aligned bias rows) and L = 4093 (bias rows staged through
    registers, a partial group of 4 keys at every row's end), four sequences sharing one pair matrix."""
    w = S.random_problem(1, 4, L, 1, 32, dtype="bf16", seed=4000 + L, mask="tail", pair="normal", mask_frac=0.1)
    say(f"long rows backward: L = {L}")
    parity(torch_dev, w, S.random_dout(w.shape, "bf16", seed=L))


def test_bwd_ds4sci_unit_test_shape(torch_dev):
    """The guide's unit test checks every gradient on (1,256,256,4,32) with both biases (section 4)."""
    w = S.random_problem(1, 256, 256, 4, 32, dtype="f16", seed=4053, mask="tail", pair="normal", mask_frac=0.1)
    parity(torch_dev, w, S.random_dout(w.shape, "f16", seed=4054))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L", [200, 72])
def test_bwd_rows_past_L_read_as_zero(torch_dev, dtype, L):
    """Rows past L are never read from memory: with NaN right after every input and L not a multiple of
    the 64-row block, every gradient stays finite and matches the oracle."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, H, D = 1, 2, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=43 + L, mask="tail", pair="normal", mask_frac=0.2)
    dout = S.random_dout(w.shape, dtype, seed=44)
    extra = 128 * H * D + 128 * L

    def dev(x):
        t = to_dev(torch, x, dtype)
        buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device="cuda")
        buf[: t.numel()] = t.reshape(-1)
        return buf[: t.numel()].view(t.shape)

    q, k, v, m, p, do = (dev(x) for x in (w.q, w.k, w.v, w.mask, w.pair, dout))
    out, lse = E.fwd(q, k, v, m, p)
    o2 = torch.full((out.numel() + extra,), float("nan"), dtype=out.dtype, device="cuda")
    o2[: out.numel()] = out.reshape(-1)
    out = o2[: out.numel()].view(out.shape)
    grads = E.bwd(q, k, v, m, p, out, lse, do)[:5]
    torch.cuda.synchronize()
    got = [f64(g) for g in grads]
    want = list(oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS))
    compare_grads(got, want, dtype, f"NaN after every input, L={L}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("L", [64, 72, 136, 200])
def test_bwd_pair_gradient_split_over_n(torch_dev, dtype, L):
    """N large enough for the workspace path (the N axis of the pair gradient split over workgroups and the
    partial sums added in order), L with partial 64-row tiles; the same gradients without a workspace.
    fp32 at these shapes (D = 32, L % 4 == 0) runs every stage on the fp32 matrix-core kernels."""
    import evoformer_biased_attention_amd as E
    w = S.random_problem(1, 24, L, 3, 32, dtype=dtype, seed=L + 7, mask="tail", pair="normal", mask_frac=0.2)
    code = {"bf16": E.EVO_DTYPE_BF16, "f16": E.EVO_DTYPE_F16, "f32": E.EVO_DTYPE_F32}[dtype]
    assert E.evo_attn_bwd_workspace_size(w.shape, code) > 0
    dout = S.random_dout(w.shape, dtype, seed=L + 8)
    split = parity(torch_dev, w, dout)
    single = parity(torch_dev, w, dout, use_ws=False)
    for a, b in zip(split[:4], single[:4]):
        np.testing.assert_array_equal(a, b)   # only the pair gradient takes another route


@pytest.mark.parametrize("d", [8, 16, 64])
def test_bwd_f32_split_over_n_head_dims(torch_dev, d):
    """fp32, D = 8, 16 and 64, with the workspace (pair gradient split over N) and without: only dpair takes
    another route, and it stays within the fp32 bound either way."""
    import evoformer_biased_attention_amd as E
    w = S.random_problem(1, 32, 136, 3, d, dtype="f32", seed=1600 + d, mask="tail", pair="normal", mask_frac=0.2)
    assert E.evo_attn_bwd_workspace_size(w.shape, E.EVO_DTYPE_F32) > 0
    dout = S.random_dout(w.shape, "f32", seed=1601 + d)
    split = parity(torch_dev, w, dout)
    single = parity(torch_dev, w, dout, use_ws=False)
    for a, b in zip(split[:4], single[:4]):
        np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# L % 8 != 0 on the matrix cores: the bias tiles are staged through registers,
# the pair gradient's workspace rows are padded to a multiple of 4 keys, and
# the last partial group of 4 keys of every bias and bias-gradient row is read
# and written element by element.  Large biases sit on the last element of
# every pair matrix and mask row (and on the first key of the last pair row).
# ---------------------------------------------------------------------------
def with_edge_biases(w):
    pf = S.storage_to_f32(w.pair, w.dtype).copy()
    pf[..., -1, -1] = 4.0
    pf[..., -1, 0] = -3.0
    mf = S.storage_to_f32(w.mask, w.dtype).copy()
    mf[..., -1] = 2.0
    w.pair, w.mask = S.to_storage(pf, w.dtype), S.to_storage(mf, w.dtype)
    return w


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L", [9, 63, 99, 130])
def test_bwd_odd_L_split_over_n(torch_dev, dtype, L):
    """With and without the workspace; only the pair gradient takes another route."""
    w = with_edge_biases(S.random_problem(1, 24, L, 3, 32, dtype=dtype, seed=L + 70, mask="tail", pair="normal",
                                          mask_frac=0.2))
    dout = S.random_dout(w.shape, dtype, seed=L + 71)
    split = parity(torch_dev, w, dout)
    single = parity(torch_dev, w, dout, use_ws=False)
    for a, b in zip(split[:4], single[:4]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [8, 16, 64])
def test_bwd_odd_L_other_head_dims(torch_dev, d, dtype):
    w = with_edge_biases(S.random_problem(1, 16, 77, 2, d, dtype=dtype, seed=d + 90, mask="tail", pair="normal"))
    parity(torch_dev, w, S.random_dout(w.shape, dtype, seed=d + 91))


def test_bwd_workspace_deterministic(torch_dev):
    w = S.random_problem(1, 40, 96, 2, 32, dtype="bf16", seed=61, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=62)
    a, _, _ = run_bwd(torch_dev, w, dout)
    b, _, _ = run_bwd(torch_dev, w, dout)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("c", [2, 4])
def test_bwd_workload_without_workspace(torch_dev, c):
    w = S.workload(c)
    parity(torch_dev, w, S.random_dout(w.shape, w.dtype, seed=100 + c), use_ws=False)


# ---------------------------------------------------------------------------
# Head dimension 64 on the matrix cores (L % 8 == 0): dq and the pair gradient
# in two 32-wide halves, dk/dv with 16-key tiles and 32-query steps.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 2, 64, 2), (1, 3, 136, 2), (2, 2, 200, 3), (1, 2, 40, 4)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bwd_head_dim_64_matrix_cores(torch_dev, shape, dtype):
    B, N, L, H = shape
    w = S.random_problem(B, N, L, H, 64, dtype=dtype, seed=6400 + B * 100 + N * 10 + L + H, mask="tail",
                         pair="normal", mask_frac=0.3)
    parity(torch_dev, w, S.random_dout(w.shape, dtype, seed=L + 64))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_head_dim_64_split_over_n(torch_dev, dtype):
    """D = 64 with the workspace (pair gradient split over N) and without: only dpair takes another route."""
    import evoformer_biased_attention_amd as E
    w = S.random_problem(1, 24, 136, 2, 64, dtype=dtype, seed=6464, mask="tail", pair="normal", mask_frac=0.2)
    assert E.evo_attn_bwd_workspace_size(w.shape, E.EVO_DTYPE_BF16 if dtype == "bf16" else E.EVO_DTYPE_F16) > 0
    dout = S.random_dout(w.shape, dtype, seed=6465)
    split = parity(torch_dev, w, dout)
    single = parity(torch_dev, w, dout, use_ws=False)
    for a, b in zip(split[:4], single[:4]):
        np.testing.assert_array_equal(a, b)


def test_bwd_head_dim_64_larger(torch_dev):
    """D = 64 at N = 128, L = 256, H = 4 (bf16, mask and pair bias): four 64-key dk/dv workgroups per
    sequence, eight 32-query steps per head."""
    w = S.random_problem(1, 128, 256, 4, 64, dtype="bf16", seed=6466, mask="tail", pair="normal", mask_frac=0.1)
    parity(torch_dev, w, S.random_dout(w.shape, "bf16", seed=6467))


@pytest.mark.parametrize("L", [200, 72])
def test_bwd_head_dim_64_rows_past_L_read_as_zero(torch_dev, L):
    """As test_bwd_rows_past_L_read_as_zero, at D = 64: NaN right after every input."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, H, D, dtype = 1, 2, 2, 64, "bf16"
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=6468 + L, mask="tail", pair="normal", mask_frac=0.2)
    dout = S.random_dout(w.shape, dtype, seed=6469)
    extra = 128 * H * D + 128 * L

    def dev(x):
        t = to_dev(torch, x, dtype)
        buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device="cuda")
        buf[: t.numel()] = t.reshape(-1)
        return buf[: t.numel()].view(t.shape)

    q, k, v, m, p, do = (dev(x) for x in (w.q, w.k, w.v, w.mask, w.pair, dout))
    out, lse = E.fwd(q, k, v, m, p)
    o2 = torch.full((out.numel() + extra,), float("nan"), dtype=out.dtype, device="cuda")
    o2[: out.numel()] = out.reshape(-1)
    out = o2[: out.numel()].view(out.shape)
    grads = E.bwd(q, k, v, m, p, out, lse, do)[:5]
    torch.cuda.synchronize()
    got = [f64(g) for g in grads]
    want = list(oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS))
    compare_grads(got, want, dtype, f"D = 64, NaN after every input, L={L}")
