"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerances (floating point):
  f32 path:  max |dO| <= 1e-4, max |dLSE| <= 1e-4
  bf16 path: max |dO| <= 2e-2, mean |dO| <= 2e-3, max |dLSE| <= 1e-2
  f16 path:  max |dO| <= 1e-2, mean |dO| <= 1e-3, max |dLSE| <= 5e-3
The bf16 budget is dominated by rounding O to bf16 (half an ulp is 2^-9
relative) and by rounding the probabilities to bf16 before the P.V product;
scores themselves are exact products of bf16 values accumulated in fp32.
binary16 carries 3 more mantissa bits than bf16, so the same two roundings
are 8 times smaller (half an ulp is 2^-12 relative); its bounds are set at
half those of bf16, which leaves the same headroom for the fp32 accumulation
and the output range (|O| < 8).

Outputs are poisoned with NaN before every launch, so an element the kernel
fails to write shows up as a mismatch.
"""
import math
import os
import sys

import numpy as np
import pytest

import oracle
import synthetic as S

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_o=1e-4, mean_o=1e-4, max_lse=1e-4),
       "bf16": dict(max_o=2e-2, mean_o=2e-3, max_lse=1e-2),
       "f16": dict(max_o=1e-2, mean_o=1e-3, max_lse=5e-3)}
THREADS = min(16, oracle.default_threads())


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


def run_gpu(torch, w, lse=True, stream=None):
    """Launch the HIP path on workload w; returns (out float64 numpy, lse float64 numpy or None)."""
    import evoformer_biased_attention_amd as E
    q, k, v = (to_dev(torch, x, w.dtype) for x in (w.q, w.k, w.v))
    mask, pair = to_dev(torch, w.mask, w.dtype), to_dev(torch, w.pair, w.dtype)
    out = torch.full_like(q, float("nan"))
    B, N, L, H, D = w.shape
    lse_t = torch.full((B, N, H, L), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    say(f"  launch {w.name} shape={w.shape} dtype={w.dtype} mask={w.mask is not None} pair={w.pair is not None}")
    E.fwd(q, k, v, mask, pair, out=out, lse=lse_t if lse else False, stream=stream)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse_t.cpu().numpy().astype(np.float64) if lse else None
    return o, l


def compare(o, l, ro, rl, dtype, what=""):
    tol = TOL[dtype]
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    do = np.abs(o - ro)
    msg = f"{what}: max|dO|={do.max():.3e} mean|dO|={do.mean():.3e}"
    if l is not None:
        neg = np.isneginf(rl)
        assert np.array_equal(np.isneginf(l), neg), f"{what}: -inf LSE rows differ"
        dl = np.abs(l[~neg] - rl[~neg]) if (~neg).any() else np.zeros(1)
        msg += f" max|dLSE|={dl.max():.3e}"
        assert dl.max() <= tol["max_lse"], msg
    say("  " + msg)
    assert do.max() <= tol["max_o"], msg
    assert do.mean() <= tol["mean_o"], msg


def parity_full(torch, w, lse=True):
    o, l = run_gpu(torch, w, lse=lse)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=w.dtype, nthreads=THREADS)
    compare(o, l, ro, rl if lse else None, w.dtype, w.name)
    return o, l


def parity_sampled(torch, w, count=4096, seed=7):
    o, l = run_gpu(torch, w)
    idx = S.sample_rows(w.shape, count, seed=seed)
    ro, rl = oracle.rows(w.q, w.k, w.v, w.mask, w.pair, dtype=w.dtype, idx=idx, nthreads=THREADS)
    b, n, h, i = idx.T
    compare(o[b, n, i, h, :], l[b, n, h, i], ro, rl, w.dtype, f"{w.name} ({len(idx)} sampled rows)")
    # properties over every row: finite, and each output is a convex combination of value rows
    vf = S.storage_to_f32(w.v, w.dtype)
    assert np.isfinite(l).all()
    vmax = np.abs(vf).max(axis=2, keepdims=True)  # [B,N,1,H,D]
    assert (np.abs(o) <= vmax * (1 + 2 ** -7) + 1e-6).all()
    return o, l


# ---------------------------------------------------------------------------
# The five named workloads at full size, in the launch configuration that the
# benchmark times.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("c", [1, 2, 3, 4, 5])
def test_workload_full_oracle(torch_dev, c):
    """Every element of out and lse of each named workload against the full oracle: MSA row attention
    (1, 2), MSA column attention (3), triangle attention around the starting (4) and ending (5) node."""
    say(f"workload {c}: full oracle comparison")
    parity_full(torch_dev, S.workload(c))


@pytest.mark.parametrize("L", [32760, 32767])
def test_longest_pair_rows(torch_dev, L):
    """The longest sequences whose pair matrix keeps every byte offset of the 16-bit kernel in 32 bits
    ((L - 1) * 2L + 2L < 2^31; L = 32768 is rejected): L = 32760 has 16-byte aligned rows (direct copies),
    L = 32767 does not (rows staged through registers).  One 2 GiB pair matrix, 512 blocks of keys per row."""
    say(f"longest pair rows: L = {L}")
    w = S.random_problem(1, 1, L, 1, 32, dtype="bf16", seed=L, mask="tail", pair="int8")
    parity_sampled(torch_dev, w, count=256)


# ---------------------------------------------------------------------------
# Ragged and edge shapes (bf16 MFMA path).
# ---------------------------------------------------------------------------
RAGGED = [
    (1, 1, 1, 1, 32), (1, 2, 5, 3, 32), (2, 3, 17, 2, 32), (1, 2, 64, 1, 32), (1, 3, 100, 2, 32),
    (2, 2, 129, 3, 32), (1, 2, 200, 4, 32), (1, 1, 255, 1, 32), (1, 2, 257, 2, 32), (3, 2, 33, 5, 32),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("bias", ["both", "mask", "pair", "none"])
def test_ragged_bf16(torch_dev, shape, bias):
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=sum(shape) * 7 + len(bias),
                         mask="tail" if bias in ("both", "mask") else None,
                         pair="normal" if bias in ("both", "pair") else None, mask_frac=0.3)
    say(f"ragged bf16 {shape} bias={bias}")
    parity_full(torch_dev, w)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 8), (1, 2, 17, 3, 16), (2, 2, 65, 2, 32), (1, 2, 100, 2, 64),
                                   (1, 3, 130, 1, 32)], ids=lambda s: "x".join(map(str, s)))
def test_ragged_f32(torch_dev, shape):
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=sum(shape), mask="tail", pair="normal", mask_frac=0.3)
    say(f"ragged f32 {shape}")
    parity_full(torch_dev, w)


# fp32 inputs take the matrix-core fp32 kernel (bias rows that are not 16-byte
# aligned, L % 4 != 0 in the dense layout, through its staged variant); D = 8
# runs as D = 16 with zero-padded chunks.  All against the full oracle.
F32_MFMA_SHAPES = [(1, 2, 4, 2, 16), (1, 3, 20, 2, 32), (2, 2, 68, 3, 32), (1, 2, 132, 2, 64), (1, 1, 256, 4, 16),
                   (1, 2, 100, 2, 32), (2, 3, 64, 2, 64), (1, 1, 192, 1, 32), (1, 2, 4, 2, 8), (2, 2, 132, 3, 8)]


@pytest.mark.parametrize("shape", F32_MFMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("bias", ["both", "mask", "pair", "none"])
def test_f32_matrix_core_path(torch_dev, shape, bias):
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=sum(shape) + len(bias), mask="tail" if bias in ("both", "mask") else None,
                         pair="normal" if bias in ("both", "pair") else None, mask_frac=0.3)
    say(f"f32 matrix-core path {shape} bias={bias}")
    parity_full(torch_dev, w)


F32_STAGED_SHAPES = [(1, 2, 5, 2, 16), (1, 3, 17, 2, 32), (2, 2, 65, 3, 32), (1, 2, 99, 2, 64), (1, 1, 130, 4, 16),
                     (1, 2, 383, 2, 32), (1, 3, 77, 2, 8)]


@pytest.mark.parametrize("shape", F32_STAGED_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("bias", ["both", "mask", "pair"])
def test_f32_matrix_core_unaligned_bias_rows(torch_dev, shape, bias):
    """L % 4 != 0: the dense bias rows start at every 4-byte alignment, so the fp32 matrix-core kernel
    reads the pair rows with unaligned 16-byte loads over their exact range and stages the mask row through
    registers.  Large biases sit on the last element of every pair and mask row."""
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=sum(shape) * 3 + len(bias),
                         mask="tail" if bias in ("both", "mask") else None,
                         pair="normal" if bias in ("both", "pair") else None, mask_frac=0.3)
    if w.pair is not None:
        w.pair = w.pair.copy()
        w.pair[..., -1] = 3.0
    if w.mask is not None:
        w.mask = w.mask.copy()
        w.mask[..., -1] = 2.0
    say(f"f32 matrix-core path, unaligned bias rows {shape} bias={bias}")
    parity_full(torch_dev, w)


@pytest.mark.parametrize("D", [32, 8])
@pytest.mark.parametrize("L", [64, 96, 66, 97])
def test_f32_infinite_and_nan_masks(torch_dev, L, D):
    """fp32 masks with -inf on part of a row, on a whole row (out = 0, lse = -inf), a finite -1e9 on a
    leading half, and a NaN (its sequence NaN).  D = 8 runs zero-padded to 16."""
    B, N, H = 1, 5, 2
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=L + 5, mask="zero", pair="normal")
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., 10:50] = -np.inf
    mf[0, 1] = -np.inf
    mf[0, 2, ..., : L // 2] = -1e9
    mf[0, 3, ..., 7] = np.nan
    w.mask = mf
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="f32", nthreads=THREADS)
    assert np.all(o[0, 1] == 0) and np.all(np.isneginf(l[0, 1]))
    assert np.isnan(o[0, 3]).all() and np.isnan(l[0, 3]).all()
    keep = np.array([True, True, True, False, True])
    compare(o[:, keep], l[:, keep], ro[:, keep], rl[:, keep], "f32", f"fp32 infinite masks, L={L}, D={D}")


def test_large_bias_magnitudes(torch_dev):
    """Biases of scale 8 (peaked softmax) and random -1e9 masks."""
    w = S.random_problem(1, 4, 192, 2, 32, dtype="bf16", seed=77, mask="random", pair="normal", mask_frac=0.5,
                         bias_scale=8.0)
    parity_full(torch_dev, w)


def test_ds4sci_unit_test_shape(torch_dev):
    """The guide's unit-test shape (1,256,256,4,32) with a mask and a random pair bias (section 4)."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "ds4sci_guide_facts.json")) as f:
        facts = json.load(f)
    shape = tuple(facts["unit_test"]["shapes_B_N_L_H_D"][0])
    w = S.random_problem(*shape, dtype="bf16", seed=4050, mask="tail", pair="normal", mask_frac=0.1)
    o, l = parity_full(torch_dev, w)


def test_without_lse(torch_dev):
    w = S.random_problem(1, 2, 70, 2, 32, dtype="bf16", seed=3, mask="tail", pair="normal")
    parity_full(torch_dev, w, lse=False)


def test_neg_inf_mask_rows(torch_dev):
    """-inf masks in bf16: partially masked rows are exact softmaxes over the rest; a row whose every key
    is -inf returns out = 0 and lse = -inf."""
    B, N, L, H, D = 1, 3, 80, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=8, mask="zero", pair="normal")
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., 10:50] = -np.inf
    mf[0, 1] = -np.inf
    w.mask = S.to_storage(mf, "bf16")
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    assert np.all(o[0, 1] == 0) and np.all(np.isneginf(l[0, 1]))
    compare(o, l, ro, rl, "bf16", "neg-inf mask")


@pytest.mark.parametrize("c", [2, 4])
def test_bf16_neg_inf_tail_masks_on_workloads(torch_dev, c):
    """The row and triangle workloads with their -1e9 mask entries replaced by -inf (bf16 keeps -inf on the
    fast path by clamping it), element by element against the full oracle."""
    w = S.workload(c)
    mf = S.storage_to_f32(w.mask, "bf16").copy()
    mf[mf <= -1e8] = -np.inf
    w.mask = S.to_storage(mf, "bf16")
    say(f"workload {c} with -inf masks")
    parity_full(torch_dev, w)


@pytest.mark.parametrize("L", [80, 77])
def test_bf16_nan_mask_values(torch_dev, L):
    """A NaN in a bf16 mask, with the sign bit set (which the -inf clamp must not turn into -inf) or clear,
    makes every row of its sequence NaN, as in the definition; the other sequences keep full parity."""
    B, N, H, D = 1, 4, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=L + 11, mask="zero", pair="normal")
    m = w.mask.copy()
    m[0, 0, 0, 0, 9] = 0xFFC1      # negative NaN
    m[0, 1, 0, 0, L - 1] = 0x7FC0  # positive NaN
    m[0, 2, 0, 0, 3:30] = 0xFF80   # -inf on part of the row
    w.mask = m
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    nan_seq = np.zeros(N, bool)
    nan_seq[:2] = True
    assert np.isnan(ro[:, nan_seq]).all() and np.isnan(rl[:, nan_seq]).all()
    assert np.isnan(o[:, nan_seq]).all(), "a NaN mask value must make its sequence's outputs NaN"
    assert np.isnan(l[:, nan_seq]).all(), "a NaN mask value must make its sequence's lse NaN"
    compare(o[:, ~nan_seq], l[:, ~nan_seq], ro[:, ~nan_seq], rl[:, ~nan_seq], "bf16", f"other sequences, L={L}")


@pytest.mark.parametrize("L", [200, 203])
def test_bf16_negative_nan_mask_later_blocks(torch_dev, L):
    """A negative NaN in a bf16 mask in a middle 64-key block (its chunk lies wholly below L, tested with one
    packed maximum) and in the last key (the last block, where chunks end past L and the test goes element by
    element): both sequences come out NaN; a sequence with a -inf run and a clean one keep full parity."""
    B, N, H, D = 1, 4, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=L + 29, mask="zero", pair="normal")
    m = w.mask.copy()
    m[0, 0, 0, 0, 130] = 0xFFC1      # negative NaN, third block
    m[0, 1, 0, 0, L - 1] = 0xFFFF    # negative NaN, last key
    m[0, 2, 0, 0, 64:128] = 0xFF80   # -inf over a whole block
    w.mask = m
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    nan_seq = np.zeros(N, bool)
    nan_seq[:2] = True
    assert np.isnan(ro[:, nan_seq]).all() and np.isnan(rl[:, nan_seq]).all()
    assert np.isnan(o[:, nan_seq]).all(), "a NaN mask value must make its sequence's outputs NaN"
    assert np.isnan(l[:, nan_seq]).all(), "a NaN mask value must make its sequence's lse NaN"
    compare(o[:, ~nan_seq], l[:, ~nan_seq], ro[:, ~nan_seq], rl[:, ~nan_seq], "bf16", f"other sequences, L={L}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L", [77, 96])
def test_neg_inf_pair_bias_exact_path(torch_dev, L, dtype):
    """-inf in the pair bias (one key, part of a row, a whole row, the last element): the identity product
    turns it into NaN and those workgroups redo their slice on the exact path, for staged (L = 77) and
    direct (L = 96) bias copies."""
    w = S.random_problem(1, 2, L, 2, 32, dtype=dtype, seed=900 + L, mask="tail", pair="normal")
    pf = S.storage_to_f32(w.pair, dtype).copy()
    pf[0, 0, 1, 5, 7] = -np.inf
    pf[0, 0, 0, 70, :40] = -np.inf
    pf[0, 0, 1, 20, :] = -np.inf
    pf[0, 0, 0, L - 1, L - 1] = -np.inf
    w.pair = S.to_storage(pf, dtype)
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, f"infinite pair bias, L={L}")


# ---------------------------------------------------------------------------
# L % 8 != 0: bias rows are not 16-byte aligned, and the kernel stages the
# bias tiles through registers with unaligned loads; a chunk that crosses the
# end of its buffer is read element by element.  Large biases on the last
# element of every pair matrix and mask row (and on the first key of the
# last pair row) make a dropped or shifted value show.
# ---------------------------------------------------------------------------
def with_edge_biases(w):
    pf = S.storage_to_f32(w.pair, w.dtype).copy()
    pf[..., -1, -1] = 6.0
    pf[..., -1, 0] = -4.0
    mf = S.storage_to_f32(w.mask, w.dtype).copy()
    mf[..., -1] = 3.0
    w.pair, w.mask = S.to_storage(pf, w.dtype), S.to_storage(mf, w.dtype)
    return w


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L", [3, 9, 31, 63, 66, 99, 130, 250])
def test_odd_L_edge_biases(torch_dev, L, dtype):
    w = with_edge_biases(S.random_problem(1, 2, L, 3, 32, dtype=dtype, seed=600 + L, mask="tail", pair="normal"))
    parity_full(torch_dev, w)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [8, 16, 64])
def test_odd_L_edge_biases_other_head_dims(torch_dev, d, dtype):
    w = with_edge_biases(S.random_problem(2, 2, 75, 2, d, dtype=dtype, seed=700 + d, mask="tail", pair="normal"))
    parity_full(torch_dev, w)


# ---------------------------------------------------------------------------
# binary16 (the same MFMA kernel on f16 operands).  A -1e9 mask is -inf in
# this format.
# ---------------------------------------------------------------------------
RAGGED_F16 = [(1, 1, 1, 1, 32), (2, 3, 17, 2, 32), (1, 2, 64, 1, 32), (2, 2, 129, 3, 32), (1, 2, 200, 4, 32),
              (1, 2, 257, 2, 32)]


@pytest.mark.parametrize("shape", RAGGED_F16, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("bias", ["both", "mask", "none"])
def test_ragged_f16(torch_dev, shape, bias):
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype="f16", seed=sum(shape) * 11 + len(bias),
                         mask="tail" if bias in ("both", "mask") else None,
                         pair="normal" if bias == "both" else None, mask_frac=0.3)
    say(f"ragged f16 {shape} bias={bias}")
    parity_full(torch_dev, w)


def test_f16_msa_row_shape(torch_dev):
    """An MSA-row-like problem in f16: per-sequence tail masks (-inf) and a pair bias."""
    w = S.random_problem(1, 32, 256, 8, 32, dtype="f16", seed=2024, mask="tail", pair="normal", mask_frac=0.1)
    parity_full(torch_dev, w)


def test_f16_ds4sci_unit_test_shapes(torch_dev):
    """The guide's unit-test shape with D = 32, in fp16, its primary dtype (section 4)."""
    w = S.random_problem(1, 256, 256, 4, 32, dtype="f16", seed=4051, mask="tail", pair="normal", mask_frac=0.1)
    parity_full(torch_dev, w)


def test_f16_large_biases_and_random_masks(torch_dev):
    w = S.random_problem(1, 4, 192, 2, 32, dtype="f16", seed=78, mask="random", pair="normal", mask_frac=0.5,
                         bias_scale=8.0)
    parity_full(torch_dev, w)


@pytest.mark.parametrize("L", [96, 99, 128])
def test_f16_fully_masked_sequences(torch_dev, L):
    """A sequence whose keys are all -inf returns out = 0 and lse = -inf; L = 96 ends in a partial key block,
    L = 99 in a partial 8-key chunk (the keys past L must not count as unmasked)."""
    B, N, H, D = 1, 3, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="f16", seed=9 + L, mask="zero", pair="normal")
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., 10:50] = -1e9
    mf[0, 1] = -1e9
    w.mask = S.to_storage(mf, "f16")
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="f16", nthreads=THREADS)
    assert np.all(o[0, 1] == 0) and np.all(np.isneginf(l[0, 1]))
    compare(o, l, ro, rl, "f16", f"f16 fully masked L={L}")


# ---------------------------------------------------------------------------
# Head dimensions 8 and 16 on the 16-bit path (zero-padded to the 32-wide
# contraction inside the kernel).
# ---------------------------------------------------------------------------
SMALL_D = [(1, 2, 17, 3), (2, 2, 64, 2), (1, 3, 100, 4), (1, 2, 257, 2), (1, 1, 1, 1)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [8, 16])
@pytest.mark.parametrize("shape", SMALL_D, ids=lambda s: "x".join(map(str, s)))
def test_small_head_dims(torch_dev, shape, d, dtype):
    B, N, L, H = shape
    w = S.random_problem(B, N, L, H, d, dtype=dtype, seed=B * 1000 + N * 100 + L + H + d, mask="tail",
                         pair="normal", mask_frac=0.3)
    say(f"small head dim {dtype} {shape} D={d}")
    parity_full(torch_dev, w)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_ds4sci_unit_test_shape_d8(torch_dev, dtype):
    """The guide's second unit-test shape (1,512,256,8,8) (section 4)."""
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "ds4sci_guide_facts.json")) as f:
        facts = json.load(f)
    shape = tuple(facts["unit_test"]["shapes_B_N_L_H_D"][1])
    assert shape == (1, 512, 256, 8, 8)
    w = S.random_problem(*shape, dtype=dtype, seed=4052, mask="tail", pair="normal", mask_frac=0.1)
    parity_full(torch_dev, w)


def test_non_default_stream(torch_dev):
    torch = torch_dev
    w = S.random_problem(1, 2, 96, 2, 32, dtype="bf16", seed=12, mask="tail", pair="normal")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = run_gpu(torch, w, stream=s.cuda_stream)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    compare(o, l, ro, rl, "bf16", "side stream")


def test_errors_write_nothing(torch_dev):
    """Rejected calls return a status and leave the outputs untouched."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    q = torch.zeros((1, 1, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    st = E.evo_attn_fwd(q, q, q, None, None, out, None, (1, 1, 32, 1, 128), E.EVO_DTYPE_BF16,
                        torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_ERR_UNSUPPORTED
    st = E.evo_attn_fwd(q, q, q, None, None, q, None, (1, 1, 32, 1, 128), E.EVO_DTYPE_BF16, None)
    assert st == E.EVO_ERR_ALIASING
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    with pytest.raises(E.EvoAttnError):
        E.fwd(q, q, q)


def nan_tailed(torch, x, dtype, extra):
    """x on the device at the very end of its allocation's useful part: `extra` NaN elements follow it."""
    t = to_dev(torch, x, dtype)
    buf = torch.full((t.numel() + extra,), float("nan"), dtype=t.dtype, device="cuda")
    buf[: t.numel()] = t.reshape(-1)
    return buf[: t.numel()].view(t.shape)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rows_past_L_read_as_zero(torch_dev, dtype):
    """Operand rows past L are never read from memory: with NaN right after every input (L = 200 ends in a
    partial 64-key block), the outputs stay finite and match the oracle."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = 1, 2, 200, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=41, mask="tail", pair="normal", mask_frac=0.2)
    extra = 128 * H * D + 128 * L
    q, k, v, m, p = (nan_tailed(torch, x, dtype, extra) for x in (w.q, w.k, w.v, w.mask, w.pair))
    out, lse = E.fwd(q, k, v, m, p)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, "NaN after every input")


# ---------------------------------------------------------------------------
# Head dimension 64 on the 16-bit path: two 32-wide halves of the contraction,
# with bias tiles copied straight into LDS for L % 8 == 0 (64, 136, 200, 256)
# and staged through registers otherwise (1, 17, 100, 257).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 2, 17, 3), (2, 2, 64, 2), (1, 3, 100, 4), (1, 2, 257, 2),
                                   (1, 3, 136, 2), (2, 2, 200, 3)],
                         ids=lambda s: "x".join(map(str, s)))
def test_head_dim_64(torch_dev, shape, dtype):
    B, N, L, H = shape
    w = S.random_problem(B, N, L, H, 64, dtype=dtype, seed=B * 100 + N * 10 + L + H, mask="tail", pair="normal",
                         mask_frac=0.3)
    say(f"head dim 64 {dtype} {shape}")
    parity_full(torch_dev, w)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_head_dim_64_msa_row_shape(torch_dev, dtype):
    """An MSA-row problem with the largest head dimension the guide's backward allows (section 5.4: D <= 64)."""
    w = S.random_problem(1, 16, 256, 4, 64, dtype=dtype, seed=64, mask="tail", pair="normal", mask_frac=0.1)
    parity_full(torch_dev, w)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_head_dim_64_masked_and_peaked(torch_dev, dtype):
    """D = 64 with -inf masks (a partly and a fully masked sequence) and biases of scale 8."""
    B, N, L, H, D = 1, 3, 128, 2, 64
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=640, mask="zero", pair="normal", bias_scale=8.0)
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., 10:50] = -np.inf
    mf[0, 1] = -np.inf
    w.mask = S.to_storage(mf, dtype)
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    assert np.all(o[0, 1] == 0) and np.all(np.isneginf(l[0, 1]))
    compare(o, l, ro, rl, dtype, "head dim 64, masked and peaked")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_head_dim_64_neg_inf_pair_bias(torch_dev, dtype):
    """-inf in the pair bias at D = 64 (one key of a row, part of a row, a whole row): the identity product
    turns it into NaN, and the workgroups that meet it redo their slice on the exact path."""
    B, N, L, H, D = 1, 2, 96, 2, 64
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=641, mask="tail", pair="normal")
    pf = S.storage_to_f32(w.pair, dtype).copy()
    pf[0, 0, 1, 5, 7] = -np.inf
    pf[0, 0, 0, 70, :40] = -np.inf
    pf[0, 0, 1, 20, :] = -np.inf
    w.pair = S.to_storage(pf, dtype)
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, "head dim 64, infinite pair bias")


def test_head_dim_64_workload_size(torch_dev):
    """Triangle attention at N = L = 384, H = 4 with D = 64 (bf16), every element against the oracle."""
    w = S.random_problem(1, 384, 384, 4, 64, dtype="bf16", seed=642, mask="tail", pair="normal")
    say("head dim 64 at N = L = 384, full oracle comparison")
    parity_full(torch_dev, w)


# ---------------------------------------------------------------------------
# Whole 64-key blocks masked by a large finite value (the guide's additive
# mask form, section 5.2).  A fully masked leading block sets the running
# maximum of every row near the mask value; the first live block must then
# wipe what that block added (its rescale factor is exactly 0).  A fully
# masked middle block must add nothing.  bf16 keeps -1e9 finite; binary16
# cannot, so it takes -3e4 (finite) as well as -1e9 (which arrives as -inf).
# L % 8 == 0 copies the bias tiles straight into LDS, L % 8 != 0 stages them.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,value", [("bf16", -1e9), ("bf16", -math.inf), ("f16", -3e4), ("f16", -1e9)])
@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("L", [256, 251])
def test_masked_leading_and_middle_blocks(torch_dev, L, D, dtype, value):
    B, N, H = 1, 4, 2
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=L + D + 7, mask="zero", pair="normal")
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 0, ..., :64] = value               # the whole leading block
    mf[0, 1, ..., 64:128] = value            # a whole middle block
    mf[0, 2, ..., :128] = value              # two leading blocks
    mf[0, 2, ..., 200:] = value              # and the tail
    mf[0, 3, ..., :64] = value               # leading block and every other block but one key
    mf[0, 3, ..., 65:] = value
    w.mask = S.to_storage(mf, dtype)
    say(f"masked blocks {dtype} value={value} L={L} D={D}")
    parity_full(torch_dev, w)


@pytest.mark.parametrize("value", [-1e9, -1e10, -1e30])
@pytest.mark.parametrize("L", [192, 77])
def test_bf16_rows_fully_masked_by_a_finite_value(torch_dev, L, value):
    """Every key of a sequence carries one large finite mask value (bf16 keeps it finite).  fp32 scores
    cannot resolve q.k next to such a value, so these rows are outside the parity bound; what the call
    returns for them is: finite values, each output a convex combination of the value rows, and lse
    equal to the oracle's within fp32 rounding of its magnitude.  The other sequences keep full parity."""
    B, N, H, D = 1, 3, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=L + 3, mask="zero", pair="normal")
    mf = np.zeros((B, N, 1, 1, L), np.float32)
    mf[0, 1] = value
    mf[0, 2, ..., L // 2:] = value
    w.mask = S.to_storage(mf, "bf16")
    o, l = run_gpu(torch_dev, w)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    full = np.zeros(N, bool)
    full[1] = True
    assert np.isfinite(o).all() and np.isfinite(l).all(), "non-finite output on a fully masked row"
    vf = S.storage_to_f32(w.v, "bf16")[:, full]
    vmax = np.abs(vf).max(axis=2, keepdims=True)
    assert (np.abs(o[:, full]) <= vmax * (1 + 2 ** -7) + 1e-6).all()
    rel = np.abs(l[:, full] - rl[:, full]) / np.abs(rl[:, full])
    say(f"  fully masked by {value}: lse relative error {rel.max():.2e}")
    assert rel.max() <= 1e-6
    compare(o[:, ~full], l[:, ~full], ro[:, ~full], rl[:, ~full], "bf16", f"other sequences, mask {value}")
