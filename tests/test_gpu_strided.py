"""Strided (zero-copy) layouts: evo_attn_fwd_strided against the fp64 oracle on dense copies.

The GPU reads views of the untransposed tensors through evo_layout_t; the
oracle gets numpy's dense transposed copies of the same values.  Section 5.3
of the guide: triangle attention around the ending node and MSA column
attention attend along the other axis of the tensors their row-wise
counterparts use.  Tolerances are those of the dense forward tests.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from test_gpu_parity import THREADS, compare, parity_full, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401
    return torch


def gpu_strided(torch, q, k, v, mask, pair, out, lse_row=None, lse_fill=None):
    """q, k, v, out: device views [B,N,L,H,D]; returns (out float64 numpy in the view's index order, lse, raw lse)."""
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = q.shape
    lay = E.layout_of(q, k, v, out, mask, pair, lse_row=lse_row)
    row = lay.lse_row
    lse_buf = torch.full((B * N * H * row,), float("nan") if lse_fill is None else lse_fill, dtype=torch.float32,
                         device="cuda")
    say(f"  strided {tuple(q.shape)} q strides {tuple(q.stride())} lse_row {row}")
    st = E.evo_attn_fwd_strided(q, k, v, mask, pair, out, lse_buf, lay, (B, N, L, H, D), E.torch_dtype_code(q.dtype),
                                torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_OK, E.evo_status_string(st)
    torch.cuda.synchronize()
    raw = lse_buf.cpu().numpy().reshape(B, N, H, row)
    return out.float().cpu().numpy().astype(np.float64), raw[..., :L].astype(np.float64), raw


def transposed_problem(B, Li, Lj, H, D, dtype, seed, mask=True, pair=True):
    """X tensors [B, Li, Lj, H, D] and biases for attention along i (n = j, l = i)."""
    w = S.random_problem(B, Lj, Li, H, D, dtype=dtype, seed=seed, mask="tail" if mask else None,
                         pair="normal" if pair else None, mask_frac=0.2)
    # w.q etc. are the dense [B, N=Lj, L=Li, H, D] tensors; X is their transpose
    X = {n: np.ascontiguousarray(getattr(w, n).transpose(0, 2, 1, 3, 4)) for n in ("q", "k", "v")}
    return w, X


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("dims", [(1, 64, 64, 4, 32), (2, 96, 40, 2, 16), (1, 100, 72, 3, 32), (1, 192, 192, 4, 32)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ending_node_reads_untransposed_tensors(torch_dev, dims, dtype):
    """Q/K/V/O of triangle attention around the ending node as views of X[B, L_i, L_j, H, D]."""
    torch = torch_dev
    B, Li, Lj, H, D = dims
    w, X = transposed_problem(B, Li, Lj, H, D, dtype, seed=sum(dims))
    xq, xk, xv = (to_dev(torch, X[n], dtype) for n in ("q", "k", "v"))
    xo = torch.full_like(xq, float("nan"))
    view = lambda t: t.permute(0, 2, 1, 3, 4)  # [B, Lj, Li, H, D], no copy
    o, l, _ = gpu_strided(torch, view(xq), view(xk), view(xv), to_dev(torch, w.mask, dtype),
                          to_dev(torch, w.pair, dtype), view(xo))
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, f"ending node {dims}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_column_attention_reads_the_msa_tensor(torch_dev, dtype):
    """MSA column attention: Q/K/V [B, N_res, N_seq, H, D] as views of the MSA tensor [B, N_seq, N_res, H, D]."""
    torch = torch_dev
    B, Nseq, Nres, H, D = 1, 128, 64, 8, 32
    w, X = transposed_problem(B, Nseq, Nres, H, D, dtype, seed=77, pair=False)
    xq, xk, xv = (to_dev(torch, X[n], dtype) for n in ("q", "k", "v"))
    xo = torch.full_like(xq, float("nan"))
    view = lambda t: t.permute(0, 2, 1, 3, 4)
    o, l, _ = gpu_strided(torch, view(xq), view(xk), view(xv), to_dev(torch, w.mask, dtype), None, view(xo))
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, None, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, "column attention")


@pytest.mark.parametrize("L", [100, 128, 200])
def test_padded_lse_rows(torch_dev, L):
    """The guide's padded LSE layout, rows of ceil(L/32)*32 (section 5.4); the padding is left untouched."""
    torch = torch_dev
    w = S.random_problem(1, 3, L, 2, 32, dtype="bf16", seed=L, mask="tail", pair="normal")
    row = (L + 31) // 32 * 32
    q, k, v, m, p = (to_dev(torch, x, "bf16") for x in (w.q, w.k, w.v, w.mask, w.pair))
    out = torch.full_like(q, float("nan"))
    o, l, raw = gpu_strided(torch, q, k, v, m, p, out, lse_row=row, lse_fill=7.0)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    compare(o, l, ro, rl, "bf16", f"padded lse L={L}")
    assert np.all(raw[..., L:] == 7.0)


@pytest.mark.parametrize("pad", [8, 3])
def test_padded_pair_rows(torch_dev, pad):
    """Pair rows L + pad apart (a slice of a wider tensor); pad = 3 leaves the rows unaligned (staged copies)."""
    torch = torch_dev
    B, N, L, H, D = 1, 4, 96, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=90 + pad, mask="tail", pair="normal")
    wide = np.zeros((B, 1, H, L, L + pad), np.uint16)
    wide[..., :L] = w.pair
    pair = to_dev(torch, wide, "bf16")[..., :L]
    q, k, v, m = (to_dev(torch, x, "bf16") for x in (w.q, w.k, w.v, w.mask))
    out = torch.full_like(q, float("nan"))
    o, l, _ = gpu_strided(torch, q, k, v, m, pair, out)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    compare(o, l, ro, rl, "bf16", f"pair rows L+{pad}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L", [77, 96])
def test_unaligned_bias_rows(torch_dev, L, dtype):
    """Pair rows L + 1 apart and mask rows L + 3 apart (slices of wider tensors): the bias rows start at
    every 2-byte alignment, also for L % 8 == 0.  Large biases sit on the last element of each row."""
    torch = torch_dev
    B, N, H, D = 2, 3, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=1200 + L, mask="tail", pair="normal")
    pf = S.storage_to_f32(w.pair, dtype).copy()
    pf[..., :, -1] = 5.0
    mf = S.storage_to_f32(w.mask, dtype).copy()
    mf[..., -1] = 3.0
    w.pair, w.mask = S.to_storage(pf, dtype), S.to_storage(mf, dtype)
    wide_p = np.zeros((B, 1, H, L, L + 1), np.uint16)
    wide_p[..., :L] = w.pair
    wide_m = np.zeros((B, N, 1, 1, L + 3), np.uint16)
    wide_m[..., :L] = w.mask
    pair = to_dev(torch, wide_p, dtype)[..., :L]
    mask = to_dev(torch, wide_m, dtype)[..., :L]
    q, k, v = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v))
    out = torch.full_like(q, float("nan"))
    o, l, _ = gpu_strided(torch, q, k, v, mask, pair, out)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, f"unaligned bias rows L={L}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("L,fill", [(77, 0.0), (99, 0.0), (130, 0.0), (77, float("nan")), (77, float("inf"))],
                         ids=["77-zeros", "99-zeros", "130-zeros", "77-nan", "77-inf"])
def test_padded_bias_rows_any_L(torch_dev, L, fill, dtype):
    """L % 8 != 0 with bias rows padded to a multiple of 8 elements: the rows start 16-byte aligned, so
    the bias tiles are copied straight into LDS and each row's last chunk is read whole, padding (keys
    past L) included.  Padding that holds NaN or inf turns the identity product's zeros into NaN; the
    workgroups that meet it redo their slice on the exact path, with the same results."""
    torch = torch_dev
    B, N, H, D = 1, 3, 2, 32
    Lp = (L + 7) // 8 * 8
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=L + 700, mask="tail", pair="normal")
    fill_bits = S.to_storage(np.full(1, fill, np.float32), dtype)[0]
    wide_p = np.full((B, 1, H, L, Lp), fill_bits, np.uint16)
    wide_p[..., :L] = w.pair
    wide_m = np.full((B, N, 1, 1, Lp), fill_bits, np.uint16)
    wide_m[..., :L] = w.mask
    pair = to_dev(torch, wide_p, dtype)[..., :L]
    mask = to_dev(torch, wide_m, dtype)[..., :L]
    q, k, v = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v))
    out = torch.full_like(q, float("nan"))
    o, l, _ = gpu_strided(torch, q, k, v, mask, pair, out)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype=dtype, nthreads=THREADS)
    compare(o, l, ro, rl, dtype, f"padded bias rows L={L} fill={fill}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_dense_layout_through_strided_entry_is_identical(torch_dev, dtype):
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    w = S.random_problem(1, 3, 80, 2, 32, dtype=dtype, seed=5, mask="tail", pair="normal")
    q, k, v, m, p = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v, w.mask, w.pair))
    o1, l1 = E.fwd(q, k, v, m, p)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    st = E.evo_attn_fwd_strided(q, k, v, m, p, o2, l2, E.evo_attn_dense_layout(w.shape), w.shape,
                                E.torch_dtype_code(q.dtype), torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_transposed_layout_at_workload_size(torch_dev):
    """Workload 5 (ending node, N = L = 768, bf16) with Q/K/V/O stored as X[B, L, N, H, D]: the launch that
    `bench.py --workload 5 --layout transposed` times, every element against the full oracle."""
    torch = torch_dev
    w = S.workload(5)
    B, N, L, H, D = w.shape
    X = {n: np.ascontiguousarray(getattr(w, n).transpose(0, 2, 1, 3, 4)) for n in ("q", "k", "v")}
    view = lambda t: t.permute(0, 2, 1, 3, 4)
    xq, xk, xv = (to_dev(torch, X[n], "bf16") for n in ("q", "k", "v"))
    xo = torch.full_like(xq, float("nan"))
    o, l, _ = gpu_strided(torch, view(xq), view(xk), view(xv), None, to_dev(torch, w.pair, "bf16"), view(xo))
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="bf16", nthreads=THREADS)
    compare(o, l, ro, rl, "bf16", "workload 5, transposed layout")


def test_ds4sci_benchmark_shape_batch16_f16(torch_dev):
    """The largest batch of the DS4Sci benchmark sweep (16 x 256 x 256, H = 4, D = 32, fp16, mask and pair
    bias), in the dense launch `bench.py --sweep ds4sci` times, every element against the full oracle."""
    w = S.random_problem(16, 256, 256, 4, 32, dtype="f16", seed=4781, mask="tail", pair="normal")
    say("ds4sci benchmark shape, batch 16, f16")
    parity_full(torch_dev, w)
