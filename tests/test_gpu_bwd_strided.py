"""Strided backward: evo_attn_bwd_strided on views against the fp64 oracle on dense copies.

Triangle attention around the ending node and MSA column attention attend
along the other axis of the tensors their row-wise counterparts use (section
5.3 of the guide).  Their training step reads Q, K, V, out and dO as views of
the untransposed tensors, and writes dQ, dK, dV into views of the same
layout; the oracle gets numpy's dense transposed copies of the same values,
and the gradients come back through the views in [B,N,L,H,D] index order.
Tolerances are those of the dense backward tests.  Every output is poisoned
with NaN before the launch, padding included, and padding must stay NaN.
"""
import numpy as np
import pytest

import oracle
import synthetic as S
from test_gpu_bwd_parity import THREADS, compare_delta, compare_grads, f64, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401
    return torch


def strided_bwd(torch, q, k, v, mask, pair, dout, lse_row=None, use_ws=True, pair_storage=None):
    """Forward and backward through the strided entry points on views q, k, v, dout [B,N,L,H,D].

    out and dq/dk/dv are allocated with the strides of dout and q/k/v.  Returns (grads as float64
    numpy in [B,N,L,H,D] order, delta [B,N,H,L], raw tensors)."""
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = q.shape
    row = L if lse_row is None else lse_row
    like = lambda t: _nan_strided(torch, t)
    out = like(dout)
    lse = torch.full((B, N, H, row), float("nan"), dtype=torch.float32, device="cuda")[..., :L]
    code = E.torch_dtype_code(q.dtype)
    lay = E.layout_of(q, k, v, out, mask, pair, lse_row=row)
    st = E.evo_attn_fwd_strided(q, k, v, mask, pair, out, lse, lay, (B, N, L, H, D), code,
                                torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_OK, E.evo_status_string(st)
    dq, dk, dv = like(q), like(k), like(v)
    dmask = like(mask) if mask is not None else None
    dpair = _nan_strided(torch, pair, pair_storage) if pair is not None else None
    delta = torch.full((B, N, H, row), float("nan"), dtype=torch.float32, device="cuda")[..., :L]
    ws_bytes = E.evo_attn_bwd_workspace_size((B, N, L, H, D), code) if (use_ws and pair is not None) else 0
    ws = torch.full((ws_bytes // 4,), float("nan"), dtype=torch.float32, device="cuda") if ws_bytes else None
    say(f"  strided bwd {tuple(q.shape)} {q.dtype} q strides {tuple(q.stride())} lse_row {row} ws {ws_bytes}")
    st = E.evo_attn_bwd_strided(q, k, v, mask, pair, out, lse, dout, dq, dk, dv, dmask, dpair, delta, lay,
                                (B, N, L, H, D), code, torch.cuda.current_stream().cuda_stream, workspace=ws,
                                workspace_bytes=ws_bytes)
    assert st == E.EVO_OK, E.evo_status_string(st)
    torch.cuda.synchronize()
    return [f64(x) for x in (dq, dk, dv, dmask, dpair)], f64(delta), (dq, dk, dv, dmask, dpair, delta, out)


def _nan_strided(torch, t, storage=None):
    """A NaN-filled tensor with t's sizes and strides (its own storage, or the given wider one)."""
    if storage is None:
        span = 1 + sum((s - 1) * st for s, st in zip(t.size(), t.stride()))
        storage = torch.full((span,), float("nan"), dtype=t.dtype, device=t.device)
    else:
        storage.fill_(float("nan"))
    return storage.as_strided(t.size(), t.stride())


def transposed(torch, x, dtype):
    """Device tensor holding x[B, N, L, H, D] transposed in memory (X[B, L, N, H, D]), returned as the
    [B, N, L, H, D] view of it."""
    return to_dev(torch, np.ascontiguousarray(x.transpose(0, 2, 1, 3, 4)), dtype).permute(0, 2, 1, 3, 4)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("dims", [(1, 64, 64, 4, 32), (2, 40, 96, 2, 16), (1, 72, 100, 3, 32), (1, 136, 136, 4, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ending_node_training_in_place(torch_dev, dims, dtype):
    """Q/K/V/O/dO and dQ/dK/dV of triangle attention around the ending node, all views of [B, L_i, L_j, H, D]
    (n = j, l = i).  L = 100 runs the vector-ALU kernels, the others the matrix cores for 16-bit."""
    torch = torch_dev
    B, N, L, H, D = dims
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=sum(dims) + 1, mask="tail", pair="normal", mask_frac=0.2)
    dout = S.random_dout(w.shape, dtype, seed=sum(dims))
    q, k, v, do = (transposed(torch, x, dtype) for x in (w.q, w.k, w.v, dout))
    got, delta, raw = strided_bwd(torch, q, k, v, to_dev(torch, w.mask, dtype), to_dev(torch, w.pair, dtype), do)
    assert all(not t.is_contiguous() for t in raw[:3])
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(got, want, dtype, f"ending node {dims}")
    compare_delta(delta, w, dout, f"ending node {dims}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_column_attention_training_in_place(torch_dev, dtype):
    """MSA column attention: [B, N_res, N_seq, H, D] views of the MSA tensor, a mask and no pair bias."""
    torch = torch_dev
    B, N, L, H, D = 1, 64, 128, 8, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=78, mask="tail", pair=None)
    dout = S.random_dout(w.shape, dtype, seed=79)
    q, k, v, do = (transposed(torch, x, dtype) for x in (w.q, w.k, w.v, dout))
    got, delta, _ = strided_bwd(torch, q, k, v, to_dev(torch, w.mask, dtype), None, do)
    want = oracle.bwd(w.q, w.k, w.v, w.mask, None, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(got, want, dtype, "column attention")
    compare_delta(delta, w, dout, "column attention")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("use_ws", [True, False], ids=["workspace", "no_workspace"])
def test_padded_lse_and_pair_rows(torch_dev, use_ws, dtype):
    """lse and delta in the guide's padded rows (ceil(L/32)*32, section 5.4) and a pair bias whose rows and
    matrices are padded (a slice of a wider tensor); dpair is written in the same padded layout and its
    padding, like delta's, is left alone.  fp32 here runs on the fp32 matrix-core kernels."""
    torch = torch_dev
    B, N, L, H, D = 1, 24, 80, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=81, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, dtype, seed=82)
    row = (L + 31) // 32 * 32
    pad_i, pad_l = L + 8, L + 16  # pair rows 88 apart; 96 rows per matrix
    wide = np.zeros((B, 1, H, pad_l, pad_i), w.pair.dtype)
    wide[..., :L, :L] = w.pair
    pair_full = to_dev(torch, wide, dtype)
    pair = pair_full[..., :L, :L]
    q, k, v, do = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v, dout))
    dpair_store = torch.empty_like(pair_full).reshape(-1)
    got, delta, raw = strided_bwd(torch, q, k, v, to_dev(torch, w.mask, dtype), pair, do, lse_row=row,
                                  use_ws=use_ws, pair_storage=dpair_store)
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(got, want, dtype, f"padded rows, workspace={use_ws}")
    compare_delta(delta, w, dout, "padded rows")
    full = dpair_store.view(B, 1, H, pad_l, pad_i).float()
    assert torch.isnan(full[..., L:, :]).all() and torch.isnan(full[..., :L, L:]).all()
    d = raw[5].as_strided((B, N, H, row), (N * H * row, H * row, row, 1))
    assert torch.isnan(d[..., L:]).all()


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("use_ws", [True, False], ids=["workspace", "no_workspace"])
@pytest.mark.parametrize("L", [77, 96])
def test_unaligned_bias_rows(torch_dev, L, use_ws, dtype):
    """Pair rows L + 1 apart (matrices L + 3 rows apart) and mask rows L + 3 apart: every bias row starts
    at another alignment, also for L % 8 == 0, so the bias tiles are staged through registers.
    dpair and dmask are written in the same layouts and their padding is left alone."""
    torch = torch_dev
    B, N, H, D = 1, 24, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=L + 300, mask="tail", pair="normal")
    pf = S.storage_to_f32(w.pair, dtype).copy()
    pf[..., :, -1] = 3.0
    w.pair = S.to_storage(pf, dtype)
    dout = S.random_dout(w.shape, dtype, seed=L + 301)
    pad_i, pad_l = L + 1, L + 3
    wide = np.zeros((B, 1, H, pad_l, pad_i), w.pair.dtype)
    wide[..., :L, :L] = w.pair
    pair_full = to_dev(torch, wide, dtype)
    pair = pair_full[..., :L, :L]
    wide_m = np.zeros((B, N, 1, 1, L + 3), w.mask.dtype)
    wide_m[..., :L] = w.mask
    mask = to_dev(torch, wide_m, dtype)[..., :L]
    q, k, v, do = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v, dout))
    dpair_store = torch.empty_like(pair_full).reshape(-1)
    got, delta, raw = strided_bwd(torch, q, k, v, mask, pair, do, use_ws=use_ws, pair_storage=dpair_store)
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(got, want, dtype, f"unaligned bias rows L={L}, workspace={use_ws}")
    compare_delta(delta, w, dout, "unaligned bias rows")
    full = dpair_store.view(B, 1, H, pad_l, pad_i).float()
    assert torch.isnan(full[..., L:, :]).all() and torch.isnan(full[..., :L, L:]).all()


@pytest.mark.parametrize("use_ws", [True, False], ids=["workspace", "no_workspace"])
@pytest.mark.parametrize("L,fill", [(77, 0.0), (99, float("nan"))], ids=["77-zeros", "99-nan"])
def test_padded_bias_rows_any_L(torch_dev, L, fill, use_ws):
    """L % 8 != 0 with the pair and mask rows (and so their gradients' rows) padded to a multiple of 8
    elements: the bias tiles are copied straight into LDS, each row's last chunk read whole with its
    padding (NaN in one case), and the gradients leave the padding alone."""
    torch = torch_dev
    B, N, H, D = 1, 24, 2, 32
    dtype = "bf16"
    Lp = (L + 7) // 8 * 8
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=L + 800, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, dtype, seed=L + 801)
    fill_bits = S.to_storage(np.full(1, fill, np.float32), dtype)[0]
    wide = np.full((B, 1, H, L, Lp), fill_bits, np.uint16)
    wide[..., :L] = w.pair
    pair_full = to_dev(torch, wide, dtype)
    pair = pair_full[..., :L]
    wide_m = np.full((B, N, 1, 1, Lp), fill_bits, np.uint16)
    wide_m[..., :L] = w.mask
    mask = to_dev(torch, wide_m, dtype)[..., :L]
    q, k, v, do = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v, dout))
    dpair_store = torch.empty_like(pair_full).reshape(-1)
    got, delta, raw = strided_bwd(torch, q, k, v, mask, pair, do, use_ws=use_ws, pair_storage=dpair_store)
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(got, want, dtype, f"padded bias rows L={L} fill={fill}, workspace={use_ws}")
    compare_delta(delta, w, dout, "padded bias rows")
    full = dpair_store.view(B, 1, H, L, Lp).float()
    assert torch.isnan(full[..., L:]).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_major_layout_runs_and_matches(torch_dev, dtype):
    """Q/K/V/dO as views of [B, N, H, L, D] (heads outermost): rows do not span every head, so the 16-bit
    call runs on the vector-ALU kernels; the gradients still match."""
    torch = torch_dev
    B, N, L, H, D = 1, 8, 64, 4, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=83, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, dtype, seed=84)
    hm = lambda x: to_dev(torch, np.ascontiguousarray(x.transpose(0, 1, 3, 2, 4)), dtype).permute(0, 1, 3, 2, 4)
    q, k, v, do = (hm(x) for x in (w.q, w.k, w.v, dout))
    got, delta, _ = strided_bwd(torch, q, k, v, to_dev(torch, w.mask, dtype), to_dev(torch, w.pair, dtype), do)
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype=dtype, nthreads=THREADS)
    compare_grads(got, want, dtype, "head-major layout")


@pytest.mark.parametrize("D", [8, 32])
def test_f32_row_offsets_past_31_bits(torch_dev, D):
    """fp32 Q rows 4,000,000 floats apart (Q, and so dQ, in 256 MB buffers): the byte offsets of the rows up
    to 128 past L exceed 2^31, which the matrix-core kernels do not form, so both passes run on the
    vector-ALU kernels; out and every gradient still match the oracle."""
    torch = torch_dev
    from test_gpu_parity import compare as compare_fwd
    B, N, L, H, rs = 1, 1, 16, 2, 4_000_000
    w = S.random_problem(B, N, L, H, D, dtype="f32", seed=95 + D, mask="tail", pair="normal", mask_frac=0.2)
    dout = S.random_dout(w.shape, "f32", seed=96 + D)
    buf = torch.zeros((L, rs), dtype=torch.float32, device="cuda")
    buf[:, : H * D].copy_(to_dev(torch, w.q, "f32").reshape(L, H * D))
    q = buf[:, : H * D].view(L, H, D)[None, None]
    assert q.stride(2) == rs
    k, v, do = (to_dev(torch, x, "f32") for x in (w.k, w.v, dout))
    got, delta, raw = strided_bwd(torch, q, k, v, to_dev(torch, w.mask, "f32"), to_dev(torch, w.pair, "f32"), do)
    ro, rl = oracle.fwd(w.q, w.k, w.v, w.mask, w.pair, dtype="f32", nthreads=THREADS)
    compare_fwd(f64(raw[6]), None, ro, None, "f32", f"rows {rs} apart, D={D}")
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="f32", nthreads=THREADS)
    compare_grads(got, want, "f32", f"rows {rs} apart, D={D}")
    compare_delta(delta, w, dout, f"rows {rs} apart, D={D}")
    del buf


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_dense_layout_through_strided_entry_is_identical(torch_dev, dtype):
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    w = S.random_problem(1, 16, 64, 2, 32, dtype=dtype, seed=85, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, dtype, seed=86)
    q, k, v, m, p, do = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v, w.mask, w.pair, dout))
    out, lse = E.fwd(q, k, v, m, p)
    code = E.torch_dtype_code(q.dtype)
    res = []
    for strided in (False, True):
        g = [torch.full_like(t, float("nan")) for t in (q, k, v, m, p)]
        delta = torch.full_like(lse, float("nan"))
        args = (q, k, v, m, p, out, lse, do, *g, delta)
        stream = torch.cuda.current_stream().cuda_stream
        if strided:
            st = E.evo_attn_bwd_strided(*args, E.evo_attn_dense_layout(w.shape), w.shape, code, stream)
        else:
            st = E.evo_attn_bwd(*args, w.shape, code, stream)
        assert st == E.EVO_OK
        res.append(g + [delta])
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_binding_bwd_returns_gradients_in_the_views_layout(torch_dev):
    """The torch wrapper allocates each gradient with its tensor's strides."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = 1, 32, 64, 4, 32
    w = S.random_problem(B, N, L, H, D, dtype="bf16", seed=87, mask="tail", pair="normal")
    dout = S.random_dout(w.shape, "bf16", seed=88)
    q, k, v, do = (transposed(torch, x, "bf16") for x in (w.q, w.k, w.v, dout))
    m, p = to_dev(torch, w.mask, "bf16"), to_dev(torch, w.pair, "bf16")
    out = torch.empty_like(do)
    lse = torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")
    st = E.evo_attn_fwd_strided(q, k, v, m, p, out, lse, E.layout_of(q, k, v, out, m, p), w.shape,
                                E.EVO_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_OK
    dq, dk, dv, dm, dp, delta = E.bwd(q, k, v, m, p, out, lse, do)
    torch.cuda.synchronize()
    assert dq.stride() == q.stride() and dk.stride() == k.stride() and dv.stride() == v.stride()
    want = oracle.bwd(w.q, w.k, w.v, w.mask, w.pair, dout, dtype="bf16", nthreads=THREADS)
    compare_grads([f64(x) for x in (dq, dk, dv, dm, dp)], want, "bf16", "binding on views")
