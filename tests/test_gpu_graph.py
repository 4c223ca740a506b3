"""The forward and backward launches captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Neither pass allocates, frees, synchronises or clears memory with a memset, so
both can be captured.  Each test replays the graph several times, with eager
work and synchronisations between the replays, changes the inputs in place
between replays, and checks every replay bit for bit against an eager call on
the same inputs.
"""
import numpy as np
import pytest

import synthetic as S
from test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401
    return torch


@pytest.mark.parametrize("L", [96, 77])
def test_forward_graph_replays(torch_dev, L):
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    w = S.random_problem(1, 6, L, 2, 32, dtype="bf16", seed=900 + L, mask="tail", pair="normal")
    q, k, v, m, p = (to_dev(torch, x, "bf16") for x in (w.q, w.k, w.v, w.mask, w.pair))
    out = torch.empty_like(q)
    lse = torch.empty((1, 6, 2, L), dtype=torch.float32, device="cuda")
    code = E.torch_dtype_code(q.dtype)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        assert E.evo_attn_fwd(q, k, v, m, p, out, lse, w.shape, code, side.cuda_stream) == E.EVO_OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = E.evo_attn_fwd(q, k, v, m, p, out, lse, w.shape, code, torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_OK
    gen = torch.Generator(device="cuda").manual_seed(L)
    for rep in range(4):
        q.copy_(torch.randn(q.shape, device="cuda", generator=gen).to(q.dtype))  # new inputs, same buffers
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = E.fwd(q, k, v, m, p)
        _ = (ref_o.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {rep}"


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_graph_replays(torch_dev, dtype, entry):
    """The backward captured and replayed: with its workspace (pair gradient split over N), or through the
    no-allocation entry point (the split's partial sums in the library's static array), on the 16-bit and the
    fp32 matrix-core kernels."""
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = 1, 24, 80, 2, 32
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=910, mask="tail", pair="normal")
    q, k, v, m, p = (to_dev(torch, x, dtype) for x in (w.q, w.k, w.v, w.mask, w.pair))
    dout = to_dev(torch, S.random_dout(w.shape, dtype, seed=911), dtype)
    out, lse = E.fwd(q, k, v, m, p)
    code = E.torch_dtype_code(q.dtype)
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(m), torch.empty_like(p)]
    delta = torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")
    ws_bytes = E.evo_attn_bwd_workspace_size(w.shape, code)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")

    def launch(stream):
        if entry == "noalloc":  # its first call on the device (the warm-up below) looks up the array's address
            return E.evo_attn_bwd_noalloc(q, k, v, m, p, out, lse, dout, *grads, delta, w.shape, code, stream)
        return E.evo_attn_bwd(q, k, v, m, p, out, lse, dout, *grads, delta, w.shape, code, stream, workspace=ws,
                              workspace_bytes=ws_bytes)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert launch(side.cuda_stream) == E.EVO_OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = launch(torch.cuda.current_stream().cuda_stream)
    assert st == E.EVO_OK
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(4):
        dout.copy_(torch.randn(dout.shape, device="cuda", generator=gen).to(dout.dtype))
        ws.fill_(float("nan"))  # the workspace's contents are not carried over between calls
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in grads] + [delta.clone()]
        ref = E.bwd(q, k, v, m, p, out, lse, dout)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep}"
