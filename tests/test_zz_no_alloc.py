"""evo_attn_bwd_noalloc (the backward pass with the library's static scratch, no allocation) against
evo_attn_bwd with a caller workspace of the recommended size, through the C ABI.

Both run the same kernels with the same split of the pair gradient's N axis, and every sum is formed in a
fixed order, so the gradients must be bit-identical.  Two calls in a row, the second on a smaller problem:
the scratch keeps the first call's partial sums, which the second must not see.
"""
import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import evoformer_biased_attention_amd  # noqa: F401
    return torch


def dev(torch, x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "f32":
        return t.to("cuda")
    return (t.view(torch.bfloat16) if dtype == "bf16" else t.view(torch.float16)).to("cuda")


def both(torch, shape, dtype, seed, over_scratch=False):
    """The static-scratch call against evo_attn_bwd with a caller workspace: of the recommended size, or, when
    that exceeds the scratch (over_scratch), of the scratch's size, which gives the same split of N."""
    import evoformer_biased_attention_amd as E
    B, N, L, H, D = shape
    w = S.random_problem(B, N, L, H, D, dtype=dtype, seed=seed, mask="tail", pair="normal")
    q, k, v, m, p = (dev(torch, x, dtype) for x in (w.q, w.k, w.v, w.mask, w.pair))
    do = dev(torch, S.random_dout(shape, dtype, seed=seed + 1), dtype)
    out, lse = E.fwd(q, k, v, m, p)
    code = E.torch_dtype_code(q.dtype)
    need = E.evo_attn_bwd_workspace_size(shape, code)
    scratch = E.evo_attn_bwd_noalloc_scratch_bytes()
    if over_scratch:
        assert need > scratch
        need = scratch
    assert 0 < need <= scratch
    stream = torch.cuda.current_stream().cuda_stream
    results = []
    for noalloc in (False, True):
        g = [torch.full_like(x, float("nan")) for x in (q, k, v, m, p)]
        delta = torch.full((B, N, H, L), float("nan"), dtype=torch.float32, device="cuda")
        print(f"  {'noalloc' if noalloc else 'workspace'} bwd {shape} {dtype} (recommended workspace {need} B)",
              flush=True)
        if noalloc:
            st = E.evo_attn_bwd_noalloc(q, k, v, m, p, out, lse, do, *g, delta, shape, code, stream)
        else:
            ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
            st = E.evo_attn_bwd(q, k, v, m, p, out, lse, do, *g, delta, shape, code, stream, workspace=ws,
                                workspace_bytes=need)
        assert st == E.EVO_OK, E.evo_status_string(st)
        torch.cuda.synchronize()
        results.append([x.clone() for x in g + [delta]])
    for name, a, b in zip(("dq", "dk", "dv", "dmask", "dpair", "delta"), *results):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), f"{name} differs between the workspace and the static-scratch call"


def test_noalloc_matches_workspace_call_twice(torch_dev):
    both(torch_dev, (1, 64, 384, 4, 32), "bf16", 7001)   # 16.5 MB of partial sums (7 chunks)
    both(torch_dev, (1, 24, 200, 2, 32), "f16", 7002)    # then a smaller problem: 0.96 MB


def test_noalloc_splits_what_fits_in_the_scratch(torch_dev):
    """N = L = 768: the recommended workspace (16 chunks, 151 MB) exceeds the 40 MiB scratch; the call splits N
    into the 4 chunks that fit, bit-identical to evo_attn_bwd given a workspace of the scratch's size.  Then a
    smaller problem that fits whole."""
    both(torch_dev, (1, 768, 768, 4, 32), "bf16", 7007, over_scratch=True)
    both(torch_dev, (1, 24, 200, 2, 32), "f16", 7008)


def test_noalloc_matches_workspace_call_twice_f32(torch_dev):
    """fp32 inputs on the fp32 matrix-core kernels, whose pair gradient uses the same split of N."""
    both(torch_dev, (1, 48, 256, 4, 32), "f32", 7005)    # 6.3 MB of partial sums
    both(torch_dev, (1, 24, 136, 2, 16), "f32", 7006)    # then a smaller problem with D = 16


def test_noalloc_without_pair_gradient_uses_no_scratch(torch_dev):
    torch = torch_dev
    import evoformer_biased_attention_amd as E
    shape = (1, 8, 96, 2, 32)
    B, N, L, H, D = shape
    w = S.random_problem(*shape, dtype="bf16", seed=7003, mask="tail", pair="normal")
    q, k, v, m, p = (dev(torch, x, "bf16") for x in (w.q, w.k, w.v, w.mask, w.pair))
    do = dev(torch, S.random_dout(shape, "bf16", seed=7004), "bf16")
    out, lse = E.fwd(q, k, v, m, p)
    stream = torch.cuda.current_stream().cuda_stream
    ref = [torch.empty_like(x) for x in (q, k, v, m)]
    got = [torch.empty_like(x) for x in (q, k, v, m)]
    d1 = torch.empty((B, N, H, L), dtype=torch.float32, device="cuda")
    d2 = torch.empty_like(d1)
    assert E.evo_attn_bwd(q, k, v, m, p, out, lse, do, *ref, None, d1, shape, E.EVO_DTYPE_BF16, stream) == E.EVO_OK
    assert E.evo_attn_bwd_noalloc(q, k, v, m, p, out, lse, do, *got, None, d2, shape, E.EVO_DTYPE_BF16,
                                  stream) == E.EVO_OK
    torch.cuda.synchronize()
    for a, b in zip(ref + [d1], got + [d2]):
        assert torch.equal(a, b)
