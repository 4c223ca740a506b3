"""The C ABI on the host: symbols, enum values and the pure-host validation.

No compute call is made here (no GPU is needed): evo_attn_check never
dereferences its pointers, so fake, aligned addresses are enough.
"""
import ctypes
import os
import re

import pytest

import evoformer_biased_attention_amd as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "evo_attn.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def test_header_declares_exactly_the_exported_names():
    decls = set(re.findall(r"^\s*(?:const\s+char\s*\*|evo_status_t|int|size_t|void)\s+(evo_\w+)\s*\(", _header_text(),
                           re.M))
    assert decls == set(E.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(E.LIB_PATH)
    for name in E.EXPORTED:
        assert hasattr(lib, name), name


def test_enum_values_match_header():
    text = _header_text()
    for name in ("EVO_DTYPE_F32", "EVO_DTYPE_BF16", "EVO_DTYPE_F16", "EVO_OK", "EVO_ERR_NULL_POINTER",
                 "EVO_ERR_BAD_SHAPE", "EVO_ERR_BAD_DTYPE", "EVO_ERR_MISALIGNED", "EVO_ERR_ALIASING",
                 "EVO_ERR_UNSUPPORTED", "EVO_ERR_HIP", "EVO_ERR_NO_BIAS", "EVO_ERR_SCRATCH"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(E, name), name


def test_status_strings():
    for s in range(10):
        assert E.evo_status_string(s) and E.evo_status_string(s) != "unknown status"
    assert E.evo_status_string(99) == "unknown status"


# Fake device addresses, 1 TiB apart and 256-byte aligned; never dereferenced.
BASE = 0x7F0000000000
GIB = 1 << 40  # far enough apart for the largest tensors checked here


def addrs(n=8):
    return [BASE + i * GIB for i in range(n)]


def check(shape=(1, 2, 64, 4, 32), dtype=E.EVO_DTYPE_BF16, **over):
    q, k, v, m, p, o, l = addrs(7)
    args = dict(q=q, k=k, v=v, mask_bias=m, pair_bias=p, out=o, lse=l)
    args.update(over)
    return E.evo_attn_check(args["q"], args["k"], args["v"], args["mask_bias"], args["pair_bias"], args["out"],
                            args["lse"], shape, dtype)


def test_valid_bf16_f16_and_f32():
    assert check() == E.EVO_OK
    assert check(dtype=E.EVO_DTYPE_F16) == E.EVO_OK
    for d in (8, 16, 32, 64):
        assert check(shape=(2, 3, 17, 2, d)) == E.EVO_OK
        assert check(shape=(2, 3, 17, 2, d), dtype=E.EVO_DTYPE_F16) == E.EVO_OK
    assert check(mask_bias=None, pair_bias=None, lse=None) == E.EVO_OK
    for d in (8, 16, 32, 64):
        assert check(shape=(2, 3, 17, 2, d), dtype=E.EVO_DTYPE_F32) == E.EVO_OK
    assert check(shape=(1, 1, 1, 1, 32)) == E.EVO_OK  # L = 1 is accepted


@pytest.mark.parametrize("name", ["q", "k", "v", "out"])
def test_null_required_pointer(name):
    assert check(**{name: None}) == E.EVO_ERR_NULL_POINTER


def test_null_shape():
    q, k, v, m, p, o, l = addrs(7)
    st = E._lib.evo_attn_check(q, k, v, m, p, o, l, None, E.EVO_DTYPE_BF16)
    assert st == E.EVO_ERR_NULL_POINTER


@pytest.mark.parametrize("shape", [(0, 1, 8, 1, 32), (1, 0, 8, 1, 32), (1, 1, 0, 1, 32), (1, 1, 8, 0, 32),
                                   (1, 1, 8, 1, 0), (-1, 1, 8, 1, 32), (1 << 20, 1 << 20, 1 << 20, 1, 32),
                                   (1, 1, 1 << 31, 1 << 10, 32)])
def test_bad_shape(shape):
    assert check(shape=shape) == E.EVO_ERR_BAD_SHAPE


def test_bad_dtype():
    assert check(dtype=3) == E.EVO_ERR_BAD_DTYPE
    assert check(dtype=-1) == E.EVO_ERR_BAD_DTYPE


@pytest.mark.parametrize("name", ["q", "k", "v", "mask_bias", "pair_bias", "out", "lse"])
def test_misaligned(name):
    a = dict(zip(["q", "k", "v", "mask_bias", "pair_bias", "out", "lse"], addrs(7)))
    assert check(**{name: a[name] + 8}) == E.EVO_ERR_MISALIGNED


def test_aliasing():
    q, k, v, m, p, o, l = addrs(7)
    assert check(out=q) == E.EVO_ERR_ALIASING
    assert check(out=k + 1024) == E.EVO_ERR_ALIASING          # overlaps inside k's extent
    assert check(lse=p) == E.EVO_ERR_ALIASING
    assert check(lse=o + 256) == E.EVO_ERR_ALIASING           # lse inside out
    assert check(out=m) == E.EVO_ERR_ALIASING
    # adjacent but disjoint extents are fine: q of (1,2,64,4,32) bf16 is 65536 bytes
    assert check(out=q + 65536) == E.EVO_OK
    assert check(mask_bias=None, out=m) == E.EVO_OK            # a NULL bias has no extent


def test_inputs_may_alias_each_other():
    q, *_ = addrs(1)
    assert check(k=q, v=q) == E.EVO_OK  # self-attention on one tensor is legal: inputs are read-only


@pytest.mark.parametrize("dtype,d", [(E.EVO_DTYPE_BF16, 128), (E.EVO_DTYPE_BF16, 24), (E.EVO_DTYPE_F16, 128),
                                     (E.EVO_DTYPE_F16, 4), (E.EVO_DTYPE_F32, 12), (E.EVO_DTYPE_F32, 128)])
def test_unsupported(dtype, d):
    assert check(shape=(1, 1, 32, 1, d), dtype=dtype) == E.EVO_ERR_UNSUPPORTED


def test_bf16_offset_limits():
    """The bf16 kernel uses 32-bit byte offsets within a slice and a pair matrix."""
    assert check(shape=(1, 1, 32767, 1, 32)) == E.EVO_OK
    assert check(shape=(1, 1, 32768, 1, 32)) == E.EVO_ERR_UNSUPPORTED      # L*L*2 = 2^31
    # one head's rows of a slice must end below 2^31 bytes: (L-1)*H*D*2 + 2D
    fits = (1, 1, 1 << 14, 1 << 11, 32)       # (2^14 - 1) * 2^17 + 64 < 2^31
    assert check(shape=fits, mask_bias=None, pair_bias=None) == E.EVO_OK
    big = (1, 1, 1 << 14, 1 << 12, 32)        # (2^14 - 1) * 2^18 + 64 > 2^31
    assert check(shape=big, mask_bias=None, pair_bias=None) == E.EVO_ERR_UNSUPPORTED
    assert check(shape=big, mask_bias=None, pair_bias=None, dtype=E.EVO_DTYPE_F32) == E.EVO_OK


def test_no_pair_bias_lifts_the_pair_row_limit():
    """Without a pair bias the kernel forms no pair offset: MSA column attention over more than 32767
    sequences is accepted, with or without a mask; with a pair bias the same L is rejected."""
    assert check(shape=(1, 1, 40000, 1, 32), mask_bias=None, pair_bias=None) == E.EVO_OK
    assert check(shape=(1, 1, 40000, 1, 32), pair_bias=None) == E.EVO_OK
    assert check(shape=(1, 1, 40000, 1, 32), dtype=E.EVO_DTYPE_F16, pair_bias=None) == E.EVO_OK
    assert check(shape=(1, 1, 40000, 1, 32)) == E.EVO_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The product path has no fallback: a missing library is an ImportError."""
    import importlib.util
    import shutil
    pkg = tmp_path / "evoformer_biased_attention_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "evoformer_biased_attention_amd", "__init__.py"), pkg / "__init__.py")
    spec = importlib.util.spec_from_file_location("evo_copy", pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_single_hip_runtime_in_process():
    """Importing the binding leaves exactly one libamdhip64 mapped (torch's, when torch is installed)."""
    import subprocess
    import sys
    code = ("import evoformer_biased_attention_amd, torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(maps)); print(sorted(maps))")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, check=True)
    assert res.stdout.splitlines()[0] == "1", res.stdout


# ---------------------------------------------------------------------------
# evo_attn_bwd_check
# ---------------------------------------------------------------------------
BWD_NAMES = ["q", "k", "v", "mask_bias", "pair_bias", "out", "lse", "dout", "dq", "dk", "dv", "dmask_bias",
             "dpair_bias", "delta", "workspace"]


def bcheck(shape=(1, 2, 64, 4, 32), dtype=E.EVO_DTYPE_BF16, workspace_bytes=1 << 20, **over):
    args = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    args.update(over)
    return E.evo_attn_bwd_check(*[args[n] for n in BWD_NAMES[:-1]], shape, dtype, workspace=args["workspace"],
                                workspace_bytes=workspace_bytes)


def test_bwd_valid():
    for dt in (E.EVO_DTYPE_F32, E.EVO_DTYPE_BF16, E.EVO_DTYPE_F16):
        for d in (8, 16, 32, 64):
            assert bcheck(shape=(2, 3, 17, 2, d), dtype=dt) == E.EVO_OK
    assert bcheck(dmask_bias=None, dpair_bias=None) == E.EVO_OK          # bias gradients are optional
    assert bcheck(mask_bias=None, pair_bias=None, dmask_bias=None, dpair_bias=None) == E.EVO_OK
    assert bcheck(shape=(1, 1, 1, 1, 8)) == E.EVO_OK


@pytest.mark.parametrize("name", ["q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv", "delta"])
def test_bwd_null_required_pointer(name):
    assert bcheck(**{name: None}) == E.EVO_ERR_NULL_POINTER


def test_bwd_bias_gradient_needs_its_bias():
    assert bcheck(mask_bias=None) == E.EVO_ERR_NO_BIAS
    assert bcheck(pair_bias=None) == E.EVO_ERR_NO_BIAS
    assert bcheck(mask_bias=None, dmask_bias=None) == E.EVO_OK


@pytest.mark.parametrize("name", BWD_NAMES)
def test_bwd_misaligned(name):
    a = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    assert bcheck(**{name: a[name] + 4}) == E.EVO_ERR_MISALIGNED


def test_bwd_aliasing():
    a = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    for o in ("dq", "dk", "dv", "dmask_bias", "dpair_bias", "delta", "workspace"):
        for i in ("q", "k", "v", "mask_bias", "pair_bias", "out", "lse", "dout"):
            assert bcheck(**{o: a[i]}) == E.EVO_ERR_ALIASING, (o, i)
    assert bcheck(dk=a["dq"]) == E.EVO_ERR_ALIASING                       # outputs may not share memory
    assert bcheck(delta=a["dv"] + 512) == E.EVO_ERR_ALIASING
    assert bcheck(dq=a["q"] + 65536) == E.EVO_OK                          # adjacent, disjoint
    assert bcheck(k=a["q"], v=a["q"]) == E.EVO_OK                         # inputs may alias


def test_bwd_bad_shape_dtype_unsupported():
    assert bcheck(shape=(1, 0, 8, 1, 32)) == E.EVO_ERR_BAD_SHAPE
    assert bcheck(dtype=7) == E.EVO_ERR_BAD_DTYPE
    for d in (4, 24, 128):
        assert bcheck(shape=(1, 1, 32, 1, d)) == E.EVO_ERR_UNSUPPORTED


def test_bwd_noalloc_host_checks():
    """evo_attn_bwd_noalloc validates on the host before any HIP call: bad arguments return the backward's
    status codes, and a shape whose recommended workspace exceeds the static scratch returns EVO_ERR_SCRATCH
    (no GPU is touched on either path)."""
    a = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    names = [n for n in BWD_NAMES if n != "workspace"]

    def call(shape=(1, 2, 64, 4, 32), dtype=E.EVO_DTYPE_BF16, **over):
        args = dict(a)
        args.update(over)
        return E.evo_attn_bwd_noalloc(*[args[n] for n in names], shape, dtype, None)

    cap = E.evo_attn_bwd_noalloc_scratch_bytes()
    assert cap == 40 << 20
    # the N = L = 384 triangle-attention shape fits (7 chunks, 16.5 MB of partial sums)
    assert 0 < E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 32), E.EVO_DTYPE_BF16) <= cap
    assert call(q=None) == E.EVO_ERR_NULL_POINTER
    assert call(dq=a["q"]) == E.EVO_ERR_ALIASING
    assert call(mask_bias=None) == E.EVO_ERR_NO_BIAS
    # N = L = 768: 16 recommended chunks of 9.4 MB; the call uses the 4 that fit (GPU test in test_zz_no_alloc)
    assert E.evo_attn_bwd_workspace_size((1, 768, 768, 4, 32), E.EVO_DTYPE_BF16) > cap
    big = (1, 32, 1280, 4, 32)  # one chunk is 26.2 MB: not even two fit
    assert E.evo_attn_bwd_workspace_size(big, E.EVO_DTYPE_BF16) > cap
    assert call(shape=big) == E.EVO_ERR_SCRATCH
    assert "static buffer" in E.evo_status_string(E.EVO_ERR_SCRATCH)


def test_bwd_workspace_rules():
    a = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    assert bcheck(workspace=None, workspace_bytes=0) == E.EVO_OK            # the workspace is optional
    assert bcheck(workspace=None, workspace_bytes=1 << 40) == E.EVO_OK      # size ignored without a pointer
    assert bcheck(workspace_bytes=0) == E.EVO_OK
    assert bcheck(workspace=a["workspace"] + 8) == E.EVO_ERR_MISALIGNED
    assert bcheck(workspace=a["dq"] + 4096) == E.EVO_ERR_ALIASING           # inside dq
    assert bcheck(workspace=a["dq"] - 4096, workspace_bytes=8192) == E.EVO_ERR_ALIASING  # runs into dq
    assert bcheck(workspace_bytes=(1 << 62) + 16) == E.EVO_ERR_BAD_SHAPE


def test_bwd_workspace_size():
    """The size is a whole number of fp32 [B,H,L,ceil4(L)] partial-sum planes (rows padded to a multiple of
    4 keys), at least two, or 0."""
    plane = lambda B, H, L: B * H * L * ((L + 3) // 4 * 4) * 4
    ws = E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 32), E.EVO_DTYPE_BF16)
    assert ws > 0 and ws % plane(1, 4, 384) == 0 and ws // plane(1, 4, 384) >= 2
    assert E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 32), E.EVO_DTYPE_F16) == ws
    assert E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 32), E.EVO_DTYPE_F32) == ws   # fp32 matrix cores
    assert E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 16), E.EVO_DTYPE_F32) == ws
    assert E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 64), E.EVO_DTYPE_F32) == ws
    assert E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 8), E.EVO_DTYPE_F32) == ws
    ws_f32_odd = E.evo_attn_bwd_workspace_size((1, 384, 383, 4, 32), E.EVO_DTYPE_F32)  # staged bias rows
    assert ws_f32_odd > 0 and ws_f32_odd % plane(1, 4, 383) == 0
    assert E.evo_attn_bwd_workspace_size((1, 384, 384, 4, 64), E.EVO_DTYPE_BF16) == ws  # matrix cores for D = 64 too
    assert E.evo_attn_bwd_workspace_size((1, 8, 384, 4, 32), E.EVO_DTYPE_BF16) == 0     # N too small to split
    for L in (100, 383, 99):                                                          # any L on the matrix cores
        ws_l = E.evo_attn_bwd_workspace_size((1, 384, L, 4, 32), E.EVO_DTYPE_BF16)
        assert ws_l > 0 and ws_l % plane(1, 4, L) == 0 and ws_l // plane(1, 4, L) >= 2
    assert E.evo_attn_bwd_workspace_size((0, 384, 384, 4, 32), E.EVO_DTYPE_BF16) == 0


# ---------------------------------------------------------------------------
# evo_attn_check_strided
# ---------------------------------------------------------------------------
def scheck(layout, shape=(1, 8, 64, 4, 32), dtype=E.EVO_DTYPE_BF16, **over):
    q, k, v, m, p, o, l = addrs(7)
    args = dict(q=q, k=k, v=v, mask_bias=m, pair_bias=p, out=o, lse=l)
    args.update(over)
    return E.evo_attn_check_strided(args["q"], args["k"], args["v"], args["mask_bias"], args["pair_bias"],
                                    args["out"], args["lse"], layout, shape, dtype)


def transposed_layout(B, N, L, H, D):
    """Q/K/V/O of ending-node attention as views of X[B, L_i(=L), L_j(=N), H, D]: n = j, l = i."""
    lay = E.evo_attn_dense_layout((B, N, L, H, D))
    for name in ("q", "k", "v", "out"):
        getattr(lay, name)[:] = [L * N * H * D, H * D, N * H * D, D]
    return lay


def test_dense_layout_values():
    lay = E.evo_attn_dense_layout((2, 3, 5, 4, 8))
    assert list(lay.q) == [3 * 5 * 4 * 8, 5 * 4 * 8, 4 * 8, 8] == list(lay.out)
    assert (lay.mask_b, lay.mask_n, lay.pair_b, lay.pair_h, lay.pair_i, lay.lse_row) == (15, 5, 100, 25, 5, 5)


def test_strided_valid():
    shape = (1, 8, 64, 4, 32)
    assert scheck(E.evo_attn_dense_layout(shape)) == E.EVO_OK
    assert scheck(transposed_layout(*shape)) == E.EVO_OK
    lay = E.evo_attn_dense_layout(shape)
    lay.lse_row = 96                                # padded lse rows
    lay.pair_i = 72                                 # padded pair rows
    assert scheck(lay) == E.EVO_OK


def test_strided_rules():
    shape = (1, 8, 64, 4, 32)
    lay = E.evo_attn_dense_layout(shape)
    lay.lse_row = 63
    assert scheck(lay) == E.EVO_ERR_BAD_SHAPE       # lse rows overlap
    assert scheck(lay, lse=None) == E.EVO_OK        # no lse: its stride is ignored
    lay = E.evo_attn_dense_layout(shape)
    lay.pair_i = 60
    assert scheck(lay) == E.EVO_ERR_BAD_SHAPE       # pair rows shorter than L
    lay = E.evo_attn_dense_layout(shape)
    lay.q[2] = 132                                  # 264 bytes: not a multiple of 16
    assert scheck(lay) == E.EVO_ERR_MISALIGNED
    lay = E.evo_attn_dense_layout(shape)
    lay.k[1] = -8
    assert scheck(lay) == E.EVO_ERR_BAD_SHAPE
    lay = E.evo_attn_dense_layout(shape)
    lay.out[3] = 16                                 # heads 16 apart with D = 32: elements collide
    assert scheck(lay) == E.EVO_ERR_ALIASING
    lay = E.evo_attn_dense_layout(shape)
    lay.out[1] = 0                                  # every n on the same rows
    assert scheck(lay) == E.EVO_ERR_ALIASING
    lay = E.evo_attn_dense_layout(shape)
    lay.q[1] = 0                                    # inputs may repeat: the same Q for every n
    assert scheck(lay) == E.EVO_OK
    lay = E.evo_attn_dense_layout(shape)
    lay.mask_n = 68                                 # unaligned bias rows are accepted (staged copies)
    lay.pair_i = 66
    assert scheck(lay) == E.EVO_OK


def test_strided_aliasing_uses_the_strided_extent():
    shape = (1, 8, 64, 4, 32)
    lay = transposed_layout(*shape)
    q, *_ = addrs(1)
    assert scheck(lay, out=q + 4096) == E.EVO_ERR_ALIASING


def test_strided_32bit_row_limits():
    """bf16: rows up to L + 128 must stay below 2^32 bytes of offset."""
    shape = (1, 2, 8, 1, 32)
    lay = E.evo_attn_dense_layout(shape)
    for name in ("q", "k", "v", "out"):
        getattr(lay, name)[:] = [1 << 30, 1 << 29, 1 << 25, 32]   # row stride 2^26 bytes
    assert scheck(lay, shape=shape, mask_bias=None, pair_bias=None) == E.EVO_ERR_UNSUPPORTED
    assert scheck(lay, shape=shape, mask_bias=None, pair_bias=None, dtype=E.EVO_DTYPE_F32) == E.EVO_OK
    for name in ("q", "k", "v", "out"):
        getattr(lay, name)[:] = [1 << 24, 1 << 23, 1 << 18, 32]
    assert scheck(lay, shape=shape, mask_bias=None, pair_bias=None) == E.EVO_OK


def test_dense_entry_matches_strided_with_dense_layout():
    for shape in ((1, 2, 64, 4, 32), (2, 3, 17, 2, 16), (1, 1, 1, 1, 8)):
        for dt in (E.EVO_DTYPE_BF16, E.EVO_DTYPE_F16, E.EVO_DTYPE_F32):
            assert check(shape=shape, dtype=dt) == scheck(E.evo_attn_dense_layout(shape), shape=shape, dtype=dt)


# ---------------------------------------------------------------------------
# evo_attn_bwd_check_strided: each gradient has the layout of its tensor
# ---------------------------------------------------------------------------
def bscheck(layout, shape=(1, 8, 64, 4, 32), dtype=E.EVO_DTYPE_BF16, workspace_bytes=1 << 20, **over):
    args = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    args.update(over)
    return E.evo_attn_bwd_check_strided(*[args[n] for n in BWD_NAMES[:-1]], layout, shape, dtype,
                                        workspace=args["workspace"], workspace_bytes=workspace_bytes)


def test_bwd_strided_valid():
    shape = (1, 8, 64, 4, 32)
    for dt in (E.EVO_DTYPE_F32, E.EVO_DTYPE_BF16, E.EVO_DTYPE_F16):
        assert bscheck(E.evo_attn_dense_layout(shape), dtype=dt) == E.EVO_OK
        assert bscheck(transposed_layout(*shape), dtype=dt) == E.EVO_OK
    lay = E.evo_attn_dense_layout(shape)
    lay.lse_row, lay.pair_i = 96, 72                # padded lse / delta rows and pair rows
    assert bscheck(lay) == E.EVO_ERR_ALIASING       # the padded rows run into the next head's matrix
    lay.pair_h, lay.pair_b = 64 * 72, 4 * 64 * 72
    assert bscheck(lay) == E.EVO_OK


def test_bwd_strided_rules():
    shape = (1, 8, 64, 4, 32)
    lay = E.evo_attn_dense_layout(shape)
    lay.lse_row = 63
    assert bscheck(lay) == E.EVO_ERR_BAD_SHAPE      # lse and delta are required: their rows must not overlap
    lay = E.evo_attn_dense_layout(shape)
    lay.pair_i = 60
    assert bscheck(lay) == E.EVO_ERR_BAD_SHAPE
    lay = E.evo_attn_dense_layout(shape)
    lay.v[:] = [8 * 64 * 200, 64 * 200, 200, 36]    # heads 72 bytes apart
    assert bscheck(lay) == E.EVO_ERR_MISALIGNED
    lay = E.evo_attn_dense_layout(shape)
    lay.mask_b = -1
    assert bscheck(lay) == E.EVO_ERR_BAD_SHAPE
    # a repeated input is fine for the forward, but its gradient would collide
    lay = E.evo_attn_dense_layout(shape)
    lay.q[1] = 0
    assert scheck(lay) == E.EVO_OK and bscheck(lay) == E.EVO_ERR_ALIASING
    lay = E.evo_attn_dense_layout(shape)
    lay.mask_n = 0                                  # one mask row for every n
    assert bscheck(lay) == E.EVO_ERR_ALIASING
    assert bscheck(lay, dmask_bias=None) == E.EVO_OK
    lay = E.evo_attn_dense_layout(shape)
    lay.pair_h = 0                                  # one pair matrix for every head
    assert bscheck(lay) == E.EVO_ERR_ALIASING
    assert bscheck(lay, dpair_bias=None) == E.EVO_OK
    lay = E.evo_attn_dense_layout(shape)
    lay.out[3] = 16                                 # dout shares out's strides: heads collide
    assert bscheck(lay) == E.EVO_OK                 # out and dout are read, never written


def test_bwd_strided_aliasing_uses_the_strided_extent():
    shape = (1, 8, 64, 4, 32)
    lay = transposed_layout(*shape)
    a = dict(zip(BWD_NAMES, addrs(len(BWD_NAMES))))
    assert bscheck(lay, dq=a["q"] + 4096) == E.EVO_ERR_ALIASING
    assert bscheck(lay, dk=a["dq"] + 8192) == E.EVO_ERR_ALIASING
    lay.lse_row = 96
    lse_bytes = ((1 * 8 * 4 - 1) * 96 + 64) * 4     # first to last element of the padded lse rows
    assert bscheck(lay, delta=a["lse"] + lse_bytes - 16) == E.EVO_ERR_ALIASING
    assert bscheck(lay, delta=a["lse"] + lse_bytes) == E.EVO_OK


def test_bwd_dense_entry_matches_strided_with_dense_layout():
    for shape in ((1, 2, 64, 4, 32), (2, 3, 17, 2, 16), (1, 1, 1, 1, 8), (1, 2, 64, 2, 64)):
        for dt in (E.EVO_DTYPE_BF16, E.EVO_DTYPE_F16, E.EVO_DTYPE_F32):
            assert bcheck(shape=shape, dtype=dt) == bscheck(E.evo_attn_dense_layout(shape), shape=shape, dtype=dt)
            assert bcheck(shape=shape, dtype=dt, dq=None) == bscheck(E.evo_attn_dense_layout(shape), shape=shape,
                                                                     dtype=dt, dq=None)


# ---------------------------------------------------------------------------
# evo_trimul_check
# ---------------------------------------------------------------------------
def tcheck(shape=(1, 4, 64), direction=E.EVO_TRIMUL_OUTGOING, dtype=E.EVO_DTYPE_BF16, **over):
    a, w, x = addrs(3)
    args = dict(a=a, w=w, x=x)
    args.update(over)
    return E.evo_trimul_check(args["a"], args["w"], args["x"], shape, direction, dtype)


def test_trimul_valid():
    for d in (E.EVO_TRIMUL_OUTGOING, E.EVO_TRIMUL_INCOMING):
        for dt in (E.EVO_DTYPE_BF16, E.EVO_DTYPE_F16):
            for shape in ((1, 1, 8), (2, 3, 72), (1, 128, 384), (1, 1, 1), (2, 3, 99)):
                assert tcheck(shape=shape, direction=d, dtype=dt) == E.EVO_OK
    a, *_ = addrs(1)
    assert tcheck(w=a) == E.EVO_OK                          # the operands may be one tensor


def test_trimul_errors():
    for name in ("a", "w", "x"):
        assert tcheck(**{name: None}) == E.EVO_ERR_NULL_POINTER
    assert tcheck(shape=(1, 0, 64)) == E.EVO_ERR_BAD_SHAPE
    assert tcheck(direction=2) == E.EVO_ERR_BAD_SHAPE
    assert tcheck(dtype=5) == E.EVO_ERR_BAD_DTYPE
    a, w, x = addrs(3)
    assert tcheck(x=a) == E.EVO_ERR_ALIASING
    assert tcheck(x=w + 64 * 64 * 2 * 4 - 16) == E.EVO_ERR_ALIASING   # starts inside w's last 16 bytes
    assert tcheck(x=x + 8) == E.EVO_ERR_MISALIGNED
    assert tcheck(dtype=E.EVO_DTYPE_F32) == E.EVO_ERR_UNSUPPORTED
    assert tcheck(shape=(1, 1, 32768)) == E.EVO_ERR_UNSUPPORTED        # L * L * 2 = 2^31


# ---------------------------------------------------------------------------
# evoformer_attention: the bias list is checked on the host before any launch
# ---------------------------------------------------------------------------
def test_evoformer_attention_bias_list_checks():
    import torch
    q = torch.zeros(1, 2, 5, 3, 8, dtype=torch.bfloat16)
    mask = torch.zeros(1, 2, 1, 1, 5, dtype=torch.bfloat16)
    pair = torch.zeros(1, 1, 3, 5, 5, dtype=torch.bfloat16)
    bad = [[mask, pair, None],                                   # more than two
           [torch.zeros(1, 2, 1, 1, 4, dtype=torch.bfloat16)],   # wrong mask shape
           [None, torch.zeros(1, 3, 1, 5, 5, dtype=torch.bfloat16)],  # pair in the mask's place of heads
           [None, pair.float()],                                 # another dtype
           [torch.zeros(1, 2, 1, 1, 10, dtype=torch.bfloat16)[..., ::2]]]  # keys not contiguous
    for biases in bad:
        with pytest.raises(ValueError):
            E.evoformer_attention(q, q, q, biases)
