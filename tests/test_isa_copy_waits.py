"""Static check of the compiled kernels (no GPU needed): every global -> LDS copy
is waited for before the next workgroup barrier.

The attention, backward and triangle-multiplication kernels issue their
global -> LDS copies (`buffer_load_dwordx4 ... offen lds`) as inline assembly
that the compiler does not track, so that the LDS reads of the other buffer
need not wait for them.  Their correctness then rests on an explicit
`s_waitcnt vmcnt(0)` between each copy and the barrier that publishes the
copied data.  This test compiles each kernel source to gfx950 assembly with the
library's own flags and walks back from every `s_barrier` to the previous one:
a copy found there with no full vector-memory wait after it fails the test.
"""
import importlib.util
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "evoformer_biased_attention_amd", "csrc")
SOURCES = ["evo_attn_bf16.hip", "evo_attn_bwd_mfma.hip", "evo_trimul.hip", "evo_attn_f32.hip", "evo_attn_bwd_f32.hip"]

pytestmark = pytest.mark.slow


def _build_flags():
    spec = importlib.util.spec_from_file_location("evo_hip_build", os.path.join(ROOT, "evoformer_biased_attention_amd",
                                                                                "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.hipcc(), [f for f in mod.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]


def _is_full_vm_wait(line):
    t = line.strip()
    return t.startswith("s_waitcnt") and ("vmcnt(0)" in t or t in ("s_waitcnt 0", "s_waitcnt 0x0"))


def unwaited_copies(asm_lines):
    """(number of barriers, number of copies, barriers reached with a copy issued after the last full
    vector-memory wait), scanning back from each barrier to the previous one."""
    barriers = copies = bad = 0
    for i, line in enumerate(asm_lines):
        t = line.strip()
        if "offen lds" in t:
            copies += 1
        if t != "s_barrier":
            continue
        barriers += 1
        j = i - 1
        while j >= 0:
            u = asm_lines[j].strip()
            if u == "s_barrier" or u.endswith(":") and not u.startswith(".") and "LBB" not in u:
                break                      # the previous barrier, or the start of the function
            if _is_full_vm_wait(u):
                break                      # everything issued before this point has landed
            if "offen lds" in u:
                bad += 1
                break
            j -= 1
    return barriers, copies, bad


def test_scan_catches_an_unwaited_copy():
    """The scan itself: a copy between the last wait and a barrier is reported, a waited one is not."""
    ok = ["s_barrier", "buffer_load_dwordx4 v1, s[0:3], 0 offen lds", "v_add_u32 v2, v3, v4",
          "s_waitcnt vmcnt(0) lgkmcnt(0)", "s_barrier"]
    assert unwaited_copies(ok) == (2, 1, 0)
    bad = ["s_barrier", "s_waitcnt vmcnt(0)", "buffer_load_dwordx4 v1, s[0:3], 0 offen lds", "s_barrier"]
    assert unwaited_copies(bad) == (2, 1, 1)
    partial = ["buffer_load_dwordx4 v1, s[0:3], 0 offen lds", "s_waitcnt vmcnt(6) lgkmcnt(0)", "s_barrier"]
    assert unwaited_copies(partial)[2] == 1


def test_every_lds_copy_is_waited_for_before_a_barrier(tmp_path):
    hipcc, flags = _build_flags()
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")

    def compile_one(src):
        out = str(tmp_path / (os.path.splitext(src)[0] + ".s"))
        res = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, src)],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return src, f.read().splitlines()

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    total_copies = 0
    for src, lines in results:
        barriers, copies, bad = unwaited_copies(lines)
        print(f"{src}: {barriers} barriers, {copies} global -> LDS copies, {bad} not waited for", flush=True)
        assert barriers > 0
        assert bad == 0, f"{src}: {bad} barrier(s) reached with a global -> LDS copy still in flight"
        total_copies += copies
    assert total_copies > 0, "no global -> LDS copies found: the scan would be vacuous"
