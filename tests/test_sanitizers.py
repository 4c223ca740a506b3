"""CPU-tier sanitizer runs (no GPU needed).

1. The C ABI's argument checks (csrc/evo_attn_api.cpp), built with g++ and
   -fsanitize=address,undefined against host-only stand-ins of the kernel
   launchers (tests/sanitize/launch_stubs.cpp), driven by a deterministic
   fuzz over adversarial sizes, strides and pointers
   (tests/sanitize/abi_fuzz.cpp).  Any signed overflow, out-of-bounds access
   or other undefined behaviour in the checks ends the run with an error.
2. The fp64 oracle (oracle/evo_ref.c) built with the same sanitizers and run
   through its forward, backward and triangle-multiplication pins in a child
   process that preloads the AddressSanitizer runtime.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "evoformer_biased_attention_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_host_checks_under_asan_ubsan(tmp_path):
    _need("g++")
    if not os.path.exists(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not available")
    exe = str(tmp_path / "abi_fuzz")
    cmd = ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}", f"-I{ROOT}/include",
           f"-I{CSRC}", "-o", exe, os.path.join(CSRC, "evo_attn_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_fuzz.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    for seed in (1, 2):
        r = subprocess.run([exe, "400000", str(seed)], capture_output=True, text=True, timeout=300)
        print(r.stdout.strip())
        assert r.returncode == 0, r.stdout + r.stderr
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
        assert " 0 failures" in r.stdout


PIN_SCRIPT = textwrap.dedent("""
    import sys
    sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
    import oracle, oracle_pins, oracle_bwd_pins, oracle_trimul_pins
    lib = oracle.load_library({lib!r})
    def ref(q, k, v, mask, pair, dtype):
        return oracle.fwd(q, k, v, mask, pair, dtype=dtype, nthreads=2, lib=lib)
    def gref(q, k, v, mask, pair, dout, dtype):
        return oracle.bwd(q, k, v, mask, pair, dout, dtype=dtype, nthreads=2, lib=lib)
    def tref(a, w, dtype, direction):
        return oracle.trimul(a, w, dtype=dtype, direction=direction, nthreads=2, lib=lib)
    n = 0
    for pin in oracle_pins.ALL_PINS:
        if "torch" in pin.__name__:  # needs PyTorch, which is not loaded under the sanitizer runtime
            continue
        pin(ref); n += 1
    for pin in oracle_bwd_pins.ALL_BWD_PINS:
        if "torch" in pin.__name__:
            continue
        pin(gref); n += 1
    for pin in oracle_trimul_pins.ALL_TRIMUL_PINS:
        if "torch" in pin.__name__:
            continue
        pin(tref); n += 1
    print("pins passed under the sanitizers:", n)
""")


def test_oracle_pins_under_asan_ubsan(tmp_path):
    _need("gcc")
    import oracle
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("AddressSanitizer runtime not found")
    lib = str(tmp_path / "libevoref_san.so")
    src = os.path.join(ROOT, "oracle", "evo_ref.c")
    subprocess.run(["gcc", *SAN, *[f for f in oracle.GCC_FLAGS if f != "-O2"], "-o", lib, src, "-lm"], check=True,
                   capture_output=True, text=True)
    script = PIN_SCRIPT.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env, timeout=900)
    print(r.stdout.strip())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr, r.stderr[-3000:]
    assert "pins passed under the sanitizers" in r.stdout
