"""Build and run the gfx950 microbenchmarks (micro.hip) and summarise them.

    python micro/run_micro.py build            # hipcc -> micro/micro (on any machine)
    python micro/run_micro.py run [--out F]    # on a GPU: run every test, JSON lines to stdout (and F)

The results give the sustained rates that the roofline figures of bench.py
are read against next to the published peaks: bf16 matrix-core FLOP/s,
v_exp_f32 and v_fma_f32 issue rates, their overlap, LDS read and
global->LDS copy bandwidth per CU, and HBM copy bandwidth.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "micro.hip")
BIN = os.path.join(HERE, "micro")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = BIN + ".tmp"
    res = subprocess.run([os.path.join(rocm, "bin", "hipcc"), *FLAGS, "-o", tmp, SRC], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, BIN)
    return BIN


def run(tests=(), out=None) -> list:
    if not os.path.exists(BIN):
        raise FileNotFoundError(f"{BIN} is not built; run `python micro/run_micro.py build` first")
    res = subprocess.run([BIN, *tests], capture_output=True, text=True, timeout=300)
    sys.stderr.write(res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"micro exited with {res.returncode}")
    rows = [json.loads(ln) for ln in res.stdout.splitlines() if ln.startswith("{")]
    text = "\n".join(json.dumps(r) for r in rows) + "\n"
    sys.stdout.write(text)
    if out:
        with open(out, "w") as f:
            f.write(text)
    return rows


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else "run"
    if cmd == "build":
        print(build())
    elif cmd == "run":
        args = sys.argv[2:]
        out = None
        if "--out" in args:
            i = args.index("--out")
            out = args[i + 1]
            del args[i:i + 2]
        run(args, out)
    else:
        raise SystemExit(__doc__)
