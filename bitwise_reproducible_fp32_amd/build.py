"""Builds libmlb.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that matter for the bits:
  -ffp-contract=off                   no implicit mul+add fusion (HIP defaults to fusing)
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division and square root
  no -ffast-math, no -fgpu-flush-denormals-to-zero   IEEE denormals
  -target-feature -packed-fp32-ops    no packed FP32 VALU instructions
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmlb.so")
SOURCES = ["mlb_api.hip", "mlb_gemm.hip", "mlb_ops.hip", "mlb_attn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l]
    return r.returncode, msgs


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compiles every source in parallel, then links libmlb.so (always rebuilds)."""
    with tempfile.TemporaryDirectory() as td:
        objs = [os.path.join(td, s + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, *(extra or []), "-c", "-o", o, os.path.join(CSRC, s)]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, msgs), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
            if verbose and msgs:
                print("\n".join(msgs), file=sys.stderr)
        rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *objs])
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
