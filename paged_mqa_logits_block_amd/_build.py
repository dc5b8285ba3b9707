"""Build libqsaidx.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqsaidx.so")
SOURCES = ["api.hip", "logits.hip", "logits_decode.hip", "logits_looped.hip", "logits_mtp.hip",
           "logits_prefill.hip", "topk.hip", "expand.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the head reduction reads every accumulator with
    # VALU ops, which would otherwise each need an AGPR-to-VGPR move first
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(out: str = LIB, extra=None, verbose: bool = False) -> str:
    """Compile every source to an object in a temporary folder (in parallel),
    link the shared library next to `out` and move it into place."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    flags = [*FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC]
    compile_flags = [f for f in flags if f != "-shared"]
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory(prefix="qsaidx_build_") as objdir:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *compile_flags, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
