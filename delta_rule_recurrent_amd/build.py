"""Build the gdnrt HIP library in-tree for gfx950 (``libgdnrt.so`` next to this file).

    python -m delta_rule_recurrent_amd.build

hipcc cross-compiles for gfx950 without a GPU. Packed fp32 VALU instructions are
disabled for every device compilation; MFMA instructions use their VGPR form.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgdnrt.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the gdnrt library)")


def sources():
    src = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    src += sorted(glob.glob(os.path.join(HERE, "csrc", "*.cpp")))
    return src


def _flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in ordinary VGPRs: kernels that also work on the
            # accumulators with VALU code then hold one copy instead of an AGPR copy
            # plus a VGPR copy
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return r.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source into libgdnrt.so (always recompiles): one object
    per source, compiled in parallel, then one shared-library link."""
    from concurrent.futures import ThreadPoolExecutor
    srcs = sources()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[hipcc()] + _flags() + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{err}")
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
