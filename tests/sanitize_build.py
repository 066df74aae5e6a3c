"""Host-sanitized build of the gdnrt library for the CPU validation tests.

Compiles every HIP source with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side only (each sanitizer flag behind -Xarch_host; the device code is compiled
as usual and never runs here) into _build/asan/libgdnrt_asan.so. The sanitizer
runtime is not linked in: a process that loads the library preloads it
(asan_runtime()), which also carries the UBSan handlers."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT, "libgdnrt_asan.so")

HOST_SANITIZE = []
for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer"):
    HOST_SANITIZE += ["-Xarch_host", f]


def asan_runtime() -> str | None:
    """The clang ASan runtime shipped with ROCm's compiler, or None."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build() -> str:
    from delta_rule_recurrent_amd import build as b
    os.makedirs(OUT, exist_ok=True)
    srcs = b.sources()
    objs = [os.path.join(OUT, os.path.basename(s) + ".o") for s in srcs]
    # -O1 -g: clearer reports; the host validation is what runs
    flags = [f for f in b._flags() if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE
    cmds = [[b.hipcc()] + flags + ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda c: subprocess.run(c, cwd=ROOT, capture_output=True, text=True), cmds))
    for r, s in zip(res, srcs):
        if r.returncode:
            raise RuntimeError(f"sanitized compile of {os.path.basename(s)} failed:\n{r.stderr[-3000:]}")
    r = subprocess.run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", LIB] + objs,
                       cwd=ROOT, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr[-3000:]}")
    return LIB
