"""Host AddressSanitizer + UndefinedBehaviorSanitizer build of the library,
for CPU-only runs of the C ABI's host side: argument checks, workspace
sizing and carving, launch-configuration arithmetic, the error paths.

Every sanitizer flag reaches the host compilation only (each one follows
-Xarch_host), so the gfx950 code objects are those of the normal build;
the result is meant for processes without a GPU, which exercise the host
code up to the point of a launch.  The library links the sanitizer
runtime dynamically, so a Python process that loads it must start with
that runtime preloaded (``runtime()`` gives its path; LD_PRELOAD), with
leak detection off (the interpreter is not instrumented).
"""
from __future__ import annotations

import os
import subprocess
import tempfile

from . import _build

LIB_PATH = os.path.join(_build.LIB_DIR, "libflint_moe_hostsan.so")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan"]


def runtime() -> str:
    """Path of the shared ASan runtime of the toolchain that builds the library."""
    out = subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the toolchain's shared ASan runtime was not found")
    return path


def build() -> str:
    os.makedirs(_build.LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="flint_hostsan_") as td:
        jobs, objs = [], []
        for s in _build.SOURCES:
            obj = os.path.join(td, os.path.splitext(s)[0] + ".o")
            cmd = ["hipcc"] + _build.compile_flags() + HOST_SAN + ["-O1", "-c", os.path.join(_build.CSRC, s),
                                                                   "-o", obj]
            jobs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for cmd, p in jobs:
            out, err = p.communicate()
            _build._check(subprocess.CompletedProcess(cmd, p.returncode, out, err), cmd)
        link = ["hipcc", f"--offload-arch={_build.ARCH}", "-shared", "-fPIC"] + HOST_SAN + objs + ["-o", tmp]
        _build._check(subprocess.run(link, capture_output=True, text=True), link)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
