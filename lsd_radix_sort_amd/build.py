"""Build the gfx950 shared library in-tree with hipcc.

    python -m lsd_radix_sort_amd.build [-v] [-j N] [-DNAME=VALUE ...] [--out PATH]

Each csrc/*.hip translation unit (the driver and C ABI, and one unit per key
kind holding that kind's kernels) compiles to an object in parallel; the
objects link into lsd_radix_sort_amd/liblsd_radix_sort.so.  Always recompiles.

-D options set the compile-time tunables of csrc/lrs_kernels.h (tile shape,
look-back window, XCD chunk, ...) in every unit; with --out the library is
written elsewhere, so a variant can be timed beside the default with
``bench.py --lib PATH`` (the A/B measurements of the design notes are made
this way).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblsd_radix_sort.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None, extra_flags: list[str] | None = None,
          out: str = LIB) -> str:
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    flags = FLAGS + list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="lrs_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s)[:-4] + ".o") for s in srcs]

        def compile_one(src_obj):
            src, obj = src_obj
            cmd = [HIPCC, *flags, "-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            # hipcc's host pass warns that it does not know the packed-fp32 feature
            noise = "is not a recognized feature for this target"
            msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
            if r.returncode != 0:
                raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{msg}")
            if msg.strip() and verbose:
                print(msg, flush=True)
            return obj

        with ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(compile_one, zip(srcs, objs)))
        tmp_lib = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    argv = sys.argv[1:]
    j = None
    out = LIB
    defines = [a for a in argv if a.startswith("-D")]
    if "-j" in argv:
        j = int(argv[argv.index("-j") + 1])
    if "--out" in argv:
        out = os.path.abspath(argv[argv.index("--out") + 1])
    print(build(verbose="-v" in argv, jobs=j, extra_flags=defines, out=out))
