"""Build the gfx950 HIP library in-tree with hipcc.

``python -m exact_attention_10_amd.build`` compiles ``csrc/*.hip`` into
``libfa_mi355x.so`` next to this file: each translation unit (the host API and
one file per kernel family) is compiled to an object in parallel, then the
objects are linked. ``--save-temps DIR`` also keeps the device assembly for
inspection.
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libfa_mi355x.so")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
DEPENDS = SOURCES + sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [
    os.path.join(ROOT, "include", "fa.h")]

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for device code (a host-pass warning about
# the unknown feature is expected and harmless).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-file device flags. The backward kernels keep every MFMA accumulator in
# the VGPR form: with the default choice the compiler places the dK/dV (or dQ)
# accumulators in AGPRs and copies them to and from VGPRs on every tile (about
# five copies per MFMA), which the VGPR form avoids.
FILE_FLAGS = {
    "fa_inst_bwd.hip": ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, cwd=None):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for a CPU-only
# check build of the library: each option reaches the host compilation only
# (device code is never instrumented). The resulting library needs the clang
# ASan runtime preloaded into the process that loads it.
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def build(output: str = LIBRARY, save_temps: str | None = None, verbose: bool = False,
          jobs: int | None = None, host_sanitize: bool = False) -> str:
    """Compile every translation unit in parallel and link the shared library.
    The library is written to a temporary name and renamed into place, so a
    failed build never leaves a partial file behind. host_sanitize builds the
    host code with ASan and UBSan (a check build, never the product)."""
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    objdir = tempfile.mkdtemp(prefix="fa_build_")
    base = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    if host_sanitize:
        base += HOST_SANITIZE_FLAGS
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        base.insert(1, "-save-temps")
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append(base + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", "-o", obj, src])
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, save_temps) for c in cmds]:
            f.result()
    tmp = output + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if host_sanitize:
        link[1:1] = HOST_SANITIZE_FLAGS
    _run(link)
    os.replace(tmp, output)
    for o in objs:
        os.unlink(o)
    os.rmdir(objdir)
    return output


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None, help="keep intermediate files in this directory")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    out = build(save_temps=a.save_temps and os.path.abspath(a.save_temps), verbose=a.verbose)
    print(out)


if __name__ == "__main__":
    main()
