"""Build the gfx950 HIP library in-tree with hipcc.

``python -m exact_attention_10_amd.build`` compiles ``csrc/*.hip`` into
``libfa_mi355x.so`` next to this file. ``--save-temps DIR`` also keeps the
device assembly for inspection.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libfa_mi355x.so")
SOURCES = [os.path.join(CSRC, "fa_api.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "fa_kernel.hpp"), os.path.join(CSRC, "fa_kernel_pingpong.hpp"),
                     os.path.join(CSRC, "fa_kernel_interleaved.hpp"),
                     os.path.join(ROOT, "include", "fa.h")]

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for device code (a host-pass warning about
# the unknown feature is expected and harmless).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(output: str = LIBRARY, save_temps: str | None = None, verbose: bool = False) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", output, *SOURCES]
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, f"-save-temps={save_temps}" if False else "-save-temps")
    if verbose:
        print(" ".join(cmd), flush=True)
    cwd = save_temps if save_temps else None
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
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
