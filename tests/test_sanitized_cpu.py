"""CPU-only check builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The fp64 oracles (forward and backward) are rebuilt with gcc and
  ``-fsanitize=address,undefined``, and exercised in a child process with the
  ASan runtime preloaded: full, row-sampled, cross-attention, fully masked and
  backward cases must run clean and give bitwise the results of the normal
  build. A copy of the forward source with a planted one-past-the-end read must
  be reported, which shows that the check build does catch such mistakes.
* The HIP library is rebuilt with host-side ASan and UBSan (device code is not
  instrumented) and the C-ABI tests (argument validation of every entry point,
  no GPU needed) run against it in a child process.

Both child processes run with leak detection off: the Python interpreter
itself keeps allocations alive until exit.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GCC_SAN = ["-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]


def _gcc_asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_oracle(src, out):
    subprocess.run(["gcc", *GCC_SAN, "-o", out, src, "-lm"], check=True)
    return out


ORACLE_SCRIPT = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import fa_inputs, oracle
fwd, bwd = {fwd!r}, {bwd!r}
def same(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))
for causal in (False, True):
    q, k, v = (fa_inputs.to_f32(x, "bf16") for x in fa_inputs.draw_qkv(2, 3, 131, 64, "bf16", 5))
    assert same(oracle.attention(q, k, v, 0.125, causal, lib_path=fwd),
                oracle.attention(q, k, v, 0.125, causal))
    assert same(oracle.attention(q, k, v, 0.125, causal, n_kv=0, lib_path=fwd),
                oracle.attention(q, k, v, 0.125, causal, n_kv=0))
    rows = np.array([[0, 0], [5, 130], [3, 64]])
    assert same(oracle.attention_rows(q, k, v, 0.125, causal, rows, n_kv=77, lib_path=fwd),
                oracle.attention_rows(q, k, v, 0.125, causal, rows, n_kv=77))
    q2, k2, v2 = (fa_inputs.to_f32(x, "fp16")
                  for x in fa_inputs.draw_qkv_cross(1, 2, 37, 90, 128, "fp16", 6))
    for align in ("top-left", "bottom-right"):
        assert same(oracle.attention(q2, k2, v2, 0.09, causal, causal_align=align, lib_path=fwd),
                    oracle.attention(q2, k2, v2, 0.09, causal, causal_align=align))
        assert same(oracle.attention_bwd(q2, k2, v2, q2, 0.09, causal, align, lib_path=bwd),
                    oracle.attention_bwd(q2, k2, v2, q2, 0.09, causal, align))
        assert same(oracle.attention_bwd_sampled(q2[0, 1], k2[0, 1], v2[0, 1], q2[0, 1], 0.09,
                                                 causal, [0, 36], [0, 89], align, lib_path=bwd),
                    oracle.attention_bwd_sampled(q2[0, 1], k2[0, 1], v2[0, 1], q2[0, 1], 0.09,
                                                 causal, [0, 36], [0, 89], align))
try:
    oracle.attention_rows(q, k, v, 0.125, False, np.array([[6, 0]]), lib_path=fwd)
    raise SystemExit("out-of-range row accepted")
except ValueError:
    pass
print("SANITIZED_ORACLE_OK", flush=True)
"""


def _run_child(code_or_args, preload, env_extra=None, timeout=600):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    env.update(env_extra or {})
    args = [sys.executable, "-c", code_or_args] if isinstance(code_or_args, str) else code_or_args
    return subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


@pytest.fixture(scope="module")
def gcc_asan():
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return rt


def test_oracles_clean_under_asan_ubsan(gcc_asan, tmp_path):
    fwd = _build_oracle(os.path.join(ROOT, "oracle", "attention_ref.c"), str(tmp_path / "f.so"))
    bwd = _build_oracle(os.path.join(ROOT, "oracle", "attention_bwd_ref.c"), str(tmp_path / "b.so"))
    res = _run_child(ORACLE_SCRIPT.format(root=ROOT, fwd=fwd, bwd=bwd), gcc_asan)
    assert res.returncode == 0 and "SANITIZED_ORACLE_OK" in res.stdout, res.stdout + res.stderr
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr


def test_planted_overrun_is_reported(gcc_asan, tmp_path):
    """The same harness must fail when the oracle reads one score past the
    visible keys (a copy of the source with the max loop running to n_vis)."""
    src = open(os.path.join(ROOT, "oracle", "attention_ref.c")).read()
    needle = "for (int64_t j = 1; j < n_vis; ++j)\n                if (s[j] > m) m = s[j];"
    assert needle in src
    bad = src.replace(needle, "for (int64_t j = 1; j <= Nk; ++j)\n                if (s[j] > m) m = s[j];")
    path = tmp_path / "bad.c"
    path.write_text(bad)
    lib = _build_oracle(str(path), str(tmp_path / "bad.so"))
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "import fa_inputs, oracle\n"
            "q, k, v = (fa_inputs.to_f32(x, 'bf16') for x in fa_inputs.draw_qkv(1, 1, 40, 64, 'bf16', 1))\n"
            f"oracle.attention(q, k, v, 0.125, False, lib_path={lib!r})\n")
    res = _run_child(code, gcc_asan)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-2000:]


def test_abi_validation_under_host_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from exact_attention_10_amd import build as fa_build
    lib = fa_build.build(output=str(tmp_path / "libfa_mi355x_hostsan.so"), host_sanitize=True)
    check = ("import os, sys\n"
             f"sys.path.insert(0, {ROOT!r})\n"
             "import exact_attention_10_amd as fa\n"
             "fa.load_library()\n"
             "maps = open('/proc/self/maps').read()\n"
             f"assert {lib!r} in maps and 'libclang_rt.asan' in maps\n"
             "print('SANITIZED_LIBRARY_LOADED', flush=True)\n")
    res = _run_child(check, rt, {"FA_MI355X_LIBRARY": lib})
    assert res.returncode == 0 and "SANITIZED_LIBRARY_LOADED" in res.stdout, res.stderr[-3000:]
    res = _run_child([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                      "-q", "-x", "-p", "no:cacheprovider"], rt, {"FA_MI355X_LIBRARY": lib})
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
