"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only; GPU code is never built with a sanitizer).

* The oracle (oracle/oracle.c) is built with gcc -fsanitize=address,undefined
  and run in a child process on a fixed problem set (the brute-force pins'
  instance shapes, random problems of every table kind and mode with -inf
  and integer logits, the full-vocabulary mode, the table update and the
  verification length); every output must equal the plain build's.
* libdt.so's host code (api.hip: argument validation, launch and workspace
  planning) is rebuilt with the host half instrumented and linked with the
  library's other objects, and the ABI tests run against it in a child
  process.

Any sanitizer report aborts the child, which fails the test.
"""

import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "sanitize_run.py")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _preload(runtime: str) -> dict:
    env = dict(os.environ, **SAN_ENV)
    env["LD_PRELOAD"] = " ".join(x for x in (runtime, os.environ.get("LD_PRELOAD", "")) if x)
    env["PYTHONPATH"] = os.pathsep.join([ROOT, HERE])
    return env


def _child(args, env, timeout=600):
    r = subprocess.run([sys.executable, DRIVER, *args], env=env, capture_output=True, text=True, timeout=timeout)
    reports = [ln for ln in r.stderr.splitlines() if "runtime error" in ln or "Sanitizer" in ln]
    assert r.returncode == 0, (f"{args[0]} run failed ({r.returncode}):\n" + "\n".join(reports[:20]) +
                               f"\n{r.stdout[-3000:]}\n{r.stderr[:3000]}")
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    return r


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    src = os.path.join(ROOT, "oracle", "oracle.c")
    flags = ["-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]
    san = tmp_path / "liboracle_san.so"
    plain = tmp_path / "liboracle_plain.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", *flags, "-o", str(san), src, "-lm"])
    subprocess.check_call(["gcc", "-O2", *flags, "-o", str(plain), src, "-lm"])
    runtime = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    _child(["oracle", str(san), str(tmp_path / "san.npz")], _preload(runtime))
    _child(["oracle", str(plain), str(tmp_path / "plain.npz")], dict(os.environ, PYTHONPATH=os.pathsep.join([ROOT, HERE])))
    a, b = np.load(tmp_path / "san.npz"), np.load(tmp_path / "plain.npz")
    assert sorted(a.files) == sorted(b.files) and len(a.files) > 100
    for key in a.files:
        assert np.array_equal(a[key], b[key], equal_nan=True), key


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    from draft_tree_construction_dt_amd import build as B
    objdir = os.path.join(B.HERE, "_build")
    others = [os.path.join(objdir, s.replace(".hip", ".o")) for s in B.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in others):
        B.build_library()
    # the sanitizer flags apply to the host half only (each behind -Xarch_host)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = tmp_path / "api_san.o"
    r = subprocess.run([B.HIPCC, *B.FLAGS, "-g", *host_san, "-c", os.path.join(B.CSRC, "api.hip"),
                        "-o", str(api_obj)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lib = tmp_path / "libdt_san.so"
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-o", str(lib), str(api_obj), *others], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    runtime = subprocess.check_output([shutil.which("clang") or "/opt/rocm/llvm/bin/clang",
                                       "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    if not os.path.isabs(runtime):
        runtime = subprocess.check_output(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                                          text=True).strip()
    r = _child(["abi", str(lib)], _preload(runtime))
    assert " passed" in r.stdout, r.stdout[-2000:]
