"""CPU runs of the oracle and of the library's host-side argument checks under
AddressSanitizer and UndefinedBehaviorSanitizer (no GPU: the sanitizers watch
host code only).

* oracle.c is built with gcc -fsanitize=address,undefined (any report aborts)
  and the oracle's pin tests run against that build, in a child process with
  gcc's libasan preloaded (the Python interpreter is not instrumented).
* The library is built with its host code under the same sanitizers (GPU code
  as usual) and the C-ABI / binding checks -- argument validation, status
  codes, workspace sizing, every one failing before a launch -- run against it
  with clang's ASan runtime preloaded.
Both builds are cached under _build/san and rebuilt when a source changes.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "_build", "san")
sys.path.insert(0, ROOT)


def _run(tests, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter's own allocations are not ours
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]


def _gcc_asan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's libasan is not installed")
    return p


def _clang_asan():
    c = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not c:
        pytest.skip("clang's ASan runtime is not installed")
    return c[-1]


def test_oracle_under_asan_ubsan():
    import oracle
    os.makedirs(SAN, exist_ok=True)
    so = os.path.join(SAN, "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "oracle.c")
    if not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        oracle.build_sanitized(so)
    out = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_" in out and "__ubsan_" in out  # the build is instrumented
    _run(["tests/test_oracle_pins.py"], {"ENTMAXKV_ORACLE_LIB": so, "LD_PRELOAD": _gcc_asan()})


def test_abi_checks_under_asan_ubsan():
    from sparse_decode_attention_page_amd import build
    so = build.build_host_sanitized(os.path.join(SAN, "libentmaxkv_san.so"))
    out = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_" in out and "__ubsan_" in out
    _run(["tests/test_abi.py", "tests/test_binding_checks.py"], {"ENTMAXKV_LIB": so, "LD_PRELOAD": _clang_asan()})
