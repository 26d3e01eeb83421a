"""The host-side ABI checks under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

libmoe.so is built a second time with the host half of every source instrumented (device
code is built as usual, sanitizers apply to host code only), into a scratch copy of the
package next to a copy of include/ and tests/test_abi_host.py.  Those ABI tests then run in a
child Python with the clang sanitizer runtime preloaded: argument validation, error strings
and every exported entry point's rejection paths execute under both sanitizers, and any
report ends the child with a non-zero status.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_routed_expert_amd")
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_checks_pass_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if rt is None or not os.path.exists(hipcc):
        pytest.skip("clang sanitizer runtime or hipcc not available")
    sys.path.insert(0, PKG)
    try:
        import build as B
    finally:
        sys.path.remove(PKG)
    root = tmp_path / "san"
    pkg = root / "mxfp4_routed_expert_amd"
    pkg.mkdir(parents=True)
    for f in glob.glob(os.path.join(PKG, "*.py")):
        shutil.copy(f, pkg)
    shutil.copytree(os.path.join(ROOT, "include"), root / "include")
    (root / "tests").mkdir()
    for f in ("test_abi_host.py", "conftest.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), root / "tests")
    lib = B.build(jobs=min(8, os.cpu_count() or 1), extra_flags=SAN_FLAGS, out=str(pkg / "libmoe.so"),
                  build_dir=os.path.join(PKG, "csrc", "_build_san"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the library is not instrumented"

    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_host.py"],
                       cwd=str(root), env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
