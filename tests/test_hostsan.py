"""The library's host code (argument checks, descriptors, error reporting)
under AddressSanitizer and UndefinedBehaviorSanitizer: the ABI tests run
against a sanitized build in a copy of the package, with the ASan runtime
preloaded.  No GPU is used: every call returns before any launch."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    from certified_kv_cache_amd import build as B
    try:
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    tree = tmp_path / "tree"
    pkg = tree / "certified_kv_cache_amd"
    pkg.mkdir(parents=True)
    for f in os.listdir(os.path.join(ROOT, "certified_kv_cache_amd")):
        if f.endswith(".py"):
            shutil.copy(os.path.join(ROOT, "certified_kv_cache_amd", f), pkg / f)
    shutil.copytree(os.path.join(ROOT, "include"), tree / "include")
    (tree / "tests").mkdir()
    for f in ("__init__.py", "conftest.py", "test_abi.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tree / "tests" / f)
    lib = B.build_sanitized(str(pkg / "libwitcert.so"))
    if shutil.which("nm"):                     # the host code is instrumented
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = {**os.environ, "LD_PRELOAD": rt, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-p", "no:cacheprovider"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
