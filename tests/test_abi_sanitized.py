"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with host-side
instrumentation (global_layers_amd/build.py, sanitize=True; device code as
usual) into a scratch copy of the package, and tests/test_abi_cpu.py runs
against it in a child process that preloads the sanitizer runtime, with any
report fatal. CPU only: no call in that file reaches the device."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if rt is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc or sanitizer runtime in this environment")
    sys.path.insert(0, ROOT)
    from global_layers_amd import build as b
    pkg = tmp_path / "global_layers_amd"
    pkg.mkdir()
    so = b.build(verbose=False, out_dir=str(pkg), sanitize=True)
    # the instrumentation is really in: the sanitizer entry points are undefined
    # in the library and come from the preloaded runtime
    nm = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert " U __asan_" in nm and " U __ubsan_" in nm
    for f in ("lib.py", "__init__.py"):
        shutil.copy(os.path.join(ROOT, "global_layers_amd", f), pkg / f)
    for d in ("tests", "oracle", "workloads", "include"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q",
                        "-p", "no:cacheprovider"], cwd=tmp_path, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "failed" not in r.stdout
