"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer: the library
is rebuilt with host-only sanitizers (device code untouched) and the CPU ABI tests, which
drive every argument check and error path without a GPU, run against it in a child
process with the sanitizer runtime preloaded.  Any report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from kronecker_factored_structured_amd import build as B
    rt = B.sanitizer_runtime()
    if not rt:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = B.build(host_sanitize=True, out=str(tmp_path / "libkron_san.so"))
    env = dict(os.environ)
    env["KRON_LIB_PATH"] = lib
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    probe = subprocess.run([sys.executable, "-c", "import kronecker_factored_structured_amd._lib as L; "
                            "L.lib(); print(L.LIB_PATH)"], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    with open(lib, "rb") as fh:   # (the build is instrumented)
        assert b"__asan_init" in fh.read()
