"""The C ABI's host code under AddressSanitizer: the argument checks of
test_abi.py run in a child process against a build of the library whose host code
is instrumented (device code unchanged), with the clang ASan runtime preloaded.
Any heap or stack error in argument validation, workspace sizing or error
reporting aborts the child with an AddressSanitizer report.  No GPU is used."""
import os
import subprocess
import sys

from sparse_attention_diffusion_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_are_clean_under_address_sanitizer():
    lib = build.build_asan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["MCS_ABI_TEST_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
