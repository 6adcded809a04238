"""The C ABI's host code under AddressSanitizer (no GPU): the host-validation
tests of test_abi.py run in a child process against libgqe_asan.so (host code
built with -fsanitize=address; device code unchanged) with the compiler's ASan
runtime preloaded, so that every host buffer (configs, per-group k arrays,
layouts) has redzones and any out-of-bounds or use-after-free access in the
library's argument checks, layout arithmetic or launch set-up aborts the
child."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_validation_under_asan():
    sys.path.insert(0, ROOT)
    from sparse_query_moe_amd import build
    if not os.path.exists(build.ASAN_LIB):
        build.build(variant="asan")
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["GQE_TEST_LIBRARY"] = build.ASAN_LIB
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), "-m", "not gpu"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
