"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle is rebuilt with both (abort on the first report) and its pin tests
run in a child process that loads that build."""
import os
import subprocess
import sys

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_formats.py", "test_oracle_quant.py", "test_oracle_gemm_route.py",
        "test_oracle_rac_grouped.py", "test_oracle_qdq.py", "test_oracle_combine.py",
        "test_oracle_fp8.py", "test_oracle_silu_softmax.py"]


def test_oracle_pins_under_asan_and_ubsan():
    path = O.build_sanitized()
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    assert os.path.isabs(asan), "gcc has no AddressSanitizer runtime"
    env = dict(os.environ, LD_PRELOAD=asan, NVFP4RAC_ORACLE_LIB=path,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in PINS]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "error" not in r.stdout.splitlines()[-1], tail
