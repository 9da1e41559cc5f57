"""AddressSanitizer + UndefinedBehaviorSanitizer build of the host code (CPU only).

tests/sanitize/build.sh compiles the libwqmm runtime's host half and the CPU oracle
instrumented (the kernels' device code as usual) into one test program; running it
exercises argument validation of every entry point, the no-device startup error, the
planner over a spread of shapes and the oracle on seeded problems. Any sanitizer report
fails the run. Needs the package's kernel objects (built by __graft_entry__.build()).
"""
from __future__ import annotations

import glob
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "tests", "sanitize", "build.sh")


def _gpu_visible() -> bool:
    return os.path.exists("/dev/kfd") and bool(glob.glob("/dev/dri/renderD*"))


@pytest.mark.skipif(not glob.glob(os.path.join(ROOT, "weight_only_quantized_matmul_amd", "_build", "*.hip.o")),
                    reason="kernel objects not built (run __graft_entry__.build())")
@pytest.mark.skipif(_gpu_visible(), reason="the host-only checks expect no GPU (no-device startup path)")
def test_sanitized_host_build_runs_clean():
    with tempfile.TemporaryDirectory() as tmp:
        b = subprocess.run(["bash", BUILD, tmp], capture_output=True, text=True, timeout=600)
        assert b.returncode == 0, b.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([os.path.join(tmp, "sanitize_main")], capture_output=True, text=True, timeout=600,
                           env=env)
        assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
        assert "all checks passed" in r.stdout
