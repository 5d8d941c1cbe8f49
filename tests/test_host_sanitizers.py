"""The library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The host side of every source is built with both sanitizers (device code as
usual, never launched here), the compiler's sanitizer runtime is preloaded
into a fresh Python, and the C-ABI validation tests (tests/test_abi.py) run
against that build: every entry point's argument checks, workspace queries
and status strings, with invalid sizes, dtypes, masks and pointers.  Any
sanitizer report ends the run with an error and fails this test.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

from block_diffusion_vlm_amd import build

ROOT = Path(__file__).resolve().parent.parent


def test_abi_validation_is_clean_under_asan_and_ubsan(tmp_path):
    try:
        rt = build.host_asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_host_sanitized(verbose=False)
    log = tmp_path / "san"
    env = dict(os.environ, BDIFF_LIB=str(lib), LD_PRELOAD=str(rt),
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    reports = "".join(p.read_text() for p in tmp_path.glob("san*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:], reports[:5000])
