"""Host side of the library under AddressSanitizer (no GPU): the library is built with
its host code instrumented (-Xarch_host -fsanitize=address; device code unchanged) and
asan_host_driver.py drives its argument validation, workspace sizing, chunk planning
and stage listing through the C ABI in a process with the sanitizer runtime preloaded.
Any invalid read or write in that code ends the process with a sanitizer report."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_side_under_address_sanitizer():
    from learned_top_sparse_amd.build import asan_runtime, build_host_asan
    lib = build_host_asan()
    env = dict(os.environ, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0")
    p = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "asan_host_driver.py"), lib], env=env,
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert "AddressSanitizer" not in p.stderr, p.stderr[-4000:]
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-4000:]
    assert "host-side calls exercised" in p.stdout
