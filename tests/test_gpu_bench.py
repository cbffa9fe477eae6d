"""The benchmark's default run, shortened: it finishes and prints one JSON line with
the fields its readers rely on (metric, value, roofline, per-workload stage times)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = [pytest.mark.gpu]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_headline_line():
    p = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline"], cwd=ROOT, capture_output=True, text=True, timeout=400)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout[-3000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "dtype", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["value"] > 0
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and 0 < r["frac"] < 1.5 and r["peak"] > 0
    for wl in ("decode_128k_paged", "decode_128k_pool4", "prefill_128k", "decode_128k_lsa", "decode_128k_lsa_paged",
               "prefill_128k_lsa", "tiny_prefill_1k", "prefill_32k", "chunk_256k", "decode_128k_pool4_paged",
               "two_stage_128k_paged", "prefill_32k_pool4", "chunk_256k_pool4"):
        assert d[wl]["ms_per_step"] > 0 and d[wl]["kernel_ms"], wl
    assert 0 < d["prefill_128k"]["roofline"]["frac"] < 1.5
    for wl in ("prefill_32k", "chunk_256k"):
        assert 0 < d[wl]["roofline"]["frac"] < 1.5 and 0 < d[wl]["step_roofline_frac"] <= 1.0, wl
        assert d[wl]["attention"]["gather_GBs"] > 0, wl
    pk = d["measured_peaks"]
    # measured ceilings below the published ones (8 TB/s, 5.0 POPS int8, 2.5 PFLOP/s bf16)
    assert 0 < pk["hbm_read_GBs"] < 8000 and 0 < pk["int8_mfma_TOPs"] < 5100 and 0 < pk["bf16_mfma_TFLOPs"] < 2600
    assert 0 < pk["gather_cold_GBs"] < pk["gather_l2_GBs"]
