"""bench.py end to end on a small workload (needs an MI355X): one JSON line with every field the
benchmark reports, the roofline and CPU-baseline objects included."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bench(*args):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args]
    print("running", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_line_has_every_field():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    d = _bench("--workload", "llama3_k2", "--steps", "3", "--warmup", "2", "--cold-steps", "2",
               "--cpu-seconds", "1")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline",
                "link_latency_wall_ms", "cold", "decode", "model_forward", "dense_comparator",
                "kernel_source_sha256_16"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "llama3_k2" and d["config"]["selected_rows"] == 84
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert rl["achieved"] > 0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    lat = d["link_latency_wall_ms"]
    assert lat["steps"] == 3 and 0 < lat["p10"] <= lat["p50"] <= lat["p90"]
    assert d["cold"]["steps"] == 2 and d["cold"]["p10"] <= d["cold"]["p90"]
    assert d["decode"]["ms"] > 0
    m = d["model_forward"]                 # 32 Llama-3-8B-shaped layers over the 84 selected rows
    assert m["layers"] == 32 and m["rows"] == 84 and m["ms"] > 0 and 0 < m["gemm_frac"] < 1
    assert set(m["gemm"]) == {"qkv", "o", "gate_up_swiglu", "down"}
    # the dense comparator's outputs agree with the link step's at the link rows (bf16 tolerance)
    assert d["dense_comparator"]["max_abs_diff_at_link_rows"] <= 2e-2

