"""The GPU output checks can fail at long key ranges (CPU only).

At long key ranges the outputs of random values average to about 0.01, below the task's
element-wise bfloat16 tolerance (2e-2 + 1e-2 |x|), so that tolerance alone accepts all-zero
outputs and attention that ignores the queries. The GPU tests therefore add two checks, and this
file shows on the CPU that each rejects such answers on the rows the GPU tests look at:

* the norm-wise bound per (row, head), ||gpu - oracle|| / ||oracle|| <= 1e-2
  (tests.harness.check_rows), on oracle rows of the 12,416-, 8,256- and 50,304-token requests
  and of the 2,048-page work item: it accepts the oracle rounded to bfloat16 and rejects zeros
  and uniform attention (the oracle with zero queries);
* the exact-mean check of the zero-query tests with structured values
  (tests.harness.assert_exact_mean): it accepts the mean rounded to bfloat16 and rejects zeros,
  the mean of the neighbouring KV head, a shifted head dimension, and value pages of the second
  half of the keys read from the first half.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import link as olink
from oracle import plan as oplan
from tests.harness import Workload, assert_exact_mean, check_rows
from workloads import CONFIGS, gen


def _bf16(x):
    return gen.round_bf16(np.asarray(x, dtype=np.float32)).astype(np.float64)


def _limit_cfg():
    base = dict(CONFIGS["llama3_k2"].__dict__)
    base.update(name="limit", num_q_heads=8, num_kv_heads=2, k=32, prefix_len=0, chunk_len=512,
                chunks_per_request=64, suffix_len=16, n_requests=1, pool_size=64, pool_draw="uniform",
                seed=77)
    return CONFIGS["llama3_k2"].__class__(**base)


CASES = {
    "batched_k16": (lambda: CONFIGS["batched_k16"], [0, 255, 511]),
    "block_zipf": (lambda: CONFIGS["block_zipf"], [0, 100, 191]),
    "long50k_k32": (lambda: CONFIGS["long50k_k32"], [0, 1600, 3199]),
    "2,048-page item": (_limit_cfg, [2047, 2048, 2063]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_normwise_check_rejects_zero_and_uniform_outputs(name):
    make, rows = CASES[name]
    cfg = make()
    wl = Workload(cfg, n_requests=1)
    segs = wl.segments()
    cached = wl.cached()
    q, k, v = wl.new_rows(segs)[0]
    want, _ = olink.link_attention(segs[0], cached, q, k, v, cfg.rope_theta, rows=rows)
    uniform, _ = olink.link_attention(segs[0], cached, np.zeros_like(q), k, v, cfg.rope_theta, rows=rows)
    check_rows(_bf16(want), want, "bf16", f"power {name} rounded")      # the right answer passes
    # the task's element-wise tolerance alone takes zeros on most of these rows
    atol, rtol = 2e-2, 1e-2
    loose = np.abs(want) <= atol + rtol * np.abs(want)
    assert loose.mean() > 0.5 or name in ("batched_k16",)
    for wrong, label in ((np.zeros_like(want), "zeros"), (_bf16(uniform), "uniform attention")):
        with pytest.raises(AssertionError):
            check_rows(wrong, want, "bf16", f"power {name} {label}")


def _structured(cfg):
    wl = Workload(cfg, n_requests=1)
    segs = wl.segments()[0]
    vals = []
    for s in segs:
        if s.kind == "suffix":
            vals.append(gen.structured_values(0, s.length, cfg.num_kv_heads, cfg.head_dim, new=True))
        else:
            cid = s.chunk_id
            vals.append(gen.structured_values(cid, s.length, cfg.num_kv_heads, cfg.head_dim))
    return segs, np.concatenate(vals).astype(np.float64)


@pytest.mark.parametrize("name", ["long50k_k32", "2,048-page item"])
def test_exact_mean_check_rejects_wrong_value_gathers(name):
    cfg = CASES[name][0]()
    segs, vals = _structured(cfg)
    n = vals.shape[0]
    G = cfg.num_q_heads // cfg.num_kv_heads
    p = np.array(oplan.selected_positions(segs)[-40:], dtype=np.int64)     # the longest rows
    csum = np.cumsum(vals, axis=0)
    want = np.repeat(csum[p] / (p + 1)[:, None, None], G, axis=1)
    assert np.abs(want).max() > 0.1                                      # O(1) outputs
    assert_exact_mean(_bf16(want), want, "rounded mean")
    # neighbouring KV head, head dimension shifted by one, second half of the keys from the first
    other_head = np.repeat((csum[p] / (p + 1)[:, None, None])[:, np.r_[1:cfg.num_kv_heads, 0]], G, axis=1)
    shifted = np.roll(want, 1, axis=-1)
    half = n // 2 // cfg.page_size * cfg.page_size
    aliased_vals = vals.copy()
    aliased_vals[half:2 * half] = vals[:half]
    acs = np.cumsum(aliased_vals, axis=0)
    aliased = np.repeat(acs[p] / (p + 1)[:, None, None], G, axis=1)
    for wrong, label in ((np.zeros_like(want), "zeros"), (other_head, "other head"), (shifted, "shifted dims"),
                         (aliased, "aliased pages")):
        with pytest.raises(AssertionError):
            assert_exact_mean(_bf16(wrong), want, label)
