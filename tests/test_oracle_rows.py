"""Pin of the oracle's row-subset path (CPU only).

``oracle.link.link_attention(rows=S)`` computes only the rows S and cuts the merged cache after
the last key at or before the largest requested position; every sampled full-size parity check
and the benchmark's CPU baseline go through it. It must give exactly the rows S of the full
result: a row attends to every key at or before its own position, so no key it sees may be cut.

* Brute-force cases: every subset is checked against tests/brute.py (dense N x N statement, no
  truncation) to 1e-12, and subsets that leave out the last row against the full call bit for
  bit (the full call's cut is then later than the subset's).
* Llama-shaped request of 5,216 tokens: subsets against the full call, bit for bit.
* The 50,304-token request: single rows against the same rows computed together with the last
  row (whose cut keeps every key), bit for bit.
* A cut that drops the last requested row's own key (side="left") fails these pins.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import link as olink
from tests.harness import Workload
from tests.test_oracle import CASES, run_brute, tiny_request
from workloads import CONFIGS


def _subsets(R, seed):
    g = np.random.default_rng(seed)
    out = [[0], [R - 1], [R // 2], list(range(R))]
    if R > 2:
        out.append(sorted(int(x) for x in g.choice(R, size=min(R - 1, 5), replace=False)))
        out.append(list(range(R - 1)))
    return [s for s in out if s]


def subset_pins_brute(case):
    req = tiny_request(500 + case, **CASES[case])
    full, full_lse = olink.link_attention(req["segs"], req["cached"], req["q"], req["k"], req["v"], req["theta"])
    R = full.shape[0]
    if R == 0:
        return 0
    bo, bl, _ = run_brute(req)
    for S in _subsets(R, case):
        out, lse = olink.link_attention(req["segs"], req["cached"], req["q"], req["k"], req["v"], req["theta"],
                                        rows=S)
        assert np.abs(out - bo[S]).max() < 1e-12 and np.abs(lse - bl[S]).max() < 1e-12, (case, S)
        if R - 1 not in S:
            assert np.array_equal(out, full[S]) and np.array_equal(lse, full_lse[S]), (case, S)
    return R


@pytest.mark.parametrize("case", range(len(CASES)))
def test_subset_rows_match_brute_force_and_full_call(case):
    subset_pins_brute(case)


def _workload(name):
    cfg = CONFIGS[name]
    wl = Workload(cfg)
    segs = wl.segments()
    return cfg, segs[0], wl.cached(), wl.new_rows(segs)[0]


def subset_pins_llama():
    cfg, segs, cached, (q, k, v) = _workload("llama3_k2")
    full, full_lse = olink.link_attention(segs, cached, q, k, v, cfg.rope_theta)
    R = full.shape[0]
    for S in _subsets(R, 3):
        out, lse = olink.link_attention(segs, cached, q, k, v, cfg.rope_theta, rows=S)
        assert np.array_equal(out, full[S]) and np.array_equal(lse, full_lse[S]), S


def test_subset_rows_of_the_5216_token_request_equal_the_full_call():
    subset_pins_llama()


def subset_pins_long(rows=(0, 31, 1600, 3167)):
    cfg, segs, cached, (q, k, v) = _workload("long50k_k32")
    R = q.shape[0]
    joint, joint_lse = olink.link_attention(segs, cached, q, k, v, cfg.rope_theta, rows=list(rows) + [R - 1])
    for i, r in enumerate(rows):
        out, lse = olink.link_attention(segs, cached, q, k, v, cfg.rope_theta, rows=[r])
        assert np.array_equal(out[0], joint[i]) and np.array_equal(lse[0], joint_lse[i]), r


def test_single_rows_of_the_50k_request_equal_rows_computed_with_the_last_row():
    subset_pins_long()


class _LeftCut:
    """numpy with searchsorted forced to side="left": the cut then drops the key at the last
    requested row's own position."""

    def __getattr__(self, name):
        return getattr(np, name)

    @staticmethod
    def searchsorted(a, v, side="left", sorter=None):
        return np.searchsorted(a, v, side="left", sorter=sorter)


def test_pins_catch_a_cut_that_drops_the_rows_own_key(monkeypatch):
    monkeypatch.setattr(olink, "np", _LeftCut())
    caught = 0
    for case in range(len(CASES)):
        try:
            subset_pins_brute(case)
        except AssertionError:
            caught += 1
    assert caught >= len(CASES) - 2      # only cases without rows, or without a cut, pass
    with pytest.raises(AssertionError):
        subset_pins_llama()
    with pytest.raises(AssertionError):
        subset_pins_long(rows=(1600,))
