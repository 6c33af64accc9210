"""Stores of keys compiled from position 0 (needs an MI355X).

EPIC (atlas.scime.ai summary, "Approach") compiles every chunk on its own from
position 0, so a chunk's token j carries its key rotated at position j. A store
made with key_layout "segment_rope" takes keys in that form, and the link step
re-rotates each one by its segment's linked start. The scatter writes the
recomputed rows' keys in the same form, at their position inside their
segment. The seeded cached keys of the workloads are taken as keys in that
form. The oracle rotates each cached key by its segment's start and each new
key by its absolute position. Tolerance as for the position-free store:
bf16 |gpu - oracle| <= 2e-2 + 1e-2 |oracle|, fp32 1e-5 + 1e-5 |oracle|.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.test_gpu_decode import check as check_decode
from tests.test_gpu_decode import rotate_at, run_decode
from tests.test_gpu_parity import EDGE, check, run_workload, small_cfg
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEG = "segment_rope"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pic.lib()


@pytest.mark.parametrize("name,sample", [("tiny", None), ("llama3_k2", None), ("batched_k16", 12),
                                         ("long50k_k32", 12), ("block_zipf", 4)])
def test_workloads(name, sample):
    cfg = CONFIGS[name]
    _say(f"{name}, segment-rotated keys")
    got, want, ex = run_workload(cfg, sample_rows=sample, key_layout=SEG)
    check(cfg, got, want, ex, f"{name} segment keys")


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases_keys_rotated_inside_attention(name):
    cfg = small_cfg(**EDGE[name])
    _say(f"edge case {name}, segment-rotated keys, rotated inside attention")
    got, want, ex = run_workload(cfg, key_layout=SEG, rope_keys=1)
    assert ex["plan"].sizes["rotated_pages"] == 0
    check(cfg, got, want, ex, f"{name} segment keys inside")


@pytest.mark.parametrize("name", [n for n, c in EDGE.items() if c.get("dtype", "bf16") == "bf16"])
def test_edge_cases_keys_rotated_ahead(name):
    cfg = small_cfg(**EDGE[name])
    _say(f"edge case {name}, segment-rotated keys, rotated ahead of attention")
    got, want, ex = run_workload(cfg, key_layout=SEG, rope_keys=2)
    assert ex["plan"].sizes["rotated_pages"] == ex["plan"].sizes["pages"]
    check(cfg, got, want, ex, f"{name} segment keys ahead")


@pytest.mark.parametrize("case", ["llama3_k2", "split_offset"])
def test_rotation_modes_are_bit_identical(case):
    """Both rotation modes rotate a stored key by its segment's start with the same table row and
    the same arithmetic."""
    if case == "llama3_k2":
        cfg, kw = CONFIGS["llama3_k2"], {}
    else:
        cfg, kw = small_cfg(chunk_len=300, chunks_per_request=6, k=20), dict(split_pages=4, pos_offset=4097)
    a, _, ex_a = run_workload(cfg, rope_keys=1, with_oracle=False, check_plan=False, key_layout=SEG, **kw)
    b, _, ex_b = run_workload(cfg, rope_keys=2, with_oracle=False, check_plan=False, key_layout=SEG, **kw)
    assert np.array_equal(a, b)
    assert np.array_equal(ex_a["lse"], ex_b["lse"])


@pytest.mark.parametrize("split,offset", [(4, 0), (-1, 100000)])
def test_split_and_offset(split, offset):
    cfg = small_cfg(chunk_len=300, chunks_per_request=6, k=20)
    got, want, ex = run_workload(cfg, split_pages=split, pos_offset=offset, key_layout=SEG)
    check(cfg, got, want, ex, f"segment keys split {split} offset {offset}")


@pytest.mark.parametrize("dtype,rope_keys", [("bf16", 1), ("bf16", 2), ("f32", 1)])
def test_scatter_writes_new_keys_rotated_inside_their_segment(dtype, rope_keys):
    """Private pages hold the new rows' keys rotated at their position inside their segment
    (within one bf16 rounding of the exact rotation; fp32 within 1e-6 relative + 4e-6), cached rows copied as
    stored, values as given, and zero padding."""
    cfg = small_cfg(k=3, chunk_len=45, **({"dtype": "f32", "kv_scale": 1.0} if dtype == "f32" else {}))
    got, want, ex = run_workload(cfg, key_layout=SEG, pos_offset=333, rope_keys=rope_keys)
    check(cfg, got, want, ex, f"segment keys scatter {dtype} rope_keys {rope_keys}")
    store, segs, rows, cached = ex["store"], ex["segs"], ex["rows"], ex["cached"]
    exp_ = ex["export"]
    B = cfg.page_size
    kp = store.k_pool.float().cpu().numpy()
    vp = store.v_pool.float().cpu().numpy()
    rel, slack = (2.0 ** -8, 1e-6) if dtype == "bf16" else (1e-6, 4e-6)
    n_checked = 0
    for i, s in enumerate(segs):
        pages = oplan.logical_pages(s, B)
        p0 = exp_["cu_pages"][i]
        qn, kn, vn = rows[i]
        row_of_seg = np.cumsum([0] + [g.recompute for g in s])
        for lp, pg in enumerate(pages):
            if not pg.private:
                continue
            seg = s[pg.segment]
            phys = exp_["block_table"][p0 + lp]
            for slot in range(B):
                j = pg.index * B + slot
                gk, gv = kp[phys][:, slot], vp[phys][:, slot]
                if slot >= pg.valid:
                    assert not gk.any() and not gv.any()
                elif j < seg.recompute:
                    r = row_of_seg[pg.segment] + j
                    wk = rotate_at(kn[r].astype(np.float64), j, cfg.rope_theta)
                    assert np.all(np.abs(gk - wk) <= rel * np.abs(wk) + slack), (i, lp, slot)
                    assert np.array_equal(gv, vn[r])
                    n_checked += 1
                else:
                    assert np.array_equal(gk, cached[seg.chunk_id][0][j])
                    assert np.array_equal(gv, cached[seg.chunk_id][1][j])
    assert n_checked > 0


@pytest.mark.parametrize("name", ["ragged_bf16", "no_prefix_no_suffix", "g8_bf16"])
def test_decode_after_link(name):
    cfg = small_cfg(**EDGE[name])
    _say(f"decode, edge case {name}, segment-rotated keys")
    check_decode(cfg, run_decode(cfg, steps=3, key_layout=SEG), f"decode {name} segment keys")


@pytest.mark.parametrize("suffix_len,steps", [(15, 4), (0, 18)])
def test_decode_steps_cross_pages(suffix_len, steps):
    cfg = small_cfg(suffix_len=suffix_len, n_requests=2, chunk_len=50)
    _say(f"decode, suffix {suffix_len}, {steps} steps, segment-rotated keys")
    check_decode(cfg, run_decode(cfg, steps=steps, key_layout=SEG), f"decode suffix {suffix_len} segment keys")


def test_decode_long50k():
    cfg = CONFIGS["long50k_k32"]
    _say("decode, long50k_k32, segment-rotated keys")
    check_decode(cfg, run_decode(cfg, steps=2, key_layout=SEG), "decode long50k segment keys")


@pytest.mark.parametrize("rope_keys", [1, 2])
def test_dense_recompute_all(rope_keys):
    """Every row recomputed: every page is private and every key arrives position-free, so the
    scatter writes all of them into the store's form before attention rotates them back out."""
    cfg = small_cfg(chunk_len=100, chunks_per_request=3, n_requests=1)
    got, want, ex = run_workload(cfg, recompute_all=True, rope_keys=rope_keys, key_layout=SEG)
    assert ex["plan"].sizes["cow_pages"] == 0
    check(cfg, got, want, ex, f"segment keys recompute_all rope_keys {rope_keys}")
