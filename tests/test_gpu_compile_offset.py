"""Keys compiled after leading tokens: LegoLink-0's compile form (needs an MI355X).

EPIC's LegoLink-0 ablation prepends four dummy tokens when a chunk is compiled and discards their
KV, with no recomputation at link time (EPIC summary, "Measured effects" table). With the dummies
at positions 0..3, a chunk's token j is stored rotated at 4 + j (store option compile_offset = 4
of PIC_KEYS_SEGMENT_ROPE), and the link step re-rotates every stored key by its segment's start
minus 4: a negative angle for a segment that starts before position 4 (a prefix or a first chunk
at position 0). New keys (recomputed rows, decode tokens) are written in the same form, rotated
at 4 + their position in the segment. Every case is checked against the fp64 oracle, both key
rotation modes must agree bit for bit, and the seeded keys are taken as already rotated (the
oracle reads them in the same form).
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
C = 4   # LegoLink-0's dummy tokens


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pic.lib()


@pytest.mark.parametrize("name,k,sample", [("llama3_k2", 0, None), ("llama3_k2", 2, None),
                                           ("batched_k16", 0, 12), ("long50k_k32", 0, 24)])
def test_workloads(name, k, sample):
    cfg = CONFIGS[name]
    _say(f"{name}, k {k}, keys compiled after {C} leading tokens")
    got, want, ex = run_workload(cfg, k=k, sample_rows=sample, key_layout=SEG, compile_offset=C)
    check(cfg, got, want, ex, f"{name} k{k} compile offset {C}")


LEGO0_EDGE = ["ragged_bf16", "ragged_f32", "k0_link_half", "no_prefix_no_suffix", "one_token_chunks",
              "page64_k40", "block_page32", "d64_f32_g8", "prefix_and_suffix_only"]


@pytest.mark.parametrize("rope_keys", [1, 2])
@pytest.mark.parametrize("name", LEGO0_EDGE)
def test_edge_cases(name, rope_keys):
    cfg = small_cfg(**EDGE[name])
    if rope_keys == 2 and cfg.dtype != "bf16":
        pytest.skip("keys are rotated ahead for bfloat16 stores only")
    _say(f"edge case {name}, rope_keys {rope_keys}, compile offset {C}")
    got, want, ex = run_workload(cfg, rope_keys=rope_keys, key_layout=SEG, compile_offset=C)
    check(cfg, got, want, ex, f"{name} compile offset {C} rope_keys {rope_keys}")


@pytest.mark.parametrize("offset", [0, 2, 4097])
def test_rotation_modes_are_bit_identical(offset):
    """A first chunk at position 0 or 2 is re-rotated by a negative angle (-4, -2); inside
    attention and in the rotation pass the sines are negated the same way."""
    cfg = small_cfg(prefix_len=0, k=0, chunk_len=150)
    a, _, ex_a = run_workload(cfg, rope_keys=1, with_oracle=False, check_plan=False, pos_offset=offset,
                              key_layout=SEG, compile_offset=C)
    b, _, ex_b = run_workload(cfg, rope_keys=2, with_oracle=False, check_plan=False, pos_offset=offset,
                              key_layout=SEG, compile_offset=C)
    assert np.array_equal(a, b) and np.array_equal(ex_a["lse"], ex_b["lse"])


@pytest.mark.parametrize("rope_keys", [1, 2])
def test_new_keys_are_written_at_the_offset(rope_keys):
    """Private pages hold the recomputed rows' keys rotated at C + their position in the segment
    (one bf16 rounding of the exact rotation)."""
    cfg = small_cfg(k=3, chunk_len=45, prefix_len=0)
    got, want, ex = run_workload(cfg, key_layout=SEG, compile_offset=C, rope_keys=rope_keys)
    check(cfg, got, want, ex, f"compile offset {C} scatter rope_keys {rope_keys}")
    store, segs, rows = ex["store"], ex["segs"], ex["rows"]
    exp_ = ex["export"]
    B = cfg.page_size
    kp = store.k_pool.float().cpu().numpy()
    n_checked = 0
    for i, s in enumerate(segs):
        p0 = exp_["cu_pages"][i]
        row_of_seg = np.cumsum([0] + [g.recompute for g in s])
        for lp, pg in enumerate(oplan.logical_pages(s, B)):
            if not pg.private:
                continue
            seg = s[pg.segment]
            phys = exp_["block_table"][p0 + lp]
            for slot in range(pg.valid):
                j = pg.index * B + slot
                if j < seg.recompute:
                    wk = rotate_at(rows[i][1][row_of_seg[pg.segment] + j].astype(np.float64), C + j, cfg.rope_theta)
                    assert np.all(np.abs(kp[phys][:, slot] - wk) <= 2.0 ** -8 * np.abs(wk) + 1e-6), (i, lp, slot)
                    n_checked += 1
    assert n_checked > 0


@pytest.mark.parametrize("rope_keys", [1, 2])
@pytest.mark.parametrize("name", ["ragged_bf16", "no_prefix_no_suffix"])
def test_decode_after_link(name, rope_keys):
    """Decode over keys rotated at C + j, whose first segments link before C (negative rotations):
    from the pools, rotated in the decode kernel (rope_keys 1), and from the link call's rotated copy,
    which each step extends with its token's key (rope_keys 2)."""
    cfg = small_cfg(**EDGE[name])
    _say(f"decode, edge case {name}, compile offset {C}, rope_keys {rope_keys}")
    check_decode(cfg, run_decode(cfg, steps=3, key_layout=SEG, compile_offset=C, rope_keys=rope_keys),
                 f"decode {name} compile offset {C} rope_keys {rope_keys}")
