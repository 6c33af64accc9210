"""Persistent attention launches (needs an MI355X).

With more work items than compute units, the bf16 attention kernels run one work group per
compute unit, each taking items from per-XCD queues through counters in the plan's workspace
that the launch puts back to zero at its end. These cases force that path with small split
pieces, on one queue (2 KV heads) and on eight (8 KV heads), with keys rotated inside
attention and ahead of it, and check that
  - every launch matches the oracle, and repeated launches over one upload are bit-identical
    (a counter left non-zero would skip items on the next launch);
  - a second plan uploaded into the same workspace, and the first one again, still give the
    right results (the upload resets the counters with the tables).
"""
from __future__ import annotations

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from tests.test_gpu_parity import _say, check, run_workload, small_cfg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pic.lib()


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _cfg(kv_heads):
    # 4-page pieces: 480 items at 2 KV heads (4 requests), 960 at 8 (2 requests)
    return small_cfg(num_q_heads=2 * kv_heads, num_kv_heads=kv_heads, chunk_len=300, chunks_per_request=6, k=20,
                     n_requests=4 if kv_heads == 2 else 2)


@pytest.mark.parametrize("kv_heads", [2, 8])
@pytest.mark.parametrize("rope_keys", [1, 2])
def test_persistent_launches_repeat_exactly(kv_heads, rope_keys):
    cfg = _cfg(kv_heads)
    _say(f"persistent launch: kv_heads {kv_heads}, rope_keys {rope_keys}")
    got, want, ex = run_workload(cfg, split_pages=4, rope_keys=rope_keys, repeat=3)
    assert ex["plan"].sizes["work_items"] > _cus(), "the case must have more items than compute units"
    check(cfg, got, want, ex, f"persistent kv{kv_heads} rope{rope_keys}")
    for i in (1, 2):
        assert np.array_equal(ex["outs"][0], ex["outs"][i]), f"launch {i} differs from launch 0"


def test_plans_sharing_a_workspace():
    cfg = _cfg(8)
    _say("two plans, one workspace")
    got, want, ex = run_workload(cfg, split_pages=4, rope_keys=2, num_pages=512)   # room for two plans
    store, plan_a = ex["store"], ex["plan"]
    ws = plan_a.workspace
    q, kn, vn = (torch.from_numpy(np.concatenate([r[j] for r in ex["rows"]])).to("cuda", torch.bfloat16).contiguous()
                 for j in range(3))
    # plan B: the same requests in larger pieces (fewer items), uploaded over plan A's tables
    plan_b = store.link_plan(ex["link_requests"], k=cfg.k, block_level=cfg.block_level, split_pages=12, rope_keys=2)
    assert plan_b.sizes["work_items"] != plan_a.sizes["work_items"]
    assert plan_b.sizes["workspace_bytes"] <= ws.numel()
    plan_b.upload(ws)
    out_b = pic.link_attend(store, plan_b, q, kn, vn)
    torch.cuda.synchronize()
    check(cfg, out_b.float().cpu().numpy(), want, dict(ex, lse=None), "plan B in plan A's workspace")
    # plan A again, into the same workspace: its first result, bit for bit
    plan_a.upload(ws)
    out_a = pic.link_attend(store, plan_a, q, kn, vn)
    torch.cuda.synchronize()
    assert np.array_equal(out_a.float().cpu().numpy(), got)
    plan_b.free()
