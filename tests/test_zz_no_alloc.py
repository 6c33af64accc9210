"""The allocation-free link call, pic_link_attend_static, against pic_link_attend (needs an MI355X).

pic_link_attend_static runs the same kernels on the library's static device scratch (64 MiB per
GPU) instead of a caller workspace, so its outputs and log-sum-exps must equal pic_link_attend's
bit for bit. Two calls run back to back on one stream, the second with a smaller request, then
the first again; each is also checked against the fp64 oracle. A plan with more work items than
compute units (persistent attention, its work counters in the scratch) repeats exactly over three
calls. A plan whose workspace exceeds the scratch is refused before any copy or launch.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import Workload, check_rows, gpu_store, oracle_outputs
from tests.test_gpu_parity import small_cfg
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pic.lib()


def _job(cfg, rope_keys, split_pages=0):
    wl = Workload(cfg)
    segs = wl.segments()
    cached = wl.cached()
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + 8, max_position=n_tokens + 1)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, rope_keys=rope_keys,
                           split_pages=split_pages)
    rows = wl.new_rows(segs)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, kn, vn = (torch.from_numpy(np.concatenate([r[i] for r in rows])).to("cuda", tdt).contiguous() for i in range(3))
    return dict(cfg=cfg, segs=segs, cached=cached, rows=rows, store=store, plan=plan, q=q, k=kn, v=vn)


def test_static_scratch_reproduces_link_attend_on_consecutive_calls():
    jobs = [_job(CONFIGS["llama3_k2"], 2), _job(small_cfg(n_requests=1, chunk_len=64, k=3), 1)]
    assert jobs[0]["plan"].sizes["rotated_pages"] > 0 and jobs[1]["plan"].sizes["rotated_pages"] == 0
    assert jobs[0]["plan"].sizes["split_items"] > 0
    assert jobs[1]["plan"].sizes["workspace_bytes"] < jobs[0]["plan"].sizes["workspace_bytes"] <= pic.STATIC_SCRATCH_BYTES
    refs = []
    for j in jobs:
        lse = torch.empty((j["plan"].rows, j["cfg"].num_q_heads), dtype=torch.float32, device="cuda")
        out = pic.link_attend(j["store"], j["plan"], j["q"], j["k"], j["v"], lse=lse)
        torch.cuda.synchronize()
        refs.append((out.float().cpu().numpy(), lse.cpu().numpy()))
    # outputs allocated up front: the static calls themselves allocate nothing
    outs = []
    for j in jobs:
        R, hq, d = j["plan"].rows, j["cfg"].num_q_heads, j["cfg"].head_dim
        outs.append((torch.full((R, hq, d), float("nan"), dtype=j["q"].dtype, device="cuda"),
                     torch.full((R, hq), float("nan"), dtype=torch.float32, device="cuda")))
    for i in (0, 1, 0):
        j = jobs[i]
        _say(f"static scratch: call on request {i} ({j['plan'].rows} rows, workspace "
             f"{j['plan'].sizes['workspace_bytes']} bytes)")
        pic.link_attend_static(j["store"], j["plan"], j["q"], j["k"], j["v"], out=outs[i][0], lse=outs[i][1])
        torch.cuda.synchronize()
        got, got_lse = outs[i][0].float().cpu().numpy(), outs[i][1].cpu().numpy()
        assert np.array_equal(got, refs[i][0]), f"request {i}: outputs differ from pic_link_attend"
        assert np.array_equal(got_lse, refs[i][1]), f"request {i}: lse differs from pic_link_attend"
        want = oracle_outputs(j["segs"], j["cached"], j["rows"], j["cfg"].rope_theta)
        check_rows(got, want[0][0], j["cfg"].dtype, f"static scratch, request {i}")
        outs[i][0].fill_(float("nan"))
        outs[i][1].fill_(float("nan"))
    for j in jobs:
        j["plan"].free()


@pytest.mark.parametrize("rope_keys", [1, 2])
def test_static_scratch_runs_persistent_launches(rope_keys):
    """A plan with more work items than compute units (4-page pieces: 360 of them) runs its
    attention on persistent work groups whose work counters sit in the static scratch. Three
    static calls, with a call on the plan's own workspace between the second and the third,
    all equal pic_link_attend bit for bit."""
    cfg = small_cfg(num_q_heads=4, num_kv_heads=2, chunk_len=300, chunks_per_request=6, k=20, n_requests=3)
    j = _job(cfg, rope_keys, split_pages=4)
    sz = j["plan"].sizes
    assert sz["work_items"] > torch.cuda.get_device_properties(0).multi_processor_count
    assert sz["workspace_bytes"] <= pic.STATIC_SCRATCH_BYTES
    R = j["plan"].rows
    lse = torch.empty((R, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    ref = pic.link_attend(j["store"], j["plan"], j["q"], j["k"], j["v"], lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = ref.float().cpu().numpy(), lse.cpu().numpy()
    out = torch.empty((R, cfg.num_q_heads, cfg.head_dim), dtype=j["q"].dtype, device="cuda")
    out_lse = torch.empty((R, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    for call in range(3):
        _say(f"static scratch, persistent launch {call} (rope_keys {rope_keys}, {sz['work_items']} items)")
        if call == 2:
            pic.link_attend(j["store"], j["plan"], j["q"], j["k"], j["v"])
        out.fill_(float("nan"))
        out_lse.fill_(float("nan"))
        pic.link_attend_static(j["store"], j["plan"], j["q"], j["k"], j["v"], out=out, lse=out_lse)
        torch.cuda.synchronize()
        assert np.array_equal(out.float().cpu().numpy(), ref), f"call {call}: outputs differ"
        assert np.array_equal(out_lse.cpu().numpy(), ref_lse), f"call {call}: lse differs"
    want = oracle_outputs(j["segs"], j["cached"], j["rows"], cfg.rope_theta)
    got = out.float().cpu().numpy()
    for i, (wo, _) in enumerate(want):
        r0 = j["plan"].export()["cu_rows"][i]
        check_rows(got[r0:r0 + wo.shape[0]], wo, cfg.dtype, f"static scratch, persistent, request {i}")
    j["plan"].free()


def test_static_scratch_refuses_a_plan_larger_than_the_scratch():
    cfg = CONFIGS["long50k_k32"]
    store = pic.Store(num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                      page_size=cfg.page_size, num_pages=3500, dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                      max_position=1 << 16)
    for c in range(98):
        store.store_chunk(c, n_tokens=512)          # pages reserved; nothing is read
    plan = store.link_plan([pic.LinkRequest(chunk_ids=list(range(98)), suffix_len=64)], k=32, rope_keys=2)
    assert plan.sizes["workspace_bytes"] > pic.STATIC_SCRATCH_BYTES
    z = torch.zeros((plan.rows, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    zk = torch.zeros((plan.rows, cfg.num_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pic.PicError) as e:
        pic.link_attend_static(store, plan, z, zk, zk)
    assert e.value.status == -6
    torch.cuda.synchronize()
    plan.free()
