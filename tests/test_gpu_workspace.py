"""Workspace ownership on the GPU (needs an MI355X).

A link call reads its plan's tables from the workspace and writes split partials and rotated keys
there, so the library keeps track of which plan each workspace region holds (the last upload into
it). pic_link_attend copies its plan's tables in when the workspace does not hold them, which also
makes the plain sequence plan -> attend work without an explicit upload; pic_link_decode, whose
rotated keys and decode tables the link call left in the workspace, refuses a workspace another
plan was uploaded into, before any launch.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import Workload, gpu_store, oracle_outputs
from tests.test_gpu_decode import decode_rows
from tests.test_gpu_parity import check, small_cfg

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


def _setup(cfg, n_req_a, n_req_b, decode=0):
    wl_a = Workload(cfg, n_requests=n_req_a)
    wl_b = Workload(cfg)
    cached = wl_b.cached()
    B = cfg.page_size
    jobs = []
    for wl in (wl_a, wl_b):
        segs = wl.segments(k=cfg.k)
        jobs.append((wl, segs, wl.new_rows(segs)))
    private = sum(p.private for _, segs, _ in jobs for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for _, segs, _ in jobs for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + 64, max_position=n_tokens + decode + 8)
    plans, tensors = [], []
    for wl, segs, rows in jobs:
        plans.append(store.link_plan(wl.link_requests(), k=cfg.k, decode=decode))
        tensors.append([torch.from_numpy(np.concatenate([r[i] for r in rows])).to("cuda", torch.bfloat16).contiguous()
                        for i in range(3)])
    return store, jobs, cached, plans, tensors


def test_attend_copies_in_a_plan_the_workspace_does_not_hold():
    """upload(A), upload(B) into one workspace, attend(A): the library sees that the workspace holds
    B and copies A's tables back in first; both results match the oracle. A third plan runs with no
    upload call at all (plan -> attend)."""
    cfg = small_cfg(n_requests=3, k=4)
    store, jobs, cached, plans, tensors = _setup(cfg, 1, 3)
    ws = torch.empty(max(p.sizes["workspace_bytes"] for p in plans), dtype=torch.uint8, device="cuda")
    plans[0].upload(ws)
    plans[1].upload(ws)
    out_a = pic.link_attend(store, plans[0], *tensors[0])
    out_b = pic.link_attend(store, plans[1], *tensors[1])
    torch.cuda.synchronize()
    for (wl, segs, rows), out, what in ((jobs[0], out_a, "A after B's upload"), (jobs[1], out_b, "B after A's")):
        plan = plans[0] if what.startswith("A") else plans[1]
        want = oracle_outputs(segs, cached, rows, cfg.rope_theta)
        check(cfg, out.float().cpu().numpy(), want, dict(export=plan.export(), sample=None, lse=None),
              f"workspace: {what}")
    fresh = store.link_plan(jobs[1][0].link_requests(), k=cfg.k)
    assert fresh.workspace is None
    out_c = pic.link_attend(store, fresh, *tensors[1])      # no upload call
    torch.cuda.synchronize()
    assert np.array_equal(out_c.float().cpu().numpy(), out_b.float().cpu().numpy())
    for p in plans + [fresh]:
        p.free()


def test_decode_refuses_a_workspace_another_plan_was_uploaded_into():
    cfg = small_cfg(n_requests=2, k=4)
    store, jobs, cached, plans, tensors = _setup(cfg, 2, 2, decode=2)
    n = plans[0].sizes["requests"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16).contiguous()
    tok = [dev(t) for t in decode_rows(cfg, n, cfg.seed, 0)]
    # reference: plan A alone in its own workspace
    pic.link_attend(store, plans[0], *tensors[0])
    ref = pic.link_decode(store, plans[0], *tok).float().cpu().numpy()
    ws = plans[0].workspace
    plans[1].upload(ws)                                       # B over A's tables and rotated keys
    with pytest.raises(pic.PicError) as e:
        pic.link_decode(store, plans[0], *tok)
    assert e.value.status == -6
    # A's link call again (the library copies A's tables back in), then decode works
    pic.link_attend(store, plans[0], *tensors[0])
    again = pic.link_decode(store, plans[0], *tok).float().cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(again, ref)
    # uploading A again without a link call leaves nothing for decode to read
    plans[0].upload(ws)
    with pytest.raises(pic.PicError) as e:
        pic.link_decode(store, plans[0], *tok)
    assert e.value.status == -7
    torch.cuda.synchronize()
    for p in plans:
        p.free()
