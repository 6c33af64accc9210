"""Store lifecycle on the GPU (needs an MI355X): least-recently-used eviction, new chunks stored
into the reclaimed pages, and link calls over old and new chunks checked against the oracle
(MEPIC abstract: chunk blocks shared across requests and batches; EPIC digest, key design: the
cache replacement policy, LRU for example).

1. Eight chunks are stored and four of them linked: those four become the most recently used.
2. Evicting down to a free-page target releases the other four, least recently used first.
3. Four new chunks are stored: they take exactly the pages the evicted chunks held.
4. Requests over surviving and new chunks are linked; every output row matches the oracle over
   the chunks' current contents, so no stale page content is read.
5. A chunk released while a plan holds it keeps its pages: the plan's link call gives the same
   bits again, and eviction does not count those pages as reclaimable.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import check_rows, gpu_store, oracle_outputs, oracle_segments
from tests.test_gpu_parity import small_cfg
from workloads import gen

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


L = 96           # tokens per chunk: 6 pages of 16
SUFFIX = 20


def _link(cfg, store, cached, requests, what, rows_seed):
    segs = [oracle_segments(cfg, ids, r, prefix_len=0, suffix_len=SUFFIX, chunk_lens=[L] * len(ids))
            for r, ids in enumerate(requests)]
    plan = store.link_plan([pic.LinkRequest(chunk_ids=ids, suffix_len=SUFFIX) for ids in requests], k=cfg.k)
    rows = [gen.new_rows(cfg, rows_seed + r, len(oplan.selected_positions(s))) for r, s in enumerate(segs)]
    q, kn, vn = (torch.from_numpy(np.concatenate([r[i] for r in rows])).to("cuda", torch.bfloat16).contiguous()
                 for i in range(3))
    out = pic.link_attend(store, plan, q, kn, vn)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    want = oracle_outputs(segs, cached, rows, cfg.rope_theta)
    ex = plan.export()
    for i, (wo, _) in enumerate(want):
        check_rows(got[ex["cu_rows"][i]:ex["cu_rows"][i + 1]], wo, "bf16", what)
    return plan, (q, kn, vn), got


def test_evict_refill_and_link():
    cfg = small_cfg(k=4, prefix_len=0)
    old_ids, new_ids = list(range(8)), [100, 101, 102, 103]
    cached = {c: gen.chunk_kv(cfg.__class__(**{**cfg.__dict__, "chunk_len": L}), c) for c in old_ids}
    store = gpu_store(cfg, cached, num_pages=64, max_position=4096)
    assert store.stats()["free_pages"] == 64 - 48
    pages_before = {c: set(store.chunk_pages(c)[0].tolist()) for c in old_ids}

    # 1. link chunks 0-3: they are now the most recently used
    p1, _, _ = _link(cfg, store, cached, [[0, 1], [2, 3]], "lifecycle: before eviction", 10)
    p1.free()
    # 2. evict down to 40 free pages: chunks 4-7, the least recently used, go
    n = store.evict(16 + 24)
    assert n == 4 and store.stats()["free_pages"] == 40
    for c in (4, 5, 6, 7):
        with pytest.raises(pic.PicError):
            store.chunk_pages(c)
    # 3. new chunks take exactly the reclaimed pages
    mk = cfg.__class__(**{**cfg.__dict__, "chunk_len": L, "seed": 991})
    for c in new_ids:
        k, v = gen.chunk_kv(mk, c)
        cached[c] = (k, v)
        store.store_chunk(c, torch.from_numpy(k).to("cuda", torch.bfloat16).contiguous(),
                          torch.from_numpy(v).to("cuda", torch.bfloat16).contiguous())
    reclaimed = set().union(*(pages_before[c] for c in (4, 5, 6, 7)))
    refilled = set().union(*(set(store.chunk_pages(c)[0].tolist()) for c in new_ids))
    assert refilled == reclaimed
    for c in (4, 5, 6, 7):
        del cached[c]
    # 4. link over surviving and new chunks
    p2, tensors, got = _link(cfg, store, cached, [[100, 0, 101], [102, 3, 103, 1]], "lifecycle: after refill", 20)
    # 5. a chunk released while the plan holds it keeps its pages
    store.release(0)
    used_by_plan = store.usage()["pages_plans_only"]
    assert used_by_plan >= 6 + p2.sizes["private_pages"]
    with pytest.raises(pic.PicError):
        store.evict(64)          # the plan's pages cannot be freed
    again = pic.link_attend(store, p2, *tensors).float().cpu().numpy()
    assert np.array_equal(again, got)
    p2.free()
    assert store.usage()["pages_plans_only"] == 0
    _say(f"lifecycle: {n} chunks evicted, {len(refilled)} pages refilled; usage {store.usage()}")
