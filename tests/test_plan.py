"""The library's planner against the oracle planner, bit for bit (CPU only).

The store runs in metadata-only mode (no device): chunk pages are reserved,
the link planner builds its tables, and the export is compared with the
oracle's row selection, position map, page ownership and copy-on-write list.
"""
from __future__ import annotations

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import Workload, compare_plan, oracle_segments
from workloads import CONFIGS


def meta_store(cfg, num_pages, max_position=1 << 20):
    return pic.Store(num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                     page_size=cfg.page_size, num_pages=num_pages, dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                     max_position=max_position, device=None)


@pytest.mark.parametrize("name", list(CONFIGS))
@pytest.mark.parametrize("pos_offset", [0, 1000])
def test_config_plans_match_oracle(name, pos_offset):
    cfg = CONFIGS[name]
    wl = Workload(cfg)
    B = cfg.page_size
    segs = wl.segments(pos_offset=pos_offset)
    pages_needed = sum(-(-cfg.chunk_len // B) for _ in wl.chunk_ids)
    pages_needed += len(wl.requests) * -(-cfg.prefix_len // B) + plan_private(segs, B)
    store = meta_store(cfg, pages_needed)
    for c in wl.chunk_ids:
        store.store_chunk(c, n_tokens=cfg.chunk_len)
    if cfg.prefix_len:
        for r in wl.requests:
            store.store_chunk(cfg.prefix_id(r), n_tokens=cfg.prefix_len)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, pos_offset=pos_offset)
    assert store.stats()["free_pages"] == 0
    compare_plan(store, plan, segs, B)
    assert plan.sizes["rows"] == sum(len(oplan.selected_positions(s)) for s in segs)
    plan.free()
    assert store.stats()["plans"] == 0


def _random_case(seed):
    g = np.random.default_rng(seed)
    B = int(g.choice([16, 32, 64]))
    n_pool = int(g.integers(1, 7))
    lens = {c: int(g.integers(1, 150)) for c in range(n_pool)}
    reqs = []
    for r in range(int(g.integers(1, 4))):
        ids = [int(x) for x in g.integers(0, n_pool, size=int(g.integers(0, 6)))]
        prefix = int(g.integers(1, 60)) if g.random() < 0.5 else 0
        reqs.append((ids, int(g.integers(0, 40)), prefix))
    k = int(g.integers(0, 40))
    block = bool(g.random() < 0.3)
    off = int(g.integers(0, 3000))
    return B, lens, reqs, k, block, off


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_match_oracle(seed):
    B, lens, reqs, k, block, off = _random_case(seed)
    cfg = CONFIGS["llama3_k2"]
    store = pic.Store(num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=B, num_pages=4000, dtype="bf16",
                      rope_theta=1e4, max_position=100000, device=None)
    for c, L in lens.items():
        store.store_chunk(c, n_tokens=L)
    link_reqs, seg_lists = [], []
    for r, (ids, S, prefix) in enumerate(reqs):
        pid = None
        if prefix:
            pid = 10_000 + r
            store.store_chunk(pid, n_tokens=prefix)
        link_reqs.append(pic.LinkRequest(ids, S, pid))
        seg_lists.append(oplan.link_segments(prefix_id=pid, prefix_len=prefix, chunk_ids=ids,
                                             chunk_lens=[lens[c] for c in ids], suffix_len=S, k=k,
                                             block_level=block, page_size=B, pos_offset=off))
    plan = store.link_plan(link_reqs, k=k, block_level=block, pos_offset=off)
    compare_plan(store, plan, seg_lists, B)
    before = store.stats()["free_pages"]
    plan.free()
    assert store.stats()["free_pages"] == before + plan_private(seg_lists, B)


def plan_private(seg_lists, B):
    return sum(p.private for segs in seg_lists for p in oplan.logical_pages(segs, B))


def test_recompute_all_selects_every_row():
    cfg = CONFIGS["tiny"]
    wl = Workload(cfg)
    store = meta_store(cfg, 200)
    for c in wl.chunk_ids:
        store.store_chunk(c, n_tokens=cfg.chunk_len)
    store.store_chunk(cfg.prefix_id(0), n_tokens=cfg.prefix_len)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, recompute_all=True)
    segs = wl.segments(recompute_all=True)
    ex = compare_plan(store, plan, segs, cfg.page_size)
    assert ex["row_pos"].tolist() == list(range(oplan.total_tokens(segs[0])))
    assert plan.sizes["cow_pages"] == 0


def test_split_options():
    """split_pages: automatic splitting and a fixed cap split the 50k request; -1 splits only
    the (tile, head) items longer than 2,048 pages (the 50k request has 3,144)."""
    cfg = CONFIGS["long50k_k32"]
    wl = Workload(cfg)
    store = meta_store(cfg, 4000)
    for c in wl.chunk_ids:
        store.store_chunk(c, n_tokens=cfg.chunk_len)
    store.store_chunk(cfg.prefix_id(0), n_tokens=cfg.prefix_len)
    for split in (0, -1, 64):
        plan = store.link_plan(wl.link_requests(), k=cfg.k, split_pages=split)
        s = plan.sizes
        assert s["split_items"] > 0
        if split == -1:
            # only tiles whose key range exceeds 2,048 pages split, each into two pieces
            assert s["split_items"] < s["work_items"]
        plan.free()


@pytest.mark.parametrize("name", ["llama3_k2", "batched_k16", "long50k_k32", "block_zipf"])
def test_automatic_key_rotation_follows_key_reuse(name):
    """rope_keys=0 rotates the keys ahead of attention exactly when the work list reads the key
    pages at least 5 times each on average: the 50k request's 50 row tiles do (25.5 reads per
    page), and so do the batched requests' 8 row tiles (5.2); the short request and the Zipf
    batch (3 row tiles per request, 2.0 and 2.2) do not."""
    cfg = CONFIGS[name]
    wl = Workload(cfg)
    B = cfg.page_size
    segs = wl.segments()
    pages_needed = sum(-(-cfg.chunk_len // B) for _ in wl.chunk_ids)
    pages_needed += len(wl.requests) * -(-cfg.prefix_len // B) + plan_private(segs, B)
    store = meta_store(cfg, pages_needed)
    for c in wl.chunk_ids:
        store.store_chunk(c, n_tokens=cfg.chunk_len)
    if cfg.prefix_len:
        for r in wl.requests:
            store.store_chunk(cfg.prefix_id(r), n_tokens=cfg.prefix_len)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, split_pages=-1)
    # reads of key pages: one per (row tile of 64 rows, KV head) and page up to the tile's last row
    G = cfg.num_q_heads // cfg.num_kv_heads
    tile = 256 // G
    reads = 0
    ex = plan.export()
    pos_map = ex["pos_map"].reshape(-1, B)
    cu_rows, cu_pages = ex["cu_rows"], ex["cu_pages"]
    for r in range(len(cu_rows) - 1):
        rp = ex["row_pos"][cu_rows[r]:cu_rows[r + 1]]
        pm = pos_map[cu_pages[r]:cu_pages[r + 1]]
        first = pm[:, 0]   # slot 0 of every page holds a token
        for t0 in range(0, len(rp), tile):
            last = rp[min(t0 + tile, len(rp)) - 1]
            reads += int(np.sum(first <= last))
    reads *= cfg.num_kv_heads
    expect = reads >= 5 * plan.sizes["pages"] * cfg.num_kv_heads
    assert (plan.sizes["rotated_pages"] > 0) == expect
    assert expect == (name in ("long50k_k32", "batched_k16"))
    plan.free()


@pytest.mark.parametrize("name,min_tiles", [("tiny", 1), ("llama3_k2", 6)])
def test_automatic_split_keeps_the_smallest_piece(name, min_tiles):
    """The automatic split never cuts a key range into pieces shorter than min_tiles key tiles
    (6 for bf16, 1 for fp32), apart from a range's last piece; above that floor it aims at the
    average load of a compute unit. Both short requests reach the floor: every item is split."""
    cfg = CONFIGS[name]
    wl = Workload(cfg)
    B = cfg.page_size
    segs = wl.segments()
    pages_needed = sum(-(-cfg.chunk_len // B) for _ in wl.chunk_ids)
    pages_needed += len(wl.requests) * -(-cfg.prefix_len // B) + plan_private(segs, B)
    store = meta_store(cfg, pages_needed)
    for c in wl.chunk_ids:
        store.store_chunk(c, n_tokens=cfg.chunk_len)
    if cfg.prefix_len:
        for r in wl.requests:
            store.store_chunk(cfg.prefix_id(r), n_tokens=cfg.prefix_len)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level)
    ppt = 64 // B
    G = cfg.num_q_heads // cfg.num_kv_heads
    ex = plan.export()
    pm = ex["pos_map"].reshape(-1, B)
    n_items = 0
    for r in range(len(ex["cu_rows"]) - 1):
        rp = ex["row_pos"][ex["cu_rows"][r]:ex["cu_rows"][r + 1]]
        first = pm[ex["cu_pages"][r]:ex["cu_pages"][r + 1], 0]
        for t0 in range(0, len(rp), 256 // G):
            need = int(np.sum(first <= rp[min(t0 + 256 // G, len(rp)) - 1]))
            n_split = -(-need // (min_tiles * ppt))
            step = -(-(-(-need // n_split)) // ppt) * ppt
            n_items += cfg.num_kv_heads * -(-need // step)
    s = plan.sizes
    assert s["work_items"] == s["split_items"] == n_items
