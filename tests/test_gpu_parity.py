"""GPU parity of the link step against the fp64 oracle (needs an MI355X).

Every case runs store_chunk -> link_plan -> plan upload -> link_attend through
the C ABI and compares the outputs with the oracle element by element:
bf16 within |gpu - oracle| <= 2e-2 + 1e-2 |oracle|, fp32 within 1e-5 + 1e-5
|oracle|. Small cases compare every row; the full-size workloads compare
sampled rows (first, last, longest and seeded random ones), which the oracle
computes one by one over the complete merged cache.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import (RESULTS, TOLERANCE, Workload, assert_close, check_rows, compare_plan, gpu_store,
                           oracle_outputs)
from workloads import CONFIGS, gen

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


def run_workload(cfg, *, n_requests=None, sample_rows=None, pos_offset=0, split_pages=0, k=None,
                 recompute_all=False, seed=0, check_plan=True, repeat=1, lse=True, num_pages=None, rope_keys=0,
                 with_oracle=True, key_layout="position_free", compile_offset=0):
    """Link a config's requests on the GPU; return (gpu outs, oracle outs or None, extras)."""
    wl = Workload(cfg, n_requests=n_requests)
    kk = cfg.k if k is None else k
    segs = wl.segments(pos_offset=pos_offset, recompute_all=recompute_all, k=kk)
    cached = wl.cached()
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=num_pages or (stored + private + 8),
                      max_position=pos_offset + n_tokens + compile_offset + 1, key_layout=key_layout,
                      compile_offset=compile_offset)
    plan = store.link_plan(wl.link_requests(), k=kk, block_level=cfg.block_level, pos_offset=pos_offset,
                           recompute_all=recompute_all, split_pages=split_pages, rope_keys=rope_keys)
    if check_plan:
        compare_plan(store, plan, segs, B)
    rows = wl.new_rows(segs)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.from_numpy(np.concatenate([r[0] for r in rows])).to("cuda", tdt).contiguous()
    kn = torch.from_numpy(np.concatenate([r[1] for r in rows])).to("cuda", tdt).contiguous()
    vn = torch.from_numpy(np.concatenate([r[2] for r in rows])).to("cuda", tdt).contiguous()
    plan.upload()
    outs = []
    lse_t = torch.empty((plan.rows, cfg.num_q_heads), dtype=torch.float32, device="cuda") if lse else None
    for _ in range(repeat):
        # every launch writes into NaN: an item a launch skipped would show
        out = torch.full((plan.rows, cfg.num_q_heads, cfg.head_dim), float("nan"), dtype=tdt, device="cuda")
        if lse_t is not None:
            lse_t.fill_(float("nan"))
        out = pic.link_attend(store, plan, q, kn, vn, out=out, lse=lse_t)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
    got_lse = lse_t.cpu().numpy() if lse else None
    ex = plan.export()
    sample = None
    if sample_rows is not None:
        sample = {}
        g = np.random.default_rng(seed)
        for i, s in enumerate(segs):
            R = len(oplan.selected_positions(s))
            pick = {0, R - 1, R // 2} | set(int(x) for x in g.integers(0, R, size=max(0, sample_rows - 3)))
            sample[i] = np.array(sorted(x for x in pick if 0 <= x < R), dtype=np.int64)
    want = (oracle_outputs(segs, cached, rows, cfg.rope_theta, sample=sample, key_layout=key_layout,
                           compile_offset=compile_offset) if with_oracle else None)
    extras = dict(store=store, plan=plan, export=ex, segs=segs, cached=cached, rows=rows, sample=sample,
                  lse=got_lse, outs=outs, link_requests=wl.link_requests())
    return outs[0], want, extras


def check(cfg, got, want, extras, what, normwise=None):
    """Element-wise tolerance on outputs and lse, and the norm-wise bound per (row, head) on the
    outputs. The norm-wise bound assumes score spreads of the Llama-shaped inputs
    (q_scale * kv_scale <= 1); other inputs record their norm-wise error without the bound."""
    atol, rtol = TOLERANCE[cfg.dtype]
    if normwise is None:
        normwise = cfg.q_scale * cfg.kv_scale <= 1.0
    ex = extras["export"]
    worst = 0.0
    for i, (wo, wl) in enumerate(want):
        r0 = ex["cu_rows"][i]
        idx = np.arange(wo.shape[0]) if extras["sample"] is None else extras["sample"][i]
        g = got[r0 + idx]
        worst = max(worst, check_rows(g, wo, cfg.dtype, what, normwise=normwise))
        if extras["lse"] is not None:
            assert_close(extras["lse"][r0 + idx], wl, atol, rtol, f"{what} request {i} lse")
    nw = RESULTS[what][1] if what in RESULTS else 0.0
    _say(f"{what}: max abs err {worst:.3e}, worst norm-wise {nw:.3e}")
    return worst


# ------------------------------------------------------------------ the five workloads
def test_tiny_fp32_all_rows():
    cfg = CONFIGS["tiny"]
    got, want, ex = run_workload(cfg)
    check(cfg, got, want, ex, "tiny")


def test_llama3_k2_all_rows():
    cfg = CONFIGS["llama3_k2"]
    got, want, ex = run_workload(cfg)
    check(cfg, got, want, ex, "llama3_k2")


def test_batched_k16_sampled():
    cfg = CONFIGS["batched_k16"]
    got, want, ex = run_workload(cfg, sample_rows=24)
    check(cfg, got, want, ex, "batched_k16")


def test_long50k_k32_sampled():
    cfg = CONFIGS["long50k_k32"]
    got, want, ex = run_workload(cfg, sample_rows=40, repeat=2)
    # its 50 row tiles per KV head read every key page many times: keys are rotated ahead
    assert ex["plan"].sizes["rotated_pages"] == ex["plan"].sizes["pages"]
    check(cfg, got, want, ex, "long50k_k32")
    assert np.array_equal(ex["outs"][0], ex["outs"][1]), "run-to-run results differ"


def test_block_zipf_sampled():
    cfg = CONFIGS["block_zipf"]
    got, want, ex = run_workload(cfg, sample_rows=6)
    check(cfg, got, want, ex, "block_zipf")


# ------------------------------------------------------------------ edge cases
def small_cfg(**over):
    base = dict(name="edge", description="edge case", num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16",
                rope_theta=5e5, page_size=16, k=3, block_level=False, prefix_len=21, chunk_len=70,
                chunks_per_request=5, suffix_len=37, n_requests=2, pool_size=6, pool_draw="uniform",
                q_scale=1.0, kv_scale=0.5, seed=77)
    base.update(over)
    return CONFIGS["tiny"].__class__(**base)


EDGE = {
    "ragged_bf16": dict(),
    "ragged_f32": dict(dtype="f32", kv_scale=1.0),
    "k0_link_half": dict(k=0),
    "k_beyond_chunk": dict(k=90),
    "block_page32": dict(block_level=True, page_size=32),
    "page64_k40": dict(page_size=64, k=40),
    "no_prefix_no_suffix": dict(prefix_len=0, suffix_len=0, k=5),
    "suffix_only": dict(chunks_per_request=0, prefix_len=0, suffix_len=300),
    "d64_bf16_g1": dict(head_dim=64, num_q_heads=4, num_kv_heads=4),
    "d64_f32_g8": dict(head_dim=64, num_q_heads=8, num_kv_heads=1, dtype="f32", kv_scale=1.0),
    "g2_many_requests": dict(num_q_heads=4, num_kv_heads=2, n_requests=5, chunk_len=33),
    "hkv8_xcd_buckets": dict(num_q_heads=32, num_kv_heads=8, chunk_len=140, k=20),
    "g8_bf16": dict(num_q_heads=16, num_kv_heads=2),
    "one_token_chunks": dict(chunk_len=1, chunks_per_request=40, pool_size=60, k=1, prefix_len=3, suffix_len=5),
    "prefix_and_suffix_only": dict(prefix_len=300, chunks_per_request=0, suffix_len=7),
    "single_head_d64": dict(num_q_heads=1, num_kv_heads=1, head_dim=64),
    "page32_d64_k33": dict(page_size=32, head_dim=64, num_q_heads=4, num_kv_heads=2, k=33, chunk_len=90),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases_all_rows(name):
    cfg = small_cfg(**EDGE[name])
    _say(f"edge case {name}")
    got, want, ex = run_workload(cfg)
    check(cfg, got, want, ex, name)


def test_large_scores():
    """Scores spread over several units of log2(e): the running maximum moves often, and the
    exponentials of stale maxima overflow fp32 on some tiles, so the exact softmax path runs."""
    cfg = small_cfg(q_scale=2.0, kv_scale=1.0, chunk_len=150, k=12)
    got, want, ex = run_workload(cfg)
    check(cfg, got, want, ex, "large scores")


def test_growing_scores():
    """Keys of later chunks scaled up: every chunk brings a new row maximum."""
    cfg = small_cfg(chunk_len=200, chunks_per_request=6, k=8, n_requests=1, prefix_len=0)
    wl = Workload(cfg)
    order = {c: i for i, c in enumerate(wl.draws[0])}
    cached = {c: (k * np.float32(1.0 + 0.6 * order[c]), v) for c, (k, v) in wl.cached().items()}
    cached = {c: (gen.round_bf16(k), v) for c, (k, v) in cached.items()}
    segs = wl.segments(k=cfg.k)
    store = gpu_store(cfg, cached, num_pages=400, max_position=4096)
    plan = store.link_plan(wl.link_requests(), k=cfg.k)
    rows = wl.new_rows(segs)
    q, kn, vn = (torch.from_numpy(np.concatenate([r[i] for r in rows])).to("cuda", torch.bfloat16).contiguous()
                 for i in range(3))
    plan.upload()
    lse_t = torch.empty((plan.rows, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    out = pic.link_attend(store, plan, q, kn, vn, lse=lse_t)
    torch.cuda.synchronize()
    want = oracle_outputs(segs, cached, rows, cfg.rope_theta)
    # keys of the later chunks are scaled up to 4x: score spreads beyond the norm-wise bound's premise
    check(cfg, out.float().cpu().numpy(), want,
          dict(export=plan.export(), sample=None, lse=lse_t.cpu().numpy()), "growing scores", normwise=False)


@pytest.mark.parametrize("split", [-1, 4, 12])
def test_split_and_merge(split):
    cfg = small_cfg(chunk_len=300, chunks_per_request=6, k=20, n_requests=2)
    _say(f"split_pages {split}")
    got, want, ex = run_workload(cfg, split_pages=split)
    if split > 0:
        assert ex["plan"].sizes["split_items"] > 0
    check(cfg, got, want, ex, f"split {split}")


@pytest.mark.parametrize("offset", [1, 4097, 100000])
def test_position_offset(offset):
    cfg = small_cfg(chunk_len=64)
    _say(f"pos_offset {offset}")
    got, want, ex = run_workload(cfg, pos_offset=offset)
    check(cfg, got, want, ex, f"offset {offset}")


def test_dense_recompute_all():
    cfg = small_cfg(chunk_len=100, chunks_per_request=3, n_requests=1)
    got, want, ex = run_workload(cfg, recompute_all=True)
    assert ex["plan"].sizes["cow_pages"] == 0
    check(cfg, got, want, ex, "recompute_all")


def test_empty_plan_is_a_noop():
    cfg = small_cfg(prefix_len=0, suffix_len=0, k=0, n_requests=1)
    wl = Workload(cfg)
    store = gpu_store(cfg, wl.cached(), num_pages=200, max_position=4096)
    plan = store.link_plan(wl.link_requests(), k=0)
    assert plan.rows == 0
    plan.upload()
    z = torch.empty((0, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, cfg.num_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    out = pic.link_attend(store, plan, z, zk, zk)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


@pytest.mark.parametrize("rope_keys", [1, 2])
def test_scatter_writes_private_pages_exactly(rope_keys):
    """Private pages hold new rows, copied cached rows and zero padding, byte for byte, with the
    keys rotated inside attention or ahead of it."""
    cfg = small_cfg(k=3, chunk_len=45)
    got, want, ex = run_workload(cfg, rope_keys=rope_keys)
    check(cfg, got, want, ex, f"scatter rope_keys {rope_keys}")
    store, segs, rows, cached = ex["store"], ex["segs"], ex["rows"], ex["cached"]
    exp_ = ex["export"]
    B = cfg.page_size
    kp = store.k_pool.float().cpu().numpy()
    vp = store.v_pool.float().cpu().numpy()
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
            want_k = np.zeros((cfg.num_kv_heads, B, cfg.head_dim), np.float32)
            want_v = np.zeros_like(want_k)
            for slot in range(pg.valid):
                j = pg.index * B + slot
                if j < seg.recompute:
                    r = row_of_seg[pg.segment] + j
                    want_k[:, slot], want_v[:, slot] = kn[r], vn[r]
                else:
                    want_k[:, slot] = cached[seg.chunk_id][0][j]
                    want_v[:, slot] = cached[seg.chunk_id][1][j]
            assert np.array_equal(kp[phys], want_k) and np.array_equal(vp[phys], want_v)


def test_page_placement_does_not_change_results():
    """Permuting the physical pages of every chunk gives bitwise identical output."""
    cfg = small_cfg(n_requests=1)
    a, _, ex_a = run_workload(cfg, check_plan=False)
    # a store with a different physical layout: occupy some pages first
    wl = Workload(cfg, n_requests=1)
    cached = wl.cached()
    store = pic.Store(num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                      page_size=cfg.page_size, num_pages=400, dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                      max_position=4096)
    dummy = torch.zeros((40, cfg.num_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    for j in range(7):
        store.store_chunk(9000 + j, dummy, dummy)
    for cid in reversed(list(cached)):
        k, v = cached[cid]
        store.store_chunk(cid, torch.from_numpy(k).to("cuda", torch.bfloat16).contiguous(),
                          torch.from_numpy(v).to("cuda", torch.bfloat16).contiguous())
    for j in range(0, 7, 2):
        store.release(9000 + j)
    plan = store.link_plan(wl.link_requests(), k=cfg.k)
    assert not np.array_equal(plan.export()["block_table"], ex_a["export"]["block_table"])
    rows = ex_a["rows"]
    q = torch.from_numpy(rows[0][0]).to("cuda", torch.bfloat16).contiguous()
    kn = torch.from_numpy(rows[0][1]).to("cuda", torch.bfloat16).contiguous()
    vn = torch.from_numpy(rows[0][2]).to("cuda", torch.bfloat16).contiguous()
    plan.upload()
    b = pic.link_attend(store, plan, q, kn, vn).float().cpu().numpy()
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ keys rotated ahead of attention
ROTATED = {n: c for n, c in EDGE.items() if c.get("dtype", "bf16") == "bf16"}


@pytest.mark.parametrize("name", list(ROTATED))
def test_edge_cases_rotated_keys(name):
    cfg = small_cfg(**ROTATED[name])
    _say(f"edge case {name}, keys rotated ahead of attention")
    got, want, ex = run_workload(cfg, rope_keys=2)
    assert ex["plan"].sizes["rotated_pages"] == ex["plan"].sizes["pages"]
    check(cfg, got, want, ex, f"{name} rotated keys")


@pytest.mark.parametrize("name,sample", [("llama3_k2", None), ("batched_k16", 12), ("block_zipf", 4)])
def test_workloads_rotated_keys(name, sample):
    cfg = CONFIGS[name]
    _say(f"{name}, keys rotated ahead of attention")
    got, want, ex = run_workload(cfg, sample_rows=sample, rope_keys=2)
    assert ex["plan"].sizes["rotated_pages"] == ex["plan"].sizes["pages"]
    check(cfg, got, want, ex, f"{name} rotated keys")


ROTATION_CASES = {
    "llama3_k2": lambda: (CONFIGS["llama3_k2"], {}),
    "long50k_k32": lambda: (CONFIGS["long50k_k32"], {}),
    "split_offset": lambda: (small_cfg(chunk_len=300, chunks_per_request=6, k=20), dict(split_pages=4, pos_offset=4097)),
    "page64_d64": lambda: (small_cfg(page_size=64, head_dim=64, num_q_heads=8, num_kv_heads=2, k=40), {}),
}


@pytest.mark.parametrize("case", list(ROTATION_CASES))
def test_rotation_modes_are_bit_identical(case):
    """Keys rotated once ahead of attention and keys rotated inside attention use the same table
    values and arithmetic, so outputs and log-sum-exps agree bit for bit."""
    cfg, kw = ROTATION_CASES[case]()
    _say(f"rotation modes, {case}")
    a, _, ex_a = run_workload(cfg, rope_keys=1, with_oracle=False, check_plan=False, **kw)
    b, _, ex_b = run_workload(cfg, rope_keys=2, with_oracle=False, check_plan=False, **kw)
    assert ex_a["plan"].sizes["rotated_pages"] == 0 and ex_b["plan"].sizes["rotated_pages"] > 0
    assert np.array_equal(a, b)
    assert np.array_equal(ex_a["lse"], ex_b["lse"])


def test_back_to_back_uploads_share_one_workspace():
    """Plan uploads are stream-ordered: uploading a plan into the workspace that a queued link call
    still reads does not disturb that call, and the store's staging buffer grows for a plan whose
    tables exceed it. Outputs match synchronised runs with their own workspaces bit for bit."""
    cfg = small_cfg(n_requests=24, chunks_per_request=24, chunk_len=100, k=4, pool_size=30)
    wl_b = Workload(cfg)
    wl_s = Workload(cfg, n_requests=1)
    cached = wl_b.cached()
    B = cfg.page_size
    jobs = []
    for wl in (wl_s, wl_b):
        segs = wl.segments(k=cfg.k)
        rows = wl.new_rows(segs)
        jobs.append((wl, segs, rows))
    private = sum(p.private for _, segs, _ in jobs for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for _, segs, _ in jobs for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + 8, max_position=n_tokens + 1)
    plans, tensors = [], []
    for wl, segs, rows in jobs:
        plans.append(store.link_plan(wl.link_requests(), k=cfg.k, split_pages=-1))
        tensors.append([torch.from_numpy(np.concatenate([r[i] for r in rows])).to("cuda", torch.bfloat16).contiguous()
                        for i in range(3)])
    assert plans[1].sizes["workspace_bytes"] > 1 << 16
    refs = []
    for plan, (q, kn, vn) in zip(plans, tensors):
        plan.upload()
        refs.append(pic.link_attend(store, plan, q, kn, vn).float().cpu().numpy())
    torch.cuda.synchronize()
    ws = torch.empty(max(p.sizes["workspace_bytes"] for p in plans), dtype=torch.uint8, device="cuda")
    outs = []
    for i in (0, 1, 0, 1):
        plans[i].upload(ws)
        outs.append((i, pic.link_attend(store, plans[i], *tensors[i])))
    torch.cuda.synchronize()
    for i, o in outs:
        assert np.array_equal(o.float().cpu().numpy(), refs[i])
    for p in plans:
        p.free()


# ------------------------------------------------------------------ the kernels' size limits
@pytest.mark.parametrize("key_layout", ["position_free", "segment_rope"])
@pytest.mark.parametrize("rope_keys", [1, 2])
def test_item_at_the_page_table_limit(rope_keys, key_layout):
    """64 chunks of 512 tokens, LegoLink-32, no prefix: the row tile of chunks 62 and 63 reads
    exactly 2,048 pages, the most one work item's LDS page table holds; the suffix tile reads
    2,049 and is split in two (for each KV head)."""
    cfg = small_cfg(chunk_len=512, chunks_per_request=64, pool_size=64, k=32, prefix_len=0, suffix_len=16,
                    n_requests=1)
    _say(f"2,048-page work item, rope_keys {rope_keys}, {key_layout} keys")
    got, want, ex = run_workload(cfg, split_pages=-1, sample_rows=24, rope_keys=rope_keys, check_plan=False,
                                 key_layout=key_layout)
    assert ex["plan"].sizes["split_items"] == 2 * cfg.num_kv_heads   # the suffix tile of each KV head
    rows = np.concatenate([ex["sample"][0], [2047, 2048, 2063]])   # rows of the last chunk pair and the suffix
    ex["sample"] = {0: np.unique(rows)}
    want = oracle_outputs(ex["segs"], ex["cached"], ex["rows"], cfg.rope_theta, sample=ex["sample"],
                          key_layout=key_layout)
    check(cfg, got, want, ex, f"2,048-page item, rope_keys {rope_keys}, {key_layout} keys")


@pytest.mark.parametrize("key_layout", ["position_free", "segment_rope"])
@pytest.mark.parametrize("rope_keys", [1, 2])
def test_positions_at_the_limit(rope_keys, key_layout):
    """The request's last positions end just below 2^22, the largest max_position a store takes
    (positions are packed with a page's valid count, and cos/sin rows addressed with 32-bit
    offsets, up to there)."""
    cfg = small_cfg(chunk_len=64, n_requests=1)
    wl = Workload(cfg, n_requests=1)
    n_tokens = oplan.total_tokens(wl.segments()[0])
    offset = (1 << 22) - n_tokens - 1
    _say(f"positions up to {offset + n_tokens - 1}, rope_keys {rope_keys}, {key_layout} keys")
    got, want, ex = run_workload(cfg, pos_offset=offset, rope_keys=rope_keys, key_layout=key_layout)
    check(cfg, got, want, ex, f"positions at 2^22, rope_keys {rope_keys}, {key_layout} keys")


def test_host_tensors_are_refused_before_any_library_call():
    """A host tensor where the kernels expect device memory is refused by the binding (a kernel
    would otherwise be handed a host address)."""
    cfg = small_cfg(k=3, chunk_len=45)
    wl = Workload(cfg, n_requests=1)
    cached = wl.cached()
    store = gpu_store(cfg, cached, num_pages=64, max_position=1024)
    k, v = next(iter(cached.values()))
    host = torch.from_numpy(np.ascontiguousarray(k)).to(torch.bfloat16)
    with pytest.raises(ValueError):
        store.store_chunk(10 ** 6, host, host)
    plan = store.link_plan(wl.link_requests(), k=cfg.k)
    with pytest.raises(ValueError):
        plan.upload(torch.empty(plan.sizes["workspace_bytes"], dtype=torch.uint8))
    plan.upload()
    R = plan.rows
    dev = torch.zeros((R, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((R, cfg.num_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        pic.link_attend(store, plan, dev, kv, kv, out=torch.empty_like(dev, device="cpu"))
    with pytest.raises(ValueError):
        pic.link_attend(store, plan, dev, kv, kv, lse=torch.empty((R, cfg.num_q_heads), dtype=torch.float32))
    with pytest.raises(ValueError):
        pic.link_attend(store, plan, dev.cpu(), kv, kv)
    torch.cuda.synchronize()
    plan.free()
