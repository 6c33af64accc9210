"""Every key is attended exactly once (needs an MI355X).

With all queries zero every score is 0, so a selected row at position p weighs each of the
p + 1 - a0 keys at positions a0 .. p equally: its log-sum-exp is ln(p + 1 - a0) and its output
is the mean of those keys' values. The link step's lse is fp32 and these sums are exact in
fp32 (whole numbers below 2^24), so it must hit ln(p + 1 - a0) within a few fp32 roundings
(|lse - ln n| <= 2e-6 + 1e-6 ln n); a key skipped or counted twice moves it by 1/n, at least
1.9e-5 at the longest request's 50,304 keys. The fp64 oracle's output tolerance, by contrast,
could not see one key tile of 64 missing out of 50,000. The outputs must equal the mean of
the merged cache's values up to bf16 rounding (fp32 store: 1e-5 + 1e-5 |mean|).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import Workload, assert_close, assert_exact_mean, gpu_store, normwise_errors, record
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


def merged_values(segs, cached, vn):
    """The merged cache's values in position order: a recomputed row's new value, else the
    cached one."""
    out = []
    r = 0
    for s in segs:
        for j in range(s.length):
            if j < s.recompute:
                out.append(vn[r])
                r += 1
            else:
                out.append(cached[s.chunk_id][1][j])
    return np.stack(out).astype(np.float64)


@pytest.mark.parametrize("name,rope_keys,key_layout,pos_offset", [
    ("tiny", 0, "position_free", 0),
    ("llama3_k2", 1, "position_free", 0),
    ("llama3_k2", 2, "segment_rope", 4097),
    ("batched_k16", 0, "position_free", 0),
    ("long50k_k32", 0, "position_free", 0),
    ("long50k_k32", 1, "segment_rope", 0),
    ("block_zipf", 0, "position_free", 0),
])
def test_zero_queries_weigh_every_key_once(name, rope_keys, key_layout, pos_offset):
    cfg = CONFIGS[name]
    _say(f"{name}: zero queries, rope_keys {rope_keys}, {key_layout}, offset {pos_offset}")
    wl = Workload(cfg)
    segs = wl.segments(pos_offset=pos_offset)
    cached = wl.cached()
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + 8, max_position=pos_offset + n_tokens + 1,
                      key_layout=key_layout)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, pos_offset=pos_offset,
                           rope_keys=rope_keys)
    rows = wl.new_rows(segs)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    kn = torch.from_numpy(np.concatenate([r[1] for r in rows])).to("cuda", tdt).contiguous()
    vn_all = np.concatenate([r[2] for r in rows])
    vn = torch.from_numpy(vn_all).to("cuda", tdt).contiguous()
    q = torch.zeros((plan.rows, cfg.num_q_heads, cfg.head_dim), dtype=tdt, device="cuda")
    plan.upload()
    lse = torch.empty((plan.rows, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    out = pic.link_attend(store, plan, q, kn, vn, lse=lse)
    torch.cuda.synchronize()
    got_lse = lse.cpu().numpy().astype(np.float64)
    got = out.float().cpu().numpy()
    ex = plan.export()
    row_pos = ex["row_pos"].astype(np.int64)
    n = (row_pos - pos_offset + 1).astype(np.float64)
    want_lse = np.broadcast_to(np.log(n)[:, None], got_lse.shape)
    err = np.abs(got_lse - want_lse)
    bad = err > 2e-6 + 1e-6 * want_lse
    assert not bad.any(), (f"lse off for {int(bad.sum())} of {bad.size}; worst {err.max():.3e} at "
                           f"{np.argwhere(bad)[0].tolist()}")
    _say(f"  lse: max |lse - ln n| {err.max():.2e} over {plan.rows} rows")
    # outputs: the running mean of the merged values, checked on a few rows per request
    atol, rtol = (2e-2, 1e-2) if cfg.dtype == "bf16" else (1e-5, 1e-5)
    G = cfg.num_q_heads // cfg.num_kv_heads
    g = np.random.default_rng(1)
    r_base = 0
    for i, s in enumerate(segs):
        R = len(oplan.selected_positions(s))
        vals = merged_values(s, cached, vn_all[r_base:r_base + R])          # [tokens][Hkv][d]
        csum = np.cumsum(vals, axis=0)
        pick = sorted({0, R - 1} | set(int(x) for x in g.integers(0, R, size=6)))
        for r in pick:
            p = int(row_pos[r_base + r]) - pos_offset
            mean = csum[p] / (p + 1)                                          # [Hkv][d]
            want = np.repeat(mean, G, axis=0)                                  # [Hq][d]
            assert_close(got[r_base + r], want, atol, rtol, f"{name} request {i} row {r} mean")
        r_base += R


@pytest.mark.parametrize("name,key_layout", [("llama3_k2", "position_free"), ("batched_k16", "segment_rope"),
                                             ("long50k_k32", "position_free"), ("block_zipf", "position_free")])
def test_zero_queries_decode_weighs_every_key_once(name, key_layout):
    """Decode step i of a request with n linked tokens: its token weighs the n linked keys, the i
    earlier decode tokens and itself, so lse = ln(n + i + 1) and the output is their values' mean.
    Every value (cached, recomputed and decoded) is a structured, bfloat16-exact one, so the mean
    is O(1) and checked to one bfloat16 rounding (tests.harness.assert_exact_mean)."""
    cfg = CONFIGS[name]
    steps = 3
    _say(f"{name}: zero-query decode, {steps} steps, {key_layout}")
    wl = Workload(cfg)
    segs = wl.segments()
    cached = structured_cache(cfg, wl)
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + len(segs) * 2 + 8,
                      max_position=n_tokens + steps + 1, key_layout=key_layout)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, decode=steps)
    rows = wl.new_rows(segs)
    vn_rows = [gen.structured_values(r, len(oplan.selected_positions(s)), cfg.num_kv_heads, cfg.head_dim, new=True)
               for r, s in zip(wl.requests, segs)]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16).contiguous()
    q, kn = (dev(np.concatenate([r[i] for r in rows])) for i in range(2))
    vn = dev(np.concatenate(vn_rows))
    plan.upload()
    pic.link_attend(store, plan, q, kn, vn)
    n_req = len(segs)
    g = np.random.default_rng(7)
    means = []
    for a, s in enumerate(segs):
        vals = merged_values(s, cached, vn_rows[a])
        means.append([vals.sum(axis=0), vals.shape[0]])
    worst = 0.0
    for i in range(steps):
        dk = (0.5 * g.standard_normal((n_req, cfg.num_kv_heads, cfg.head_dim))).astype(np.float32)
        dv = gen.structured_values(500 + i, n_req, cfg.num_kv_heads, cfg.head_dim)
        dq = np.zeros((n_req, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
        dvb = dv.astype(np.float64)
        lse = torch.empty((n_req, cfg.num_q_heads), dtype=torch.float32, device="cuda")
        out = pic.link_decode(store, plan, dev(dq), dev(dk), dev(dv), lse=lse)
        torch.cuda.synchronize()
        got_lse = lse.cpu().numpy().astype(np.float64)
        got = out.float().cpu().numpy()
        G = cfg.num_q_heads // cfg.num_kv_heads
        for a, s in enumerate(segs):
            means[a][0] = means[a][0] + dvb[a]
            means[a][1] += 1
            cnt = means[a][1]
            assert cnt == oplan.total_tokens(s) + i + 1
            want_lse = np.log(cnt)
            err = np.abs(got_lse[a] - want_lse)
            assert np.all(err <= 2e-6 + 1e-6 * want_lse), (a, i, float(err.max()))
            want = np.repeat(means[a][0] / cnt, G, axis=0)
            worst = max(worst, assert_exact_mean(got[a], want, f"{name} decode step {i} request {a} mean"))
        _say(f"  step {i}: max |lse - ln n| {np.abs(got_lse - np.log([m[1] for m in means])[:, None]).max():.2e}")
    record(f"zero q, structured V: {name} decode", worst, 0.0, n_req * steps)
    plan.free()


# ------------------------------------------------------------------ values with an O(1) mean
# With zero queries every weight is exactly 1 (exp2 of 0) and the output is the mean of the
# values of every key at or before the row. The values of workloads.gen.structured_values are
# multiples of 1/16 that bfloat16 holds exactly and whose float32 sums stay exact, so the link
# step's output is that mean up to the float32 normalisation and the final bfloat16 rounding:
# |gpu - mean| <= 2^-9 |mean| + 1e-5 (split ranges add a float32 merge). The test bound is
# 2^-8 |mean| + 1e-4 (tests.harness.assert_exact_mean). The means are O(1) and differ between heads and dimensions by at least
# 1/16 and between sets of segments by O(1/16), so a missing value vector, a wrong KV head or
# dimension order, or value pages read from another chunk's pages move them far outside it, at
# any key range. (The element-wise tolerance of the benchmark spec, 2e-2 + 1e-2 |x|, is larger than the
# outputs of random values at long key ranges, which average to about 0.01.)
def _limit_cfg():
    from tests.test_gpu_parity import small_cfg
    # the row tile of chunks 62 and 63 reads exactly 2,048 pages (split_pages = -1)
    return small_cfg(chunk_len=512, chunks_per_request=64, pool_size=64, k=32, prefix_len=0, suffix_len=16,
                     n_requests=1)


STRUCTURED_CASES = {
    "long50k_k32 ahead": (lambda: CONFIGS["long50k_k32"], dict(rope_keys=2), "position_free"),
    "long50k_k32 inside": (lambda: CONFIGS["long50k_k32"], dict(rope_keys=1), "position_free"),
    "long50k_k32 compiled from 0": (lambda: CONFIGS["long50k_k32"], dict(rope_keys=0), "segment_rope"),
    "batched_k16": (lambda: CONFIGS["batched_k16"], dict(rope_keys=0), "position_free"),
    "block_zipf": (lambda: CONFIGS["block_zipf"], dict(rope_keys=0), "position_free"),
    "2,048-page item inside": (_limit_cfg, dict(rope_keys=1, split_pages=-1), "position_free"),
    "2,048-page item ahead": (_limit_cfg, dict(rope_keys=2, split_pages=-1), "position_free"),
    "llama3_k2 split": (lambda: CONFIGS["llama3_k2"], dict(rope_keys=0, split_pages=4), "position_free"),
}


def structured_cache(cfg, wl):
    """The workload's cached keys with structured values in place of the random ones."""
    cached = wl.cached()
    return {cid: (k, gen.structured_values(cid, k.shape[0], cfg.num_kv_heads, cfg.head_dim))
            for cid, (k, v) in cached.items()}


@pytest.mark.parametrize("case", list(STRUCTURED_CASES))
def test_zero_queries_structured_values_every_row(case):
    make, opts, key_layout = STRUCTURED_CASES[case]
    cfg = make()
    _say(f"{case}: zero queries, structured values, every row")
    wl = Workload(cfg)
    segs = wl.segments()
    cached = structured_cache(cfg, wl)
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + 8, max_position=n_tokens + 1, key_layout=key_layout)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, **opts)
    if "2,048" in case:
        assert plan.sizes["split_items"] == 2 * cfg.num_kv_heads
    rows = wl.new_rows(segs)
    vn_rows = [gen.structured_values(r, len(oplan.selected_positions(s)), cfg.num_kv_heads, cfg.head_dim, new=True)
               for r, s in zip(wl.requests, segs)]
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    kn = torch.from_numpy(np.concatenate([r[1] for r in rows])).to("cuda", tdt).contiguous()
    vn = torch.from_numpy(np.concatenate(vn_rows)).to("cuda", tdt).contiguous()
    q = torch.zeros((plan.rows, cfg.num_q_heads, cfg.head_dim), dtype=tdt, device="cuda")
    lse = torch.empty((plan.rows, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    out = pic.link_attend(store, plan, q, kn, vn, lse=lse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    ex = plan.export()
    G = cfg.num_q_heads // cfg.num_kv_heads
    worst = 0.0
    worst_nw = 0.0
    r_base = 0
    for i, s in enumerate(segs):
        R = len(oplan.selected_positions(s))
        vals = merged_values(s, cached, vn_rows[i])                         # [tokens][Hkv][d], exact
        csum = np.cumsum(vals, axis=0)
        p = ex["row_pos"][r_base:r_base + R].astype(np.int64)             # offset 0: index = position
        want = np.repeat(csum[p] / (p + 1)[:, None, None], G, axis=1)       # [R][Hq][d]
        worst = max(worst, assert_exact_mean(got[r_base:r_base + R], want, f"{case} request {i}"))
        worst_nw = max(worst_nw, float(normwise_errors(got[r_base:r_base + R], want).max()))
        n = (p + 1).astype(np.float64)
        lerr = np.abs(got_lse[r_base:r_base + R] - np.log(n)[:, None])
        assert np.all(lerr <= 2e-6 + 1e-6 * np.log(n)[:, None]), (case, i, float(lerr.max()))
        r_base += R
    record(f"zero q, structured V: {case}", worst, worst_nw, plan.rows)
    _say(f"  every row of {plan.rows}: max |gpu - mean| {worst:.2e}, worst norm-wise {worst_nw:.2e}")
    plan.free()
