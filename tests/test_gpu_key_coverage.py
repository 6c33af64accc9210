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
from tests.harness import Workload, assert_close, gpu_store
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
    earlier decode tokens and itself, so lse = ln(n + i + 1) and the output is their values' mean."""
    cfg = CONFIGS[name]
    steps = 3
    _say(f"{name}: zero-query decode, {steps} steps, {key_layout}")
    wl = Workload(cfg)
    segs = wl.segments()
    cached = wl.cached()
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + len(segs) * 2 + 8,
                      max_position=n_tokens + steps + 1, key_layout=key_layout)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, decode=steps)
    rows = wl.new_rows(segs)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16).contiguous()
    q, kn, vn = (dev(np.concatenate([r[i] for r in rows])) for i in range(3))
    plan.upload()
    pic.link_attend(store, plan, q, kn, vn)
    n_req = len(segs)
    g = np.random.default_rng(7)
    means = []
    for a, s in enumerate(segs):
        vals = merged_values(s, cached, rows[a][2])
        means.append([vals.sum(axis=0), vals.shape[0]])
    for i in range(steps):
        dk = (0.5 * g.standard_normal((n_req, cfg.num_kv_heads, cfg.head_dim))).astype(np.float32)
        dv = (0.5 * g.standard_normal((n_req, cfg.num_kv_heads, cfg.head_dim))).astype(np.float32)
        dq = np.zeros((n_req, cfg.num_q_heads, cfg.head_dim), dtype=np.float32)
        dvb = torch.from_numpy(dv).to(torch.bfloat16).float().numpy().astype(np.float64)
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
            assert_close(got[a], want, 2e-2, 1e-2, f"{name} decode step {i} request {a} mean")
        _say(f"  step {i}: max |lse - ln n| {np.abs(got_lse - np.log([m[1] for m in means])[:, None]).max():.2e}")
    plan.free()
