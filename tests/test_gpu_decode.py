"""Decode after link on the GPU against the fp64 oracle (needs an MI355X).

After link_attend, every request's new token at the position after its last
linked token attends over the linked cache and itself. For the oracle that
token is one more row of the request's suffix (a suffix of one row when the
request has none): its output is the oracle's attention of that row, computed
from the pages' definition over the merged cache. Tolerance as for the link
step: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| in bf16.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import TOLERANCE, Workload, assert_close, gpu_store, oracle_outputs
from tests.test_gpu_parity import EDGE, small_cfg
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


def with_decode_row(segs):
    """The request's segments with the decode token as one more suffix row."""
    last = segs[-1]
    if last.kind == "suffix":
        return segs[:-1] + [dataclasses.replace(last, length=last.length + 1, recompute=last.recompute + 1)]
    return segs + [oplan.Segment("suffix", None, 1, last.start + last.length, 1)]


def decode_rows(cfg, n, seed):
    g = np.random.default_rng([seed, 4242])
    d = cfg.head_dim
    q = gen.round_bf16(g.standard_normal((n, cfg.num_q_heads, d), dtype=np.float32) * np.float32(cfg.q_scale))
    k = gen.round_bf16(g.standard_normal((n, cfg.num_kv_heads, d), dtype=np.float32) * np.float32(cfg.kv_scale))
    v = gen.round_bf16(g.standard_normal((n, cfg.num_kv_heads, d), dtype=np.float32) * np.float32(cfg.kv_scale))
    return q, k, v


def run_decode(cfg, *, n_requests=None, pos_offset=0, repeat=1, with_oracle=True):
    wl = Workload(cfg, n_requests=n_requests)
    segs = wl.segments(pos_offset=pos_offset, k=cfg.k)
    cached = wl.cached()
    rows = wl.new_rows(segs)
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = gpu_store(cfg, cached, num_pages=stored + private + 8, max_position=pos_offset + n_tokens + 2)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, pos_offset=pos_offset,
                           decode=True)
    n = len(segs)
    assert plan.sizes["decode_items"] > 0 and plan.sizes["rotated_pages"] == plan.sizes["pages"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16).contiguous()
    q, kn, vn = (dev(np.concatenate([r[i] for r in rows])) for i in range(3))
    plan.upload()
    pic.link_attend(store, plan, q, kn, vn)
    dq, dk, dv = decode_rows(cfg, n, cfg.seed)
    outs = []
    lse = torch.empty((n, cfg.num_q_heads), dtype=torch.float32, device="cuda")
    for _ in range(repeat):
        out = pic.link_decode(store, plan, dev(dq), dev(dk), dev(dv), lse=lse)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
    want = None
    if with_oracle:
        ext = [with_decode_row(s) for s in segs]
        ext_rows = [(np.concatenate([r[0], dq[i:i + 1]]), np.concatenate([r[1], dk[i:i + 1]]),
                     np.concatenate([r[2], dv[i:i + 1]])) for i, r in enumerate(rows)]
        sample = {i: np.array([len(oplan.selected_positions(s)) - 1]) for i, s in enumerate(ext)}
        want = oracle_outputs(ext, cached, ext_rows, cfg.rope_theta, sample=sample)
    plan.free()
    return outs, lse.cpu().numpy(), want


def check(cfg, outs, lse, want, what):
    atol, rtol = TOLERANCE[cfg.dtype]
    worst = 0.0
    for i, (wo, wl) in enumerate(want):
        worst = max(worst, assert_close(outs[0][i:i + 1], wo, atol, rtol, f"{what} request {i} out"))
        assert_close(lse[i:i + 1], wl, atol, rtol, f"{what} request {i} lse")
    _say(f"{what}: max abs err {worst:.3e}")


DECODE_EDGE = {n: c for n, c in EDGE.items() if c.get("dtype", "bf16") == "bf16"}


@pytest.mark.parametrize("name", list(DECODE_EDGE))
def test_decode_edge_cases(name):
    cfg = small_cfg(**DECODE_EDGE[name])
    _say(f"decode, edge case {name}")
    outs, lse, want = run_decode(cfg)
    check(cfg, outs, lse, want, f"decode {name}")


@pytest.mark.parametrize("name", ["llama3_k2", "batched_k16", "long50k_k32", "block_zipf"])
def test_decode_workloads(name):
    cfg = CONFIGS[name]
    _say(f"decode, {name}")
    outs, lse, want = run_decode(cfg, repeat=2)
    check(cfg, outs, lse, want, f"decode {name}")
    assert np.array_equal(outs[0], outs[1]), "run-to-run results differ"


@pytest.mark.parametrize("offset", [1, 100000])
def test_decode_position_offset(offset):
    cfg = small_cfg(chunk_len=64)
    _say(f"decode, pos_offset {offset}")
    outs, lse, want = run_decode(cfg, pos_offset=offset)
    check(cfg, outs, lse, want, f"decode offset {offset}")
