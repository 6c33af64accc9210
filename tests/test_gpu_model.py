"""Decoder layers around the link step on the GPU, against the fp64 oracle (needs an MI355X).

* pic_linear with each epilogue (plain, residual, SiLU(gate) * up) and pic_rmsnorm against the
  oracle's explicit-loop statements, on shapes spanning several tiles with ragged row counts;
  bound: one bfloat16 rounding of the float32 result, |gpu - oracle| <= 2^-8 |oracle| + 1e-4;
* pic_link_attend_layer on each layer of a three-layer store against the oracle link attention
  over that layer's cache;
* pic_link_forward: two layers (d_model 512, d_ff 1,024) over two linked requests, every output
  row against the oracle layers (activations held in bfloat16 at the same steps), norm-wise per
  row and element by element (tests.harness.check_hidden), with keys rotated inside attention or
  ahead, split key ranges, and LegoLink-0's compile form.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import model as omodel
from oracle import native
from oracle import plan as oplan
from tests.harness import Workload, check_hidden, check_rows, oracle_outputs, record
from workloads import MODEL_LINK, MODEL_SHAPES, gen

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", torch.bfloat16).contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def one_rounding(got, want, what):
    err = np.abs(got - want)
    bad = ~(err <= 2.0 ** -8 * np.abs(want) + 1e-4)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} off; worst {err.max():.3e}"
    record(what, float(err.max()), 0.0, got.shape[0])


SHAPES = [(300, 384, 320), (1, 128, 64), (129, 256, 576), (700, 1024, 1024)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("epilogue", [0, 1, 2])
def test_linear(m, n, k, epilogue):
    g = np.random.default_rng([m, n, k, epilogue])
    a = gen.round_bf16(g.standard_normal((m, k), dtype=np.float32))
    w = gen.round_bf16(g.standard_normal((n, k), dtype=np.float32) / np.float32(np.sqrt(k)))
    ref = native.linear(a, w)
    if epilogue == 1:
        r = gen.round_bf16(g.standard_normal((m, n), dtype=np.float32))
        want = ref + r
        got = pic.linear(dev(a), dev(w), 1, residual=dev(r))
    elif epilogue == 2:
        wg, wu = omodel.split_gate_up(w)
        want = omodel.silu(native.linear(a, wg)) * native.linear(a, wu)
        got = pic.linear(dev(a), dev(w), 2)
    else:
        want = ref
        got = pic.linear(dev(a), dev(w), 0)
    torch.cuda.synchronize()
    one_rounding(host(got), want, f"linear epilogue {epilogue}")


@pytest.mark.parametrize("epilogue", [0, 1, 2])
def test_linear_large_grid(epilogue):
    """A grid on which 256 x 256 tiles need fewer rounds of the compute units (500 rows: 2 row
    tiles, the last partial, against 4 of 128 rows; 65,536 columns: 256 column tiles) runs the
    large-tile kernel; 512 sampled output columns (for SwiGLU: their gate and up rows of W) are
    checked against the oracle."""
    m, n, k = 500, 65536, 64
    g = np.random.default_rng([m, n, k, epilogue, 1])
    a = gen.round_bf16(g.standard_normal((m, k), dtype=np.float32))
    w = gen.round_bf16(g.standard_normal((n, k), dtype=np.float32) / np.float32(np.sqrt(k)))
    n_out = n // 2 if epilogue == 2 else n
    cols = np.sort(g.choice(n_out, 512, replace=False))
    if epilogue == 2:
        wg, wu = omodel.split_gate_up(w)
        want = omodel.silu(native.linear(a, wg[cols])) * native.linear(a, wu[cols])
        got = pic.linear(dev(a), dev(w), 2)
    elif epilogue == 1:
        r = gen.round_bf16(g.standard_normal((m, n), dtype=np.float32))
        want = native.linear(a, w[cols]) + r[:, cols]
        got = pic.linear(dev(a), dev(w), 1, residual=dev(r))
    else:
        want = native.linear(a, w[cols])
        got = pic.linear(dev(a), dev(w), 0)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (m, n_out)
    one_rounding(host(got[:, torch.as_tensor(cols, device="cuda")]), want, f"linear, large grid, epilogue {epilogue}")


def test_linear_residual_in_place():
    g = np.random.default_rng(5)
    a = gen.round_bf16(g.standard_normal((200, 256), dtype=np.float32))
    w = gen.round_bf16(g.standard_normal((256, 256), dtype=np.float32) / np.float32(16))
    x = gen.round_bf16(g.standard_normal((200, 256), dtype=np.float32))
    xt = dev(x)
    pic.linear(dev(a), dev(w), 1, residual=xt, out=xt)
    torch.cuda.synchronize()
    one_rounding(host(xt), x + native.linear(a, w), "linear residual in place")


@pytest.mark.parametrize("rows,dm", [(1, 512), (37, 4096), (130, 8192), (5, 64)])
def test_rmsnorm(rows, dm):
    g = np.random.default_rng([rows, dm])
    x = gen.round_bf16(3.0 * g.standard_normal((rows, dm), dtype=np.float32))
    w = gen.round_bf16(1.0 + 0.1 * g.standard_normal(dm, dtype=np.float32))
    got = pic.rmsnorm(dev(x), dev(w), 1e-5)
    torch.cuda.synchronize()
    one_rounding(host(got), native.rmsnorm(x, w, 1e-5), "rmsnorm")


# ------------------------------------------------------------------ layered store and the forward pass
def layered_store(cfg, wl, n_layers, *, key_layout="position_free", compile_offset=0):
    """A store holding every layer's seeded K/V of the workload's chunks and prefixes."""
    ids = list(wl.chunk_ids) + ([cfg.prefix_id(r) for r in wl.requests] if cfg.prefix_len else [])
    cached = [{} for _ in range(n_layers)]
    for cid in wl.chunk_ids:
        for l in range(n_layers):
            cached[l][cid] = gen.chunk_kv(cfg, cid, l)
    if cfg.prefix_len:
        for r in wl.requests:
            for l in range(n_layers):
                cached[l][cfg.prefix_id(r)] = gen.prefix_kv(cfg, r, l)
    segs = wl.segments()
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-cached[0][c][0].shape[0] // B) for c in ids)
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    store = pic.Store(num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                      page_size=B, num_pages=stored + private + 8, dtype="bf16", rope_theta=cfg.rope_theta,
                      max_position=n_tokens + compile_offset + 1, key_layout=key_layout, compile_offset=compile_offset,
                      num_layers=n_layers)
    for cid in ids:
        k = np.stack([cached[l][cid][0] for l in range(n_layers)])
        v = np.stack([cached[l][cid][1] for l in range(n_layers)])
        if n_layers == 1:
            k, v = k[0], v[0]
        store.store_chunk(cid, dev(k), dev(v))
    return store, cached, segs


def test_link_attend_layer_reads_its_own_layer():
    cfg = MODEL_LINK
    wl = Workload(cfg)
    store, cached, segs = layered_store(cfg, wl, 3)
    plan = store.link_plan(wl.link_requests(), k=cfg.k)
    rows = wl.new_rows(segs)
    q, kn, vn = (dev(np.concatenate([r[i] for r in rows])) for i in range(3))
    ex = plan.export()
    for l in (2, 0, 1):
        out = pic.link_attend_layer(store, plan, l, q, kn, vn)
        torch.cuda.synchronize()
        want = oracle_outputs(segs, cached[l], rows, cfg.rope_theta)
        got = host(out)
        for i, (wo, _) in enumerate(want):
            check_rows(got[ex["cu_rows"][i]:ex["cu_rows"][i + 1]], wo, "bf16", f"layered store, layer {l}")
    with pytest.raises(pic.PicError):
        pic.link_attend_layer(store, plan, 3, q, kn, vn)
    plan.free()


FORWARD_CASES = {
    "inside": dict(rope_keys=1),
    "ahead": dict(rope_keys=2),
    "split": dict(rope_keys=0, split_pages=4),
    "legolink0": dict(rope_keys=0, k=0, key_layout="segment_rope", compile_offset=4),
}


@pytest.mark.parametrize("case", list(FORWARD_CASES))
def test_two_layer_forward_matches_the_oracle(case):
    opts = dict(FORWARD_CASES[case])
    key_layout = opts.pop("key_layout", "position_free")
    c_off = opts.pop("compile_offset", 0)
    kk = opts.pop("k", None)
    shape = MODEL_SHAPES["small2"]
    cfg = MODEL_LINK if kk is None else MODEL_LINK.__class__(**{**MODEL_LINK.__dict__, "k": kk})
    _say(f"two-layer forward, {case}")
    wl = Workload(cfg)
    store, cached, segs = layered_store(cfg, wl, shape.n_layers, key_layout=key_layout, compile_offset=c_off)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, **opts)
    dm = cfg.num_q_heads * cfg.head_dim
    weights = [gen.layer_weights(shape.weight_seed, l, d_model=dm, d_ff=shape.d_ff, num_q_heads=cfg.num_q_heads,
                                 num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim)
               for l in range(shape.n_layers)]
    x0 = np.concatenate([gen.hidden_states(shape.weight_seed, r, len(oplan.selected_positions(s)), dm)
                         for r, s in zip(wl.requests, segs)])
    model = pic.Model(d_model=dm, d_ff=shape.d_ff, norm_eps=shape.norm_eps,
                      layers=[{k: dev(v) for k, v in w.items()} for w in weights])
    x = dev(x0)
    pic.link_forward(store, plan, model, x)
    torch.cuda.synchronize()
    got = host(x)
    want = omodel.forward(x0, weights, segs, cached, cfg.rope_theta, num_q_heads=cfg.num_q_heads,
                          num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim, eps=shape.norm_eps,
                          key_layout=key_layout, compile_offset=c_off)
    assert np.abs(want).max() > 1.0                 # the layers move the rows by O(1)
    assert np.abs(want - omodel.round_bf16(x0)).max() > 0.5
    check_hidden(got, want, f"two-layer forward, {case}")
    _say(f"  {plan.rows} rows: max abs {np.abs(got - want).max():.3e}")
    plan.free()
