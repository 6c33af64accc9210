"""Decode after link on the GPU against the fp64 oracle (needs an MI355X).

After link_attend, decode step i gives every request's token i, at the i-th
position after its last linked token, attention over the linked cache, the
tokens of the earlier steps (which the library appended to the request's
reserved decode slots) and itself. For the oracle the decode tokens are more
rows of the request's suffix (a suffix of their own when the request has
none): step i's output is the oracle's attention of the (i+1)-th added row,
computed from the pages' definition over the merged cache. Tolerance as for
the link step: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| in bf16.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

import position_independent_kv_legolink_amd as pic
from oracle import plan as oplan
from tests.harness import TOLERANCE, Workload, assert_close, check_rows, gpu_store, oracle_outputs
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


def decode_rows(cfg, n, seed, step=0):
    g = np.random.default_rng([seed, 4242, step])
    d = cfg.head_dim
    q = gen.round_bf16(g.standard_normal((n, cfg.num_q_heads, d), dtype=np.float32) * np.float32(cfg.q_scale))
    k = gen.round_bf16(g.standard_normal((n, cfg.num_kv_heads, d), dtype=np.float32) * np.float32(cfg.kv_scale))
    v = gen.round_bf16(g.standard_normal((n, cfg.num_kv_heads, d), dtype=np.float32) * np.float32(cfg.kv_scale))
    return q, k, v


def rotate_at(x, pos, theta):
    """RoPE of x [..][d] at one position, as complex multiplication (fp64)."""
    d = x.shape[-1]
    h = d // 2
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * pos * theta ** (-2.0 * np.arange(h) / d))
    return np.concatenate([z.real, z.imag], axis=-1)


def run_decode(cfg, *, n_requests=None, pos_offset=0, repeat=1, with_oracle=True, steps=1,
               key_layout="position_free", compile_offset=0, rope_keys=0):
    wl = Workload(cfg, n_requests=n_requests)
    segs = wl.segments(pos_offset=pos_offset, k=cfg.k)
    cached = wl.cached()
    rows = wl.new_rows(segs)
    B = cfg.page_size
    private = sum(p.private for s in segs for p in oplan.logical_pages(s, B))
    stored = sum(-(-v[0].shape[0] // B) for v in cached.values())
    n_tokens = max(oplan.total_tokens(s) for s in segs)
    decode_pages = len(segs) * (-(-steps // B) + 1)
    store = gpu_store(cfg, cached, num_pages=stored + private + decode_pages + 8,
                      max_position=pos_offset + n_tokens + steps + compile_offset + 1, key_layout=key_layout,
                      compile_offset=compile_offset)
    plan = store.link_plan(wl.link_requests(), k=cfg.k, block_level=cfg.block_level, pos_offset=pos_offset,
                           decode=steps, rope_keys=rope_keys)
    n = len(segs)
    assert plan.sizes["decode_items"] > 0
    if rope_keys:
        assert plan.sizes["rotated_pages"] == (plan.sizes["pages"] if rope_keys == 2 else 0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", torch.bfloat16).contiguous()
    q, kn, vn = (dev(np.concatenate([r[i] for r in rows])) for i in range(3))
    tokens = [decode_rows(cfg, n, cfg.seed, i) for i in range(steps)]
    results = []   # per step: (outputs of each repeat, lse, oracle)
    for _ in range(repeat):
        # a link call zeroes the decode slots and restarts the steps
        plan.upload()
        pic.link_attend(store, plan, q, kn, vn)
        for i, (dq, dk, dv) in enumerate(tokens):
            lse = torch.empty((n, cfg.num_q_heads), dtype=torch.float32, device="cuda")
            out = pic.link_decode(store, plan, dev(dq), dev(dk), dev(dv), lse=lse)
            torch.cuda.synchronize()
            if len(results) <= i:
                results.append([[], None, None])
            results[i][0].append(out.float().cpu().numpy())
            results[i][1] = lse.cpu().numpy()
    if with_oracle:
        for i in range(steps):
            ext = list(segs)
            for _ in range(i + 1):
                ext = [with_decode_row(s) for s in ext]
            ext_rows = [tuple(np.concatenate([r[c]] + [tokens[j][c][a:a + 1] for j in range(i + 1)])
                              for c in range(3)) for a, r in enumerate(rows)]
            sample = {a: np.array([len(oplan.selected_positions(s)) - 1]) for a, s in enumerate(ext)}
            results[i][2] = oracle_outputs(ext, cached, ext_rows, cfg.rope_theta, sample=sample,
                                           key_layout=key_layout, compile_offset=compile_offset)
    # every step wrote its token's key into the token's decode slot of the pool, in the store's
    # key form: pre-RoPE, or rotated at the token's position inside its segment
    ex = plan.export()
    kp = store.k_pool.float().cpu().numpy()
    B = cfg.page_size
    for a, sg in enumerate(segs):
        end = sg[-1].start + sg[-1].length
        seg0 = sg[-1].start if sg[-1].kind == "suffix" else end
        pm = ex["pos_map"][ex["cu_pages"][a] * B:ex["cu_pages"][a + 1] * B]
        for i in range(steps):
            slot = int(np.nonzero(pm == end + i)[0][0])
            phys = int(ex["block_table"][ex["cu_pages"][a] + slot // B])
            got = kp[phys, :, slot % B]
            want = tokens[i][1][a].astype(np.float64)
            if key_layout == "segment_rope":
                want = rotate_at(want, end + i - seg0 + compile_offset, cfg.rope_theta)
                assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-6), f"decode slot {a}/{i}"
            else:
                assert np.array_equal(got, want), f"decode slot {a}/{i}"
    with pytest.raises(pic.PicError) as e:   # every reserved step is used
        pic.link_decode(store, plan, *(dev(t) for t in tokens[-1]))
    assert e.value.status == -7
    plan.free()
    return results


def check(cfg, results, what):
    atol, rtol = TOLERANCE[cfg.dtype]
    worst = 0.0
    for step, (outs, lse, want) in enumerate(results):
        for i, (wo, wl) in enumerate(want):
            worst = max(worst, check_rows(outs[0][i:i + 1], wo, cfg.dtype, what,
                                          normwise=cfg.q_scale * cfg.kv_scale <= 1.0))
            assert_close(lse[i:i + 1], wl, atol, rtol, f"{what} step {step} request {i} lse")
        for o in outs[1:]:
            assert np.array_equal(o, outs[0]), f"{what} step {step}: run-to-run results differ"
    _say(f"{what}: {len(results)} steps, max abs err {worst:.3e}")


DECODE_EDGE = {n: c for n, c in EDGE.items() if c.get("dtype", "bf16") == "bf16"}


@pytest.mark.parametrize("name", list(DECODE_EDGE))
def test_decode_edge_cases(name):
    cfg = small_cfg(**DECODE_EDGE[name])
    _say(f"decode, edge case {name}")
    check(cfg, run_decode(cfg, steps=3), f"decode {name}")


@pytest.mark.parametrize("name", ["llama3_k2", "batched_k16", "long50k_k32", "block_zipf"])
def test_decode_workloads(name):
    cfg = CONFIGS[name]
    _say(f"decode, {name}")
    check(cfg, run_decode(cfg, repeat=2, steps=2), f"decode {name}")


@pytest.mark.parametrize("offset", [1, 100000])
def test_decode_position_offset(offset):
    cfg = small_cfg(chunk_len=64)
    _say(f"decode, pos_offset {offset}")
    check(cfg, run_decode(cfg, pos_offset=offset, steps=2), f"decode offset {offset}")


@pytest.mark.parametrize("suffix_len,steps", [(15, 4), (16, 3), (0, 18), (5, 40)])
def test_decode_steps_cross_pages(suffix_len, steps):
    """Decode tokens fill the suffix's last page, then new pages (page 16): a suffix one short of
    a page, a full page, no suffix (the tokens get pages of their own) and 40 steps."""
    cfg = small_cfg(suffix_len=suffix_len, n_requests=2, chunk_len=50)
    _say(f"decode, suffix {suffix_len}, {steps} steps")
    check(cfg, run_decode(cfg, steps=steps), f"decode suffix {suffix_len}")


@pytest.mark.parametrize("key_layout", ["position_free", "segment_rope"])
def test_decode_positions_at_the_limit(key_layout):
    """Decode tokens at the last positions below 2^22, the largest max_position a store takes."""
    cfg = small_cfg(chunk_len=64, n_requests=1)
    steps = 3
    n_tokens = oplan.total_tokens(Workload(cfg, n_requests=1).segments()[0])
    offset = (1 << 22) - n_tokens - steps - 1
    _say(f"decode, positions up to {offset + n_tokens + steps - 1}, {key_layout} keys")
    check(cfg, run_decode(cfg, pos_offset=offset, steps=steps, key_layout=key_layout),
          f"decode positions at 2^22, {key_layout} keys")


@pytest.mark.parametrize("key_layout", ["position_free", "segment_rope"])
def test_decode_does_not_depend_on_the_link_rotation_mode(key_layout):
    """Decode reads the rotated copy when the link call rotated the keys ahead of attention
    (rope_keys 2), else the pools, rotating the keys itself (rope_keys 1): both match the oracle,
    and for keys rotated inside their segment (one cos/sin row per page either way) they agree bit
    for bit. Position-free keys are rotated from one row per key ahead and from two rows (angle
    addition) in decode, which may round differently."""
    cfg = small_cfg(chunk_len=80, n_requests=3, suffix_len=7)
    _say(f"decode after both link rotation modes, {key_layout} keys")
    runs = {rk: run_decode(cfg, steps=3, key_layout=key_layout, rope_keys=rk) for rk in (1, 2)}
    for rk, res in runs.items():
        check(cfg, res, f"decode after rope_keys {rk}, {key_layout} keys")
    if key_layout == "segment_rope":
        for (o1, l1, _), (o2, l2, _) in zip(runs[1], runs[2]):
            assert np.array_equal(o1[0], o2[0]) and np.array_equal(l1, l2)
