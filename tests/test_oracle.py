"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

* closed-form scores of one- and two-frequency rotations (sign, pairing, scale);
* the dense special case (one chunk, every row recomputed) against torch's
  scaled_dot_product_attention in fp64 over tensors rotated with complex
  multiplication;
* shift invariance of RoPE scores (relative-position identity);
* equality with the brute-force dense-matrix statement on tiny ragged inputs;
* independence of a first chunk's recomputed rows from every cached value;
* GQA: repeating each KV head reproduces the grouped result bit for bit;
* closed-form plan sizes of the five workloads and the per-token selection rule.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import link as olink
from oracle import native
from oracle import plan as oplan
from tests import brute
from workloads import CONFIGS, gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def tiny_request(seed, *, hq=4, hkv=2, d=8, prefix_len=5, chunk_lens=(7, 20, 3),
                 suffix_len=6, k=2, block_level=False, page_size=4, pos_offset=0,
                 recompute_all=False, theta=1e4):
    g = np.random.default_rng(seed)
    prefix = None
    cached = {}
    if prefix_len:
        prefix = (g.standard_normal((prefix_len, hkv, d)), g.standard_normal((prefix_len, hkv, d)))
        cached[1000] = prefix
    chunks = []
    for i, L in enumerate(chunk_lens):
        c = (g.standard_normal((L, hkv, d)) * 0.7, g.standard_normal((L, hkv, d)))
        chunks.append(c)
        cached[i] = c
    segs = oplan.link_segments(prefix_id=1000 if prefix_len else None, prefix_len=prefix_len,
                               chunk_ids=list(range(len(chunk_lens))), chunk_lens=list(chunk_lens),
                               suffix_len=suffix_len, k=k, block_level=block_level,
                               page_size=page_size, pos_offset=pos_offset,
                               recompute_all=recompute_all)
    R = len(oplan.selected_positions(segs))
    qn = g.standard_normal((R, hq, d))
    kn = g.standard_normal((R, hkv, d)) * 0.7
    vn = g.standard_normal((R, hkv, d))
    return dict(segs=segs, cached=cached, prefix=prefix, chunks=chunks, q=qn, k=kn, v=vn,
                theta=theta, suffix_len=suffix_len, kk=k, block_level=block_level,
                page_size=page_size, pos_offset=pos_offset, recompute_all=recompute_all)


def run_oracle(req, **over):
    r = dict(req, **over)
    return olink.link_attention(r["segs"], r["cached"], r["q"], r["k"], r["v"], r["theta"])


def run_brute(req):
    return brute.link_request(prefix=req["prefix"], chunks=req["chunks"], suffix_len=req["suffix_len"],
                              k=req["kk"], block_level=req["block_level"], page_size=req["page_size"],
                              pos_offset=req["pos_offset"], q_new=req["q"], k_new=req["k"],
                              v_new=req["v"], theta=req["theta"], recompute_all=req["recompute_all"])


# ----------------------------------------------------------- closed forms
def test_closed_form_single_frequency_sign():
    """d = 2, theta^0 = 1: q = (0, 1), k = (1, 0) give score -sin(p - t) / sqrt(2)."""
    for p, t0 in [(1, 0), (7, 3), (40, 1), (1000, 998)]:
        k = np.array([[[1.0, 0.0]], [[1.0, 0.0]]])
        v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
        q = np.array([[[0.0, 1.0]]])
        out, lse = native.attention(k, v, np.array([t0, p]), q, np.array([p]), 1e4)
        s0 = -math.sin(p - t0) / math.sqrt(2.0)
        s1 = 0.0
        w0 = math.exp(s0) / (math.exp(s0) + math.exp(s1))
        assert abs(out[0, 0, 0] - w0) < 1e-14
        assert abs(out[0, 0, 1] - (1 - w0)) < 1e-14
        assert abs(lse[0, 0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-14


def test_closed_form_second_frequency_pairing():
    """d = 4: dimension 1 pairs with 3 and rotates at theta^(-1/2)."""
    theta = 1e4
    w1 = theta ** -0.5
    p, t0 = 9, 2
    q = np.zeros((1, 1, 4)); q[0, 0, 3] = 1.0          # imaginary part of pair 1
    k = np.zeros((2, 1, 4)); k[:, 0, 1] = 1.0           # real part of pair 1
    v = np.zeros((2, 1, 4)); v[0, 0, 0] = 1.0; v[1, 0, 2] = 1.0
    out, lse = native.attention(k, v, np.array([t0, p]), q, np.array([p]), theta)
    s0 = -math.sin((p - t0) * w1) / 2.0                 # sqrt(4) = 2
    w = math.exp(s0) / (math.exp(s0) + 1.0)
    assert abs(out[0, 0, 0] - w) < 1e-14 and abs(out[0, 0, 2] - (1 - w)) < 1e-14
    assert abs(out[0, 0, 1]) < 1e-15 and abs(out[0, 0, 3]) < 1e-15


def test_causal_bound_is_inclusive_and_excludes_future():
    """A key at the row's own position is attended; a later one is not."""
    d = 2
    k = np.array([[[0.0, 0.0]], [[5.0, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    q = np.array([[[0.0, 0.0]]])
    out, _ = native.attention(k, v, np.array([3, 4]), q, np.array([3]), 1e4)
    assert np.allclose(out[0, 0], [1.0, 0.0], atol=0, rtol=0)
    out, _ = native.attention(k, v, np.array([3, 4]), q, np.array([4]), 1e4)
    assert np.allclose(out[0, 0], [0.5, 0.5], atol=1e-15)


# ------------------------------------------------------- dense special case
def _rotate_complex(x, pos, theta):
    """RoPE as multiplication of (x_i + i x_{i+d/2}) by exp(i pos theta^(-2i/d))."""
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    freq = theta ** (-2.0 * np.arange(h) / d)
    ph = np.exp(1j * pos[:, None] * freq[None, :])        # [N][h]
    z = z * ph[:, None, :]
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("offset", [0, 7, 5000])
@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 16), (8, 8, 8), (6, 2, 32)])
def test_dense_case_equals_sdpa(offset, hq, hkv, d):
    L = 37
    req = tiny_request(3, hq=hq, hkv=hkv, d=d, prefix_len=0, chunk_lens=(L,), suffix_len=0,
                       k=L, page_size=8, pos_offset=offset)
    out, lse = run_oracle(req)
    pos = offset + np.arange(L)
    qr = torch.from_numpy(_rotate_complex(req["q"], pos, req["theta"])).permute(1, 0, 2)
    kr = torch.from_numpy(_rotate_complex(req["k"], pos, req["theta"])).permute(1, 0, 2)
    vv = torch.from_numpy(req["v"]).permute(1, 0, 2)
    kr = kr.repeat_interleave(hq // hkv, dim=0)
    vv = vv.repeat_interleave(hq // hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(qr[None], kr[None], vv[None],
                                                           is_causal=True)[0]
    ref = ref.permute(1, 0, 2).numpy()
    assert np.abs(out - ref).max() < 1e-12
    # lse against logsumexp of the explicit score matrix
    S = torch.einsum("hqd,hkd->hqk", qr, kr) / math.sqrt(d)
    S = S.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
    assert np.abs(lse - torch.logsumexp(S, -1).T.numpy()).max() < 1e-12


def test_suffix_only_is_dense():
    req = tiny_request(4, prefix_len=0, chunk_lens=(), suffix_len=19, page_size=4, pos_offset=3)
    out, _ = run_oracle(req)
    bo, _, _ = run_brute(req)
    assert np.abs(out - bo).max() < 1e-12


# ------------------------------------------------------------ invariants
@pytest.mark.parametrize("delta", [1, 4097, 100000])
def test_shift_invariance(delta):
    req = tiny_request(5, chunk_lens=(9, 4, 13), k=3, page_size=4)
    base, base_lse = run_oracle(req)
    req2 = tiny_request(5, chunk_lens=(9, 4, 13), k=3, page_size=4, pos_offset=delta)
    assert [s.start - delta for s in req2["segs"]] == [s.start for s in req["segs"]]
    out, lse = run_oracle(req2)
    assert np.abs(out - base).max() < 1e-10
    assert np.abs(lse - base_lse).max() < 1e-10


CASES = [
    dict(),                                                    # prefix, ragged chunks, suffix, k=2
    dict(k=0),                                                 # link half of LegoLink-0
    dict(k=50),                                                # k beyond every chunk length
    dict(block_level=True),
    dict(prefix_len=0),                                        # first chunk also recomputed
    dict(suffix_len=0),
    dict(prefix_len=0, suffix_len=0, chunk_lens=(5,), k=1),
    dict(page_size=1, chunk_lens=(3, 2), k=1),
    dict(pos_offset=11, chunk_lens=(16, 1, 8), page_size=8, k=9),
    dict(recompute_all=True),
    dict(hq=8, hkv=8),
    dict(hq=6, hkv=1, d=4),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_brute_force(case):
    req = tiny_request(100 + case, **CASES[case])
    if req["q"].shape[0] == 0:
        out, lse = run_oracle(req)
        assert out.shape[0] == 0
        return
    out, lse = run_oracle(req)
    bo, bl, bpos = run_brute(req)
    assert list(bpos) == oplan.selected_positions(req["segs"])
    assert np.abs(out - bo).max() < 1e-12
    assert np.abs(lse - bl).max() < 1e-12


# ------------------------------------------- keys compiled from position 0
@pytest.mark.parametrize("case", range(len(CASES)))
def test_keys_compiled_from_zero_equal_position_free(case):
    """Cached keys handed over rotated at 0..L-1 of their own segment (EPIC: every chunk encoded
    from position 0) and re-rotated by the segment's start give the position-free result:
    R(start) R(j) = R(start + j). The compiled form is made here by complex multiplication."""
    req = tiny_request(300 + case, **CASES[case])
    base, base_lse = run_oracle(req)
    compiled = {cid: (_rotate_complex(k, np.arange(k.shape[0]), req["theta"]), v)
                for cid, (k, v) in req["cached"].items()}
    out, lse = olink.link_attention(req["segs"], compiled, req["q"], req["k"], req["v"], req["theta"],
                                    key_layout="segment_rope")
    assert np.abs(out - base).max() < 1e-12
    assert np.abs(lse - base_lse).max() < 1e-12
    if any(s.kind != "suffix" and s.start > 0 and s.recompute < s.length for s in req["segs"]) and len(base):
        # read as position-free, the compiled keys would give another result
        wrong, _ = olink.link_attention(req["segs"], compiled, req["q"], req["k"], req["v"], req["theta"])
        assert np.abs(wrong - base).max() > 1e-3


@pytest.mark.parametrize("offset", [4, 7])
@pytest.mark.parametrize("case", [0, 1, 3, 4, 6, 8])
def test_keys_compiled_after_dummy_tokens_equal_position_free(case, offset):
    """LegoLink-0's compile step puts c dummy tokens first and drops their KV (EPIC summary,
    "Measured effects" table), so token j of a chunk is encoded at position c + j. Keys handed
    over rotated at c + j (complex multiplication here) and re-rotated by the segment's start
    minus c, negative for a chunk linked before position c, give the position-free result:
    R(start - c) R(c + j) = R(start + j). Read with c = 0 they give another."""
    req = tiny_request(700 + case, **CASES[case])
    base, base_lse = run_oracle(req)
    compiled = {cid: (_rotate_complex(k, offset + np.arange(k.shape[0]), req["theta"]), v)
                for cid, (k, v) in req["cached"].items()}
    out, lse = olink.link_attention(req["segs"], compiled, req["q"], req["k"], req["v"], req["theta"],
                                    key_layout="segment_rope", compile_offset=offset)
    assert np.abs(out - base).max() < 1e-12
    assert np.abs(lse - base_lse).max() < 1e-12
    cached_pos = [s.start + j for s in req["segs"] if s.kind != "suffix" for j in range(s.recompute, s.length)]
    sel = oplan.selected_positions(req["segs"])
    if cached_pos and sel and min(cached_pos) <= max(sel):      # some row attends a cached key
        wrong, _ = olink.link_attention(req["segs"], compiled, req["q"], req["k"], req["v"], req["theta"],
                                        key_layout="segment_rope")
        assert np.abs(wrong - base).max() > 1e-3


def test_first_chunk_rows_ignore_cached_values():
    req = tiny_request(7, prefix_len=0, chunk_lens=(10, 12), k=4, page_size=4)
    base, _ = run_oracle(req)
    cached = {key: (kv[0] + 3.0, kv[1] - 2.0) for key, kv in req["cached"].items()}
    out, _ = run_oracle(req, cached=cached)
    assert np.array_equal(out[:4], base[:4])           # rows of chunk 0: all their keys are new
    assert np.abs(out[4:] - base[4:]).max() > 1e-3      # later rows do see cached values


def test_gqa_equals_repeated_kv_heads():
    req = tiny_request(8, hq=8, hkv=2, d=8)
    base, base_lse = run_oracle(req)
    g = 4
    cached = {key: (np.repeat(kv[0], g, axis=1), np.repeat(kv[1], g, axis=1))
              for key, kv in req["cached"].items()}
    out, lse = run_oracle(req, cached=cached, k=np.repeat(req["k"], g, axis=1),
                          v=np.repeat(req["v"], g, axis=1))
    assert np.array_equal(out, base) and np.array_equal(lse, base_lse)


# ------------------------------------------------------------ plan pins
def _config_segments(cfg, request=0):
    ids = gen.request_chunks(cfg)[request]
    return oplan.link_segments(prefix_id=cfg.prefix_id(request) if cfg.prefix_len else None,
                               prefix_len=cfg.prefix_len, chunk_ids=ids,
                               chunk_lens=[cfg.chunk_len] * len(ids), suffix_len=cfg.suffix_len,
                               k=cfg.k, block_level=cfg.block_level, page_size=cfg.page_size)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_plan_sizes_match_closed_forms(name):
    golden = json.load(open(os.path.join(GOLDEN, "plan_counts.json")))
    cfg = CONFIGS[name]
    assert cfg.page_size == golden["page_size"]
    for r in range(min(cfg.n_requests, 3)):
        segs = _config_segments(cfg, r)
        pages = oplan.logical_pages(segs, cfg.page_size)
        got = dict(rows=len(oplan.selected_positions(segs)), tokens=oplan.total_tokens(segs),
                   pages=len(pages), private=sum(p.private for p in pages),
                   cow=sum(p.cow for p in pages))
        assert got == golden[name]


@pytest.mark.parametrize("seed", range(20))
def test_selection_rule_by_enumeration(seed):
    g = np.random.default_rng(seed)
    B = int(g.choice([1, 2, 4, 8, 16]))
    lens = [int(x) for x in g.integers(1, 40, size=int(g.integers(0, 5)))]
    prefix_len = int(g.integers(0, 20))
    S = int(g.integers(0, 20))
    k = int(g.integers(0, 34))
    block = bool(g.integers(0, 2))
    off = int(g.integers(0, 1000))
    segs = oplan.link_segments(prefix_id=77 if prefix_len else None, prefix_len=prefix_len,
                               chunk_ids=list(range(len(lens))), chunk_lens=lens, suffix_len=S,
                               k=k, block_level=block, page_size=B, pos_offset=off)
    # enumerate every token: selected iff its offset in its segment is below that segment's count
    sel, pos, start = [], off, off
    bounds = ([("p", prefix_len)] if prefix_len else []) + [("c", L) for L in lens] + \
             ([("s", S)] if S else [])
    for kind, L in bounds:
        r = 0 if kind == "p" else (L if kind == "s" else (min(B, L) if block else min(k, L)))
        for j in range(L):
            if j < r:
                sel.append(start + j)
        start += L
    assert oplan.selected_positions(segs) == sel
    pages = oplan.logical_pages(segs, B)
    pmap = oplan.position_map(pages, B)
    assert len(pmap) == len(pages) * B
    assert sorted(x for x in pmap if x >= 0) == list(range(off, off + oplan.total_tokens(segs)))
    sel_set = set(sel)
    for i, p in enumerate(pages):
        slots = pmap[i * B:(i + 1) * B]
        held = [x for x in slots if x >= 0]
        assert held == slots[: p.valid] and all(x == -1 for x in slots[p.valid:])
        n_sel = sum(x in sel_set for x in held)
        assert p.private == (n_sel > 0)
        assert p.n_new == n_sel and all(x in sel_set for x in held[:n_sel])
        assert p.cow == (0 < n_sel < p.valid)
    for (lp, s), position in zip(oplan.row_slots(segs, B), sel):
        assert pmap[lp * B + s] == position
