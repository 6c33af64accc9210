"""Pins of the oracle decoder layers (oracle/model.py, oracle/model.c) against facts fixed
outside them (CPU only).

* the explicit-loop projection y = a W^T against numpy's matrix product, on shapes where a
  transposed operand would fail;
* RMSNorm on rows with closed-form results: a constant row, a row with one non-zero entry,
  rows of +-1;
* SiLU at points with closed forms (sigmoid(ln 3) = 3/4);
* a layer whose output and down projections are zero leaves x unchanged, bit for bit;
* a layer with identity-block projections equals its independent statement: the brute-force
  attention of tests/brute.py on q = k = v = RMSNorm(x) added to x, then an MLP written with
  separate gate and up matrices (interleaved by an explicit loop here);
* the bfloat16 rounding: exact for bf16 values, ties to even, round to nearest otherwise.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import model as omodel
from oracle import native
from oracle import plan as oplan
from tests import brute


def test_linear_matches_the_matrix_product():
    g = np.random.default_rng(0)
    for m, n, k in ((1, 1, 1), (7, 5, 3), (33, 64, 48), (16, 16, 16)):
        a = g.standard_normal((m, k))
        w = g.standard_normal((n, k))
        got = native.linear(a, w)
        want = a @ w.T
        assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())
    # a square case: y = a W^T, not a W
    a = g.standard_normal((8, 8))
    w = g.standard_normal((8, 8))
    assert np.abs(native.linear(a, w) - a @ w).max() > 1e-3


def test_rmsnorm_closed_forms():
    dm, eps = 16, 1e-5
    w = np.linspace(0.5, 2.0, dm)
    c = -3.0
    got = native.rmsnorm(np.full((1, dm), c), w, eps)
    assert np.allclose(got[0], c / math.sqrt(c * c + eps) * w, rtol=1e-14, atol=0)
    x = np.zeros((1, dm))
    x[0, 5] = 2.0
    got = native.rmsnorm(x, w, eps)
    want = np.zeros(dm)
    want[5] = 2.0 / math.sqrt(4.0 / dm + eps) * w[5]
    assert np.allclose(got[0], want, rtol=1e-14, atol=0)
    pm = np.where(np.arange(dm) % 3 == 0, 1.0, -1.0)[None]
    assert np.allclose(native.rmsnorm(pm, w, eps)[0], pm[0] * w / math.sqrt(1.0 + eps), rtol=1e-14, atol=0)


def test_silu_closed_forms():
    assert omodel.silu(np.array([0.0]))[0] == 0.0
    assert abs(omodel.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(omodel.silu(np.array([-math.log(3.0)]))[0] + 0.25 * math.log(3.0)) < 1e-15


def test_bf16_rounding():
    exact = np.array([1.0, -2.5, 0.0078125, 2.0 ** 100 * 1.5], dtype=np.float64)
    assert np.array_equal(omodel.round_bf16(exact), np.float32(exact).astype(np.float64))
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even mantissa (1)
    assert omodel.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert omodel.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert omodel.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -12]))[0] == 1.0 + 2.0 ** -7


def _tiny(seed, hq=4, hkv=2, hd=8, chunk_lens=(7, 12), prefix_len=5, suffix_len=4, k=2):
    g = np.random.default_rng(seed)
    dm = hq * hd
    cached = {1000: (g.standard_normal((prefix_len, hkv, hd)), g.standard_normal((prefix_len, hkv, hd)))}
    for i, L in enumerate(chunk_lens):
        cached[i] = (g.standard_normal((L, hkv, hd)), g.standard_normal((L, hkv, hd)))
    segs = oplan.link_segments(prefix_id=1000, prefix_len=prefix_len, chunk_ids=list(range(len(chunk_lens))),
                               chunk_lens=list(chunk_lens), suffix_len=suffix_len, k=k, block_level=False,
                               page_size=4)
    R = len(oplan.selected_positions(segs))
    x = g.standard_normal((R, dm))
    return g, segs, cached, x


def test_zero_output_and_down_projections_leave_x_unchanged():
    g, segs, cached, x = _tiny(1)
    hq, hkv, hd, dff = 4, 2, 8, 64
    dm = hq * hd
    xb = omodel.round_bf16(x)
    w = dict(attn_norm=np.ones(dm), w_qkv=g.standard_normal(((hq + 2 * hkv) * hd, dm)) / math.sqrt(dm),
             w_o=np.zeros((dm, hq * hd)), mlp_norm=np.ones(dm), w_gate_up=g.standard_normal((2 * dff, dm)),
             w_down=np.zeros((dm, dff)))
    out = omodel.layer_forward(xb, w, [segs], cached, 1e4, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, eps=1e-5)
    assert np.array_equal(out, xb)


def test_identity_block_layer_equals_its_independent_statement():
    """W_q = I, W_k = W_v = the first Hkv * d rows of I, W_o = I: the attention sublayer adds the
    brute-force attention of the normed rows; then an MLP with separate gate and up matrices."""
    g, segs, cached, x = _tiny(2)
    hq, hkv, hd, dff, eps, theta = 4, 2, 8, 64, 1e-5, 1e4
    dm, kvd = hq * hd, hkv * hd
    eye = np.eye(dm)
    w_qkv = np.concatenate([eye, eye[:kvd], eye[:kvd]])
    attn_norm = 1.0 + 0.1 * g.standard_normal(dm)
    mlp_norm = 1.0 + 0.1 * g.standard_normal(dm)
    w_gate = g.standard_normal((dff, dm)) / math.sqrt(dm)
    w_up = g.standard_normal((dff, dm)) / math.sqrt(dm)
    w_down = g.standard_normal((dm, dff)) / math.sqrt(dff)
    w_gate_up = np.zeros((2 * dff, dm))
    for r in range(2 * dff):                       # rows: 32 gate, 32 up, ...
        blk, j = divmod(r, 64)
        w_gate_up[r] = w_gate[32 * blk + j] if j < 32 else w_up[32 * blk + j - 32]
    w = dict(attn_norm=attn_norm, w_qkv=w_qkv, w_o=eye, mlp_norm=mlp_norm, w_gate_up=w_gate_up, w_down=w_down)
    got = omodel.layer_forward(x, w, [segs], cached, theta, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, eps=eps,
                               round_bf16_acts=False)
    # independent statement
    R = x.shape[0]
    h = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps) * attn_norm
    q = h.reshape(R, hq, hd)
    kv = h[:, :kvd].reshape(R, hkv, hd)
    chunks = [cached[i] for i in range(2)]
    bo, _, _ = brute.link_request(prefix=cached[1000], chunks=chunks, suffix_len=4, k=2, block_level=False,
                                  page_size=4, pos_offset=0, q_new=q, k_new=kv, v_new=kv, theta=theta)
    x1 = x + bo.reshape(R, dm)
    h1 = x1 / np.sqrt((x1 * x1).mean(axis=1, keepdims=True) + eps) * mlp_norm
    z = h1 @ w_gate.T
    want = x1 + ((z / (1.0 + np.exp(-z))) * (h1 @ w_up.T)) @ w_down.T
    assert np.abs(got - want).max() < 1e-10


def test_the_pins_catch_a_swapped_gate_and_up():
    g, segs, cached, x = _tiny(3)
    hq, hkv, hd, dff = 4, 2, 8, 64
    dm = hq * hd
    w = dict(attn_norm=np.ones(dm), w_qkv=g.standard_normal(((hq + 2 * hkv) * hd, dm)) / math.sqrt(dm),
             w_o=np.zeros((dm, hq * hd)), mlp_norm=np.ones(dm), w_gate_up=g.standard_normal((2 * dff, dm)) / 6,
             w_down=g.standard_normal((dm, dff)) / 8)
    kw = dict(num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, eps=1e-5, round_bf16_acts=False)
    base = omodel.layer_forward(x, w, [segs], cached, 1e4, **kw)
    swapped = dict(w)
    blocks = w["w_gate_up"].reshape(dff // 32, 2, 32, dm)[:, ::-1]
    swapped["w_gate_up"] = blocks.reshape(2 * dff, dm)
    assert np.abs(omodel.layer_forward(x, swapped, [segs], cached, 1e4, **kw) - base).max() > 1e-3
