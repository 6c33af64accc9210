"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case compiles a copy of oracle/attention.c with one plausible mistake
(a flipped rotation sign, a wrong pairing frequency, a dropped scale, an
exclusive causal bound, a wrong GQA head map, a one-pass softmax without the
maximum, a key rotation that ignores the per-key rotation position) into a
temporary directory and runs the closed-form, dense-case and compiled-from-0
pins against it. Every mutant has to fail at least one of them; the
unmodified source has to pass all of them.
"""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest
import torch

from oracle import native

MUTANTS = {
    "original": None,
    "rotation_sign": ("y[i] = x[i] * c - x[i + half] * s;", "y[i] = x[i] * c + x[i + half] * s;"),
    "frequency_exponent": ("pow(rope_theta, -2.0 * i / d)", "pow(rope_theta, -1.0 * i / d)"),
    "dropped_scale": ("s *= inv_sqrt_d;", ""),
    "exclusive_causal": ("if (key_pos[t] > p)\n                    continue;\n                const double *kt",
                         "if (key_pos[t] >= p)\n                    continue;\n                const double *kt"),
    "gqa_modulo": ("int g = h / group;", "int g = h % n_kv_heads;"),
    "value_head": ("const double *vt = v + ((size_t)t * n_kv_heads + g) * d;",
                   "const double *vt = v + ((size_t)t * n_kv_heads + 0) * d;"),
    "rotation_position_ignored": ("key_rot ? key_rot[t] : key_pos[t]", "key_pos[t]"),
}


def _build(tmp_path, name):
    src = open(native.SOURCE).read()
    if MUTANTS[name] is not None:
        old, new = MUTANTS[name]
        assert old in src, name
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return native.load(str(so))


def _closed_form_ok(fn):
    p, t0 = 7, 3
    k = np.array([[[1.0, 0.0]], [[1.0, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    q = np.array([[[0.0, 1.0]]])
    out, lse = native.attention(k, v, np.array([t0, p]), q, np.array([p]), 1e4, entry=fn)
    s0 = -math.sin(p - t0) / math.sqrt(2.0)
    w0 = math.exp(s0) / (math.exp(s0) + 1.0)
    return abs(out[0, 0, 0] - w0) < 1e-14 and abs(lse[0, 0] - math.log(math.exp(s0) + 1.0)) < 1e-14


def _causal_ok(fn):
    k = np.array([[[0.0, 0.0]], [[5.0, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    q = np.array([[[0.0, 0.0]]])
    out, _ = native.attention(k, v, np.array([3, 4]), q, np.array([3]), 1e4, entry=fn)
    return bool(np.isfinite(out).all() and np.allclose(out[0, 0], [1.0, 0.0], atol=0, rtol=0))


def _dense_ok(fn, compiled_from_zero=False):
    """One segment at offset 5, every row attending: scaled_dot_product_attention over tensors
    rotated by complex multiplication. With compiled_from_zero the keys are handed over
    rotated at 0..L-1 (a chunk encoded on its own) and rotated by the segment's start."""
    g = np.random.default_rng(0)
    L, hq, hkv, d, theta = 23, 4, 2, 16, 1e4
    q = g.standard_normal((L, hq, d))
    k = g.standard_normal((L, hkv, d))
    v = g.standard_normal((L, hkv, d))
    pos = np.arange(L) + 5
    h = d // 2
    freq = theta ** (-2.0 * np.arange(h) / d)

    def rot_at(x, at):
        z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * at[:, None] * freq[None, :])[:, None, :]
        return np.concatenate([z.real, z.imag], -1)

    if compiled_from_zero:
        out, _ = native.attention(rot_at(k, np.arange(L)), v, pos, q, pos, theta, entry=fn,
                                  key_rot=np.full(L, 5))
    else:
        out, _ = native.attention(k, v, pos, q, pos, theta, entry=fn)

    def rot(x):
        return torch.from_numpy(rot_at(x, pos)).permute(1, 0, 2)

    ref = torch.nn.functional.scaled_dot_product_attention(
        rot(q)[None], rot(k).repeat_interleave(hq // hkv, 0)[None],
        torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None],
        is_causal=True)[0].permute(1, 0, 2).numpy()
    return bool(np.isfinite(out).all() and np.abs(out - ref).max() < 1e-12)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistakes(tmp_path, name):
    fn = _build(tmp_path, name)
    verdicts = [_closed_form_ok(fn), _causal_ok(fn), _dense_ok(fn), _dense_ok(fn, compiled_from_zero=True)]
    if name == "original":
        assert all(verdicts)
    else:
        assert not all(verdicts), f"mutant {name} passed every pin"
