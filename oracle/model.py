"""Oracle forward of the selected rows through decoder layers around the link step.

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

At link time only the recomputed rows (the first k tokens of every chunk, and the suffix) run
through the model; every other token's K/V of every layer is the compile step's (EPIC,
atlas.scime.ai summary, "Approach"; "Key results" and "Limitations": 7-9B Llama-class models).
One layer, for the rows' hidden states x:

    h = RMSNorm(x) * attn_norm,  RMSNorm(x) = x / sqrt(mean(x^2) + eps)
    q, k, v = h W_qkv^T          (W_qkv rows: the query heads, then the key heads, then the values)
    a = link attention of q over the layer's merged cache, with k, v the rows' new K/V
    x = x + a W_o^T
    h = RMSNorm(x) * mlp_norm
    x = x + (SiLU(h W_gate^T) * (h W_up^T)) W_down^T,   SiLU(z) = z / (1 + exp(-z))

Readings where the pages are silent (Llama-3 conventions, the plainest reading of a
"Llama-3-8B-shaped" layer): pre-norm RMSNorm, SwiGLU MLP, no biases. The gate and up weights
come as one matrix whose rows alternate 32 gate rows and 32 up rows (the weight layout of the
library's fused gate/up projection). Activations are held in bfloat16 between these steps (the
model's tensor type): each step computes in fp64 from the bfloat16 values it reads and rounds its
result once (float32, then bfloat16 with round-to-nearest-even); ``round_bf16=False`` keeps fp64
throughout.
"""
from __future__ import annotations

import numpy as np

from . import native
from .link import link_attention


def round_bf16(x):
    """fp64 -> float32 -> bfloat16 (round to nearest, ties to even), returned as fp64."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


def split_gate_up(w_gate_up):
    """Gate and up weights from the interleaved matrix (rows: 32 gate, 32 up, ...)."""
    w = np.asarray(w_gate_up, dtype=np.float64)
    n2, k = w.shape
    blocks = w.reshape(n2 // 64, 2, 32, k)
    return blocks[:, 0].reshape(-1, k), blocks[:, 1].reshape(-1, k)


def layer_forward(x, w, seg_lists, cached, theta, *, num_q_heads, num_kv_heads, head_dim, eps,
                  key_layout="position_free", compile_offset=0, round_bf16_acts=True):
    """One layer over the rows of every request (rows of request i are seg_lists[i]'s selected
    rows, requests in order). ``w``: dict of attn_norm, w_qkv, w_o, mlp_norm, w_gate_up, w_down;
    ``cached``: the layer's cached (K, V) per store id. Returns the new x [R][d_model]."""
    rb = round_bf16 if round_bf16_acts else (lambda a: np.asarray(a, dtype=np.float64))
    x = np.asarray(x, dtype=np.float64)
    R = x.shape[0]
    qd, kvd = num_q_heads * head_dim, num_kv_heads * head_dim
    h = rb(native.rmsnorm(x, w["attn_norm"], eps))
    qkv = native.linear(h, w["w_qkv"])
    q = rb(qkv[:, :qd]).reshape(R, num_q_heads, head_dim)
    k = rb(qkv[:, qd:qd + kvd]).reshape(R, num_kv_heads, head_dim)
    v = rb(qkv[:, qd + kvd:]).reshape(R, num_kv_heads, head_dim)
    a = np.empty((R, num_q_heads, head_dim))
    r0 = 0
    for segs in seg_lists:
        n = sum(s.recompute for s in segs)
        if n:
            out, _ = link_attention(segs, cached, q[r0:r0 + n], k[r0:r0 + n], v[r0:r0 + n], theta,
                                    key_layout=key_layout, compile_offset=compile_offset)
            a[r0:r0 + n] = out
        r0 += n
    if r0 != R:
        raise ValueError("rows do not match the plans")
    a = rb(a).reshape(R, qd)
    x = rb(x + native.linear(a, w["w_o"]))
    h = rb(native.rmsnorm(x, w["mlp_norm"], eps))
    w_gate, w_up = split_gate_up(w["w_gate_up"])
    act = rb(silu(native.linear(h, w_gate)) * native.linear(h, w_up))
    return rb(x + native.linear(act, w["w_down"]))


def forward(x, layers, seg_lists, cached_per_layer, theta, **kw):
    """Every layer in order; ``layers`` and ``cached_per_layer`` are per-layer lists."""
    for w, cached in zip(layers, cached_per_layer):
        x = layer_forward(x, w, seg_lists, cached, theta, **kw)
    return x
