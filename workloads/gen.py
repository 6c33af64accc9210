"""Seeded synthetic inputs for the link workloads.

Every array is drawn from numpy's PCG64 keyed by (config seed, kind, identifier),
so a pooled chunk's position-free K/V is the same in every request that links
it. Values are drawn in float32, scaled, and (for bf16 workloads) rounded to
bfloat16 with round-to-nearest-even; the rounded values are returned as
float32 arrays so that every consumer sees exactly the same numbers.

This module holds no part of the link step: it does not select rows, place
tokens or compute attention.
"""
from __future__ import annotations

import numpy as np

from .configs import LinkConfig

KIND_CHUNK_K = 1
KIND_CHUNK_V = 2
KIND_Q = 3
KIND_K_NEW = 4
KIND_V_NEW = 5
KIND_PREFIX_K = 6
KIND_PREFIX_V = 7
KIND_DRAW = 8
KIND_Q_ALL = 9


KIND_WEIGHT = 10
KIND_HIDDEN = 11


def rng(seed: int, kind: int, ident: int, layer: int = 0) -> np.random.Generator:
    """PCG64 keyed by (seed, kind, id) — and the decoder layer for layers after the first."""
    key = [seed, kind, ident] + ([layer] if layer else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    # NaN/Inf never occur for finite normal draws; keep them untouched anyway.
    bad = ~np.isfinite(x)
    if bad.any():
        out = out.copy()
        out[bad] = x[bad]
    return out


def normal(seed: int, kind: int, ident: int, shape, scale: float, dtype: str, layer: int = 0) -> np.ndarray:
    a = rng(seed, kind, ident, layer).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    if dtype == "bf16":
        a = round_bf16(a)
    return a


def chunk_kv(cfg: LinkConfig, chunk_id: int, layer: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Position-free K and V of one pooled chunk at one decoder layer, each [chunk_len][Hkv][d]."""
    shape = (cfg.chunk_len, cfg.num_kv_heads, cfg.head_dim)
    return (normal(cfg.seed, KIND_CHUNK_K, chunk_id, shape, cfg.kv_scale, cfg.dtype, layer),
            normal(cfg.seed, KIND_CHUNK_V, chunk_id, shape, cfg.kv_scale, cfg.dtype, layer))


def prefix_kv(cfg: LinkConfig, request: int, layer: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Cached K and V of a request's prefix at one decoder layer, each [prefix_len][Hkv][d]."""
    shape = (cfg.prefix_len, cfg.num_kv_heads, cfg.head_dim)
    return (normal(cfg.seed, KIND_PREFIX_K, request, shape, cfg.kv_scale, cfg.dtype, layer),
            normal(cfg.seed, KIND_PREFIX_V, request, shape, cfg.kv_scale, cfg.dtype, layer))


def layer_weights(seed: int, layer: int, *, d_model: int, d_ff: int, num_q_heads: int, num_kv_heads: int,
                  head_dim: int) -> dict:
    """Random bf16 weights of one decoder layer (float32 arrays of bf16 values): projections
    N(0, 1/fan_in) as [out][in], norm weights 1 + 0.1 N(0, 1)."""
    qd, kvd = num_q_heads * head_dim, num_kv_heads * head_dim
    shapes = dict(attn_norm=(d_model,), w_qkv=(qd + 2 * kvd, d_model), w_o=(d_model, qd), mlp_norm=(d_model,),
                  w_gate_up=(2 * d_ff, d_model), w_down=(d_model, d_ff))
    out = {}
    for i, (name, shape) in enumerate(shapes.items()):
        g = rng(seed, KIND_WEIGHT, i, layer + 1)
        a = g.standard_normal(shape, dtype=np.float32)
        if len(shape) == 1:
            a = np.float32(1.0) + np.float32(0.1) * a
        else:
            a *= np.float32(1.0 / np.sqrt(shape[1]))
        out[name] = round_bf16(a)
    return out


def hidden_states(seed: int, request: int, n_rows: int, d_model: int) -> np.ndarray:
    """Hidden states [n][d_model] of a request's selected rows entering the first layer, N(0, 1), bf16."""
    return normal(seed, KIND_HIDDEN, request, (n_rows, d_model), 1.0, "bf16")


def new_rows(cfg: LinkConfig, request: int, n_rows: int):
    """New Q [n][Hq][d] and new K, V [n][Hkv][d] for the n recomputed rows of a request."""
    qs = (n_rows, cfg.num_q_heads, cfg.head_dim)
    ks = (n_rows, cfg.num_kv_heads, cfg.head_dim)
    return (normal(cfg.seed, KIND_Q, request, qs, cfg.q_scale, cfg.dtype),
            normal(cfg.seed, KIND_K_NEW, request, ks, cfg.kv_scale, cfg.dtype),
            normal(cfg.seed, KIND_V_NEW, request, ks, cfg.kv_scale, cfg.dtype))


def request_chunks(cfg: LinkConfig) -> list[list[int]]:
    """Chunk ids linked by every request, in prompt order."""
    out = []
    for r in range(cfg.n_requests):
        if cfg.pool_draw == "sequential":
            ids = list(range(cfg.chunks_per_request))
        elif cfg.pool_draw == "uniform":
            g = rng(cfg.seed, KIND_DRAW, r)
            ids = [int(i) for i in g.choice(cfg.pool_size, size=cfg.chunks_per_request, replace=False)]
        elif cfg.pool_draw == "zipf":
            # p(rank) ~ rank^-s over ranks 1..pool_size, drawn one at a time
            # without replacement; chunk id = rank - 1.
            g = rng(cfg.seed, KIND_DRAW, r)
            w = np.arange(1, cfg.pool_size + 1, dtype=np.float64) ** (-cfg.zipf_s)
            avail = np.ones(cfg.pool_size, dtype=bool)
            ids = []
            for _ in range(cfg.chunks_per_request):
                p = np.where(avail, w, 0.0)
                p /= p.sum()
                pick = int(g.choice(cfg.pool_size, p=p))
                avail[pick] = False
                ids.append(pick)
        else:
            raise ValueError(f"unknown pool draw {cfg.pool_draw!r}")
        out.append(ids)
    return out


def used_chunks(cfg: LinkConfig) -> list[int]:
    """Distinct chunk ids referenced by any request, ascending."""
    return sorted({c for ids in request_chunks(cfg) for c in ids})


def structured_values(ident: int, n: int, hkv: int, d: int, new: bool = False) -> np.ndarray:
    """Values [n][Hkv][d] whose every entry is a multiple of 1/16 below 4 in magnitude, so that
    bfloat16 holds them and float32 sums of up to 2^18 of them exactly.

    Entry (token j, head g, dim e) of a stored segment ``ident``:
    (A(g, e) + B(g, e) * U(ident) + W(j)) / 16, with A = (7g + 3e) mod 11 - 5,
    B = (5g + e) mod 7 - 3, U = 37 * ident mod 29 - 14 and W = j mod 5 - 2; recomputed rows
    (``new``, ``ident`` = request) take (A + 4B - 1) / 16. A mean over any long run of tokens then
    keeps an O(1) part that differs between heads, dimensions and sets of segments.
    """
    g = np.arange(hkv)[:, None]
    e = np.arange(d)[None, :]
    a = (7 * g + 3 * e) % 11 - 5
    b = (5 * g + e) % 7 - 3
    if new:
        base = (a + 4 * b - 1)[None].repeat(n, axis=0)
    else:
        u = (37 * int(ident)) % 29 - 14
        w = np.arange(n) % 5 - 2
        base = (a + b * u)[None] + w[:, None, None]
    return (base / 16.0).astype(np.float32)
