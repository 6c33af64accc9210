"""Oracle link step for one request: merged cache, then attention of the recomputed rows.

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

The merged cache is the request's tokens in prompt order. A recomputed row takes
its new K/V; every other token keeps the cached, position-free K/V of its
segment. The new K/V are in place before any row attends. Every recomputed row
therefore sees every other recomputed row's new K/V at its linked position
(EPIC, atlas.scime.ai summary, "Approach"; MEPIC, searcharxiv.org abstract).
"""
from __future__ import annotations

import numpy as np

from . import native
from .plan import selected_positions, token_positions


def merged_cache(segs, cached: dict, k_new, v_new):
    """Token-level K, V [N][Hkv][d] (fp64) and absolute positions [N] of one request.

    ``cached`` maps a segment's store id to its position-free (K, V), each
    [length][Hkv][d]; ``k_new``/``v_new`` hold the recomputed rows in the
    order of ``selected_positions(segs)``.
    """
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    hkv, d = k_new.shape[1], k_new.shape[2]
    ks, vs = [], []
    r = 0
    for s in segs:
        if s.kind == "suffix":
            kk = np.zeros((s.length, hkv, d))
            vv = np.zeros((s.length, hkv, d))
        else:
            ck, cv = cached[s.chunk_id]
            if ck.shape[0] != s.length:
                raise ValueError("cached segment length mismatch")
            kk = np.array(ck, dtype=np.float64)
            vv = np.array(cv, dtype=np.float64)
        kk[: s.recompute] = k_new[r: r + s.recompute]
        vv[: s.recompute] = v_new[r: r + s.recompute]
        r += s.recompute
        ks.append(kk)
        vs.append(vv)
    if r != k_new.shape[0]:
        raise ValueError("number of new rows does not match the plan")
    if not ks:
        return np.zeros((0, hkv, d)), np.zeros((0, hkv, d)), np.zeros(0, dtype=np.int64)
    return (np.concatenate(ks), np.concatenate(vs),
            np.asarray(token_positions(segs), dtype=np.int64))


def link_attention(segs, cached: dict, q_new, k_new, v_new, rope_theta, rows=None):
    """Outputs [R'][Hq][d] and lse [R'][Hq] (fp64) of the recomputed rows.

    ``rows`` optionally restricts the computation to a subset of row indices
    (for sampled checks at full size); the merged cache is always complete.
    """
    k, v, key_pos = merged_cache(segs, cached, k_new, v_new)
    row_pos = np.asarray(selected_positions(segs), dtype=np.int64)
    q = np.asarray(q_new, dtype=np.float64)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[rows]
        row_pos = row_pos[rows]
        # keys after the last requested row cannot contribute
    if q.shape[0] == 0:
        return np.zeros((0,) + q.shape[1:]), np.zeros((0, q.shape[1]))
    limit = int(row_pos.max())
    n = int(np.searchsorted(key_pos, limit, side="right"))
    return native.attention(k[:n], v[:n], key_pos[:n], q, row_pos, rope_theta)
