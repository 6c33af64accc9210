"""Oracle link step for one request: merged cache, then attention of the recomputed rows.

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

The merged cache is the request's tokens in prompt order. A recomputed row takes
its new K/V; every other token keeps the cached, position-free K/V of its
segment. The new K/V are in place before any row attends. Every recomputed row
therefore sees every other recomputed row's new K/V at its linked position
(EPIC, atlas.scime.ai summary, "Approach"; MEPIC, searcharxiv.org abstract).

Cached keys come in one of two forms. Position-free keys (MEPIC abstract) are
rotated at each token's absolute position. Keys compiled from position 0 (EPIC
summary, "Approach": a chunk is encoded on its own, so token j of a segment
carries the rotation of position j) are re-rotated by the segment's linked
start, the offset the chunk is moved by. A chunk compiled after c leading
tokens whose KV is then dropped (EPIC summary, "Measured effects" table: the
LegoLink-0 ablation prepends four dummy tokens during compilation and discards
them; read here as the dummies taking positions 0..c-1, so token j of the chunk
was encoded at position c + j) carries the rotation of c + j, and moves by the
segment's start minus c, which is negative for a chunk linked before position
c. New rows are always given position-free and are rotated at their absolute
position.
"""
from __future__ import annotations

import numpy as np

from . import native
from .plan import selected_positions, token_positions


KEY_LAYOUTS = ("position_free", "segment_rope")


def merged_cache(segs, cached: dict, k_new, v_new, key_layout="position_free", compile_offset=0):
    """Token-level K, V [N][Hkv][d] (fp64), absolute positions [N] and the
    position each key is rotated by [N] of one request.

    ``cached`` maps a segment's store id to its cached (K, V), each
    [length][Hkv][d], with keys in the form ``key_layout`` names;
    ``k_new``/``v_new`` hold the recomputed rows (position-free keys) in the
    order of ``selected_positions(segs)``. With ``key_layout="segment_rope"``,
    cached token j of a segment carries the rotation of ``compile_offset + j``.
    """
    if key_layout not in KEY_LAYOUTS:
        raise ValueError(f"unknown key layout {key_layout!r}")
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    hkv, d = k_new.shape[1], k_new.shape[2]
    ks, vs, rot = [], [], []
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
        # rotation of each key: its absolute position, except cached keys compiled from
        # position 0, which move by the segment's start
        pos = s.start + np.arange(s.length, dtype=np.int64)
        if key_layout == "segment_rope" and s.kind != "suffix":
            pos[s.recompute:] = s.start - compile_offset
        rot.append(pos)
    if r != k_new.shape[0]:
        raise ValueError("number of new rows does not match the plan")
    if not ks:
        return (np.zeros((0, hkv, d)), np.zeros((0, hkv, d)), np.zeros(0, dtype=np.int64),
                np.zeros(0, dtype=np.int64))
    return (np.concatenate(ks), np.concatenate(vs),
            np.asarray(token_positions(segs), dtype=np.int64), np.concatenate(rot))


def link_attention(segs, cached: dict, q_new, k_new, v_new, rope_theta, rows=None,
                   key_layout="position_free", compile_offset=0):
    """Outputs [R'][Hq][d] and lse [R'][Hq] (fp64) of the recomputed rows.

    ``rows`` optionally restricts the computation to a subset of row indices
    (for sampled checks at full size); the merged cache is always complete.
    """
    if compile_offset < 0:
        raise ValueError("compile_offset must be >= 0")
    k, v, key_pos, key_rot = merged_cache(segs, cached, k_new, v_new, key_layout, compile_offset)
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
    return native.attention(k[:n], v[:n], key_pos[:n], q, row_pos, rope_theta, key_rot=key_rot[:n])
