"""Brute-force statement of the link step for tiny inputs (numpy, fp64).

Written independently of oracle/: it re-derives segment starts and the selected
tokens from the request description, materialises one d x d rotation matrix per
position, forms the full N x N causal score matrix of the merged cache for
every token (queries of non-recomputed tokens are zero), takes the softmax of
every row and only then keeps the recomputed rows.
"""
from __future__ import annotations

import numpy as np


def rotation_matrix(pos: int, d: int, theta: float) -> np.ndarray:
    """Block rotation acting on the planes (i, i + d/2), angle pos * theta^(-2i/d)."""
    h = d // 2
    R = np.zeros((d, d))
    for i in range(h):
        a = pos * theta ** (-2.0 * i / d)
        R[i, i] = np.cos(a)
        R[i, i + h] = -np.sin(a)
        R[i + h, i] = np.sin(a)
        R[i + h, i + h] = np.cos(a)
    return R


def link_request(*, prefix, chunks, suffix_len, k, block_level, page_size, pos_offset,
                 q_new, k_new, v_new, theta, recompute_all=False):
    """prefix: None or (K, V); chunks: list of (K, V), each [L][Hkv][d].

    Returns (out [R][Hq][d], lse [R][Hq], selected positions [R]).
    """
    q_new = np.asarray(q_new, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    hq, d = q_new.shape[1], q_new.shape[2]
    hkv = k_new.shape[1]
    # token table: (cached K or None, cached V, is_selected)
    tokens = []
    if prefix is not None:
        pk, pv = prefix
        for j in range(pk.shape[0]):
            tokens.append((pk[j], pv[j], recompute_all))
    for ck, cv in chunks:
        L = ck.shape[0]
        if recompute_all:
            r = L
        elif block_level:
            r = min(page_size, L)
        else:
            r = min(k, L)
        for j in range(L):
            tokens.append((ck[j], cv[j], j < r))
    for j in range(suffix_len):
        tokens.append((None, None, True))
    N = len(tokens)
    positions = pos_offset + np.arange(N)
    sel = np.array([t[2] for t in tokens], dtype=bool)
    if sel.sum() != q_new.shape[0]:
        raise ValueError("wrong number of new rows")
    K = np.zeros((N, hkv, d))
    V = np.zeros((N, hkv, d))
    Q = np.zeros((N, hq, d))
    r = 0
    for n, (ck, cv, s) in enumerate(tokens):
        if s:
            K[n], V[n], Q[n] = k_new[r], v_new[r], q_new[r]
            r += 1
        else:
            K[n], V[n] = ck, cv
    rots = [rotation_matrix(int(p), d, theta) for p in positions]
    Qr = np.stack([Q[n] @ rots[n].T for n in range(N)])     # [N][Hq][d]
    Kr = np.stack([K[n] @ rots[n].T for n in range(N)])     # [N][Hkv][d]
    group = hq // hkv
    Kr = np.repeat(Kr, group, axis=1)                       # kv head of q head h is h // group
    Vr = np.repeat(V, group, axis=1)
    mask = positions[None, :] <= positions[:, None]         # [query, key]
    out = np.zeros((N, hq, d))
    lse = np.zeros((N, hq))
    for h in range(hq):
        S = (Qr[:, h, :] @ Kr[:, h, :].T) / np.sqrt(d)
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        W = np.exp(S - m)
        Z = W.sum(axis=1, keepdims=True)
        out[:, h, :] = (W / Z) @ Vr[:, h, :]
        lse[:, h] = (m + np.log(Z))[:, 0]
    return out[sel], lse[sel], positions[sel]
