"""Masked softmax attention (oracle; test infrastructure).

The attention that a block mask leaves is ordinary softmax attention with
the pruned pairs removed: additive mask 0 / -inf on block pairs (SPADE
review page, referee report minor comment on Eq. (2)).  Online-softmax
kernels are an exact reorganisation of it (SPADE review page, ledger axiom
on FlashAttention-style online softmax), so the oracle computes the
definition directly, in fp64:
    O_q = sum_k softmax_k(scale * q . k) v_k   over the allowed keys of q.
A query with no allowed key gets O = 0 (reading; only the fine-grained
mask can produce one).
"""
from __future__ import annotations

import numpy as np


def attention_dense(q, k, v, allowed=None, scale=None):
    """q [nq, d], k [nk, d], v [nk, dv]; allowed [nq, nk] bool or None."""
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q64.shape[1])
    s = (q64 @ k64.T) * scale
    if allowed is not None:
        s = np.where(allowed, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(mx)
    mx = np.where(empty, 0.0, mx)
    e = np.exp(s - mx)
    z = e.sum(axis=1, keepdims=True)
    p = e / np.where(z > 0, z, 1.0)
    out = p @ v64
    return np.where(empty, 0.0, out)


def block_sparse_attention(q, k, v, members, rows, query_tiles=None, scale=None):
    """One head. q,k,v [N, d]; rows[i] = kept key tiles of query tile i.

    Returns fp64 O [N, d] (rows of tiles not in query_tiles stay zero).
    """
    N, d = q.shape
    out = np.zeros((N, v.shape[1]), dtype=np.float64)
    tiles = range(len(members)) if query_tiles is None else query_tiles
    for i in tiles:
        qi = members[i]
        keys = np.concatenate([members[j] for j in rows[i]]) if rows[i] else \
            np.zeros(0, dtype=np.int64)
        if keys.size == 0:
            continue
        out[qi] = attention_dense(q[qi], k[keys], v[keys], None, scale)
    return out


def token_mask(members, rows, N):
    """Expand a tile-level row list to the token-level boolean mask."""
    tid = np.empty(N, dtype=np.int64)
    for i, m in enumerate(members):
        tid[m] = i
    nT = len(members)
    blk = np.zeros((nT, nT), dtype=bool)
    for i, r in enumerate(rows):
        blk[i, r] = True
    return blk[tid][:, tid]


def fine_attention(q, k, v, group_rows, kept, query_groups=None, scale=None):
    """One head: group g's queries attend to the keys in kept[g]."""
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    gs = range(len(group_rows)) if query_groups is None else query_groups
    for g in gs:
        rws = group_rows[g]
        ks = kept[g]
        if len(ks) == 0:
            continue
        out[rws] = attention_dense(q[rws], k[ks], v[ks], None, scale)
    return out
