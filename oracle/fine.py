"""Fine-grained M x 1 slice mask (oracle; test infrastructure).

FG-Attn verdict page: the unit of skipping is an M x 1 slice, M contiguous
queries against one key (pith_extraction.key_machinery, core_discovery).
One of its two training-free masks pools the queries of a group into their
mean q_avg and keeps the keys whose score k . q_avg passes a threshold
(referee_report.major_comments[1]; the printed threshold formula is garbled
and its constant undefined).

Readings:
  * groups are M consecutive raster rows, the last one possibly shorter;
  * q_avg uses the exact-sum rule of the tile summarizer (fp32 result);
  * score s_gj = sum_c k_j[c] * q_avg_g[c] added left to right in fp64
    (each product exact); the threshold's monotone map of the score is
    dropped since only the order matters;
  * per head the threshold tau is the K-th largest score over all
    (group, key) pairs with K = ceil(keep * G * N); pairs with s >= tau are
    kept (ties at tau are kept).
"""
from __future__ import annotations

import math

import numpy as np

from .select import _assert_exact_sum


def groups(N, M):
    return [np.arange(g, min(g + M, N)) for g in range(0, N, M)]


def group_means(q, M):
    q64 = np.asarray(q, dtype=np.float64)
    gs = groups(q64.shape[0], M)
    out = np.zeros((len(gs), q64.shape[1]), dtype=np.float32)
    for g, rows in enumerate(gs):
        blk = q64[rows]
        _assert_exact_sum(blk)
        out[g] = (blk.sum(axis=0) / float(len(rows))).astype(np.float32)
    return out


def group_scores(qbar, k):
    """s[g, j] with the fixed left-to-right fp64 order over channels."""
    qb = np.asarray(qbar, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    acc = np.zeros((qb.shape[0], k64.shape[0]), dtype=np.float64)
    for c in range(qb.shape[1]):
        acc = acc + np.outer(qb[:, c], k64[:, c])
    return acc


def keep_count(keep, G, N):
    return max(1, int(math.ceil(keep * G * N - 1e-9)))


def threshold(s, kcount):
    """K-th largest value of s."""
    flat = s.ravel()
    return float(np.partition(flat, flat.size - kcount)[flat.size - kcount])


def kept_lists(s, tau):
    """Per group: ascending key indices with s >= tau."""
    return [np.nonzero(s[g] >= tau)[0].astype(np.int32) for g in range(s.shape[0])]
