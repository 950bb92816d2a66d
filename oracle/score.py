"""Cluster scoring and selection (fp64), one head.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import SCORE_QUEST, SCORE_MEAN, SEL_TOPK, SEL_DENSITY, SEL_TOPP, SEL_DENSE


def quest_scores(cq: np.ndarray, kmax: np.ndarray, kmin: np.ndarray, count: np.ndarray) -> np.ndarray:
    """AdaCluster eq. (1), in its literal per-dimension max form:
    S[r, c] = sum_d max(q_d * max(K_c^d), q_d * min(K_c^d)).

    The query side is the query-cluster centre (the pages score per query
    cluster; the centre is the mean of the normalised member queries and is
    not re-normalised).  The key side is each key cluster's per-dimension
    max and min vectors.  Empty clusters score -inf."""
    a = cq[:, None, :] * kmax[None, :, :]
    b = cq[:, None, :] * kmin[None, :, :]
    S = np.sum(np.maximum(a, b), axis=2)
    S[:, count == 0] = -np.inf
    return S


def quest_scores_split(cq: np.ndarray, kmax: np.ndarray, kmin: np.ndarray) -> np.ndarray:
    """The same bound as two products, S = q+ . max + q- . min, with
    q+ = max(q, 0) and q- = min(q, 0) (the reading of AdaCluster eq. (2)
    under which it equals eq. (1): the key operands are the per-cluster max
    and min vectors)."""
    qp = np.maximum(cq, 0.0)
    qm = np.minimum(cq, 0.0)
    return qp @ kmax.T + qm @ kmin.T


def token_quest_scores(q_tokens: np.ndarray, kmax: np.ndarray, kmin: np.ndarray, count: np.ndarray,
                       chunk: int = 64) -> np.ndarray:
    """Quest bound of every query token against every key cluster: AdaCluster
    Algorithm 2 in its literal shape (one score per query row and key
    column, here per key cluster: [L_q, N_k]), each entry eq. (1):
    S[i, c] = sum_d max(q_i[d] * max(K_c^d), q_i[d] * min(K_c^d)).

    q_tokens are the layer's query rows as they enter attention (not
    normalised).  Empty clusters score -inf.  Rows are processed in chunks
    only to bound memory; each entry is the same per-dimension sum."""
    out = np.empty((q_tokens.shape[0], kmax.shape[0]))
    for i in range(0, q_tokens.shape[0], chunk):
        out[i:i + chunk] = quest_scores(q_tokens[i:i + chunk], kmax, kmin, count)
    return out


def mean_scores(cq: np.ndarray, kmean: np.ndarray, count: np.ndarray) -> np.ndarray:
    """Mean-based cluster score (the "w/o Quest" ablation of AdaCluster
    §4.4): S[r, c] = c_r . mean(K_c)."""
    S = cq @ kmean.T
    S[:, count == 0] = -np.inf
    return S


def scores(p, cq, kst) -> np.ndarray:
    if p.score_mode == SCORE_QUEST:
        return quest_scores(cq, kst["kmax"], kst["kmin"], kst["count"])
    if p.score_mode == SCORE_MEAN:
        return mean_scores(cq, kst["kmean"], kst["count"])
    raise ValueError(p.score_mode)


def order_clusters(S_row: np.ndarray, count: np.ndarray) -> np.ndarray:
    """Non-empty clusters ordered by score descending, ties by index ascending."""
    c = np.nonzero(count > 0)[0]
    return c[np.lexsort((c, -S_row[c]))]


def select_row(S_row, count, rho_r, L, d, p) -> np.ndarray:
    """Key clusters selected for one query cluster (argtopk of AdaCluster
    Algorithm 3, and the budgeted variants).  Returned in selection order.

    TOPK     the first min(K, #non-empty) clusters.
    DENSITY  token budget ceil(rho*L): clusters in order until their summed
             sizes reach the budget (the crossing cluster included).
    TOPP     pi_c = softmax_c(rho_r * S_rc * scale + ln n_c) over non-empty
             clusters (rho_r restores the query magnitude that normalisation
             removed; ln n_c counts the cluster's n_c tokens); the shortest
             prefix in score order whose mass reaches p.
    At least one cluster is always selected; empty clusters never are.
    """
    order = order_clusters(S_row, count)
    if order.size == 0:
        return order
    if p.sel_mode == SEL_TOPK:
        n = min(max(p.topk, 1), order.size)
    elif p.sel_mode == SEL_DENSITY:
        budget = math.ceil(p.sel_param * L)
        cum = np.cumsum(count[order])
        n = int(np.searchsorted(cum, budget, side="left")) + 1
        n = min(max(n, 1), order.size)
    elif p.sel_mode == SEL_TOPP:
        z = rho_r * S_row[order] * p.attn_scale(d) + np.log(count[order].astype(np.float64))
        z = z - np.max(z)
        w = np.exp(z)
        pi = w / np.sum(w)
        cum = np.cumsum(pi)
        n = int(np.searchsorted(cum, p.sel_param, side="left")) + 1
        n = min(max(n, 1), order.size)
    elif p.sel_mode == SEL_DENSE:
        n = order.size
    else:
        raise ValueError(p.sel_mode)
    return order[:n]


def select(S, count, rho, L, d, p):
    return [select_row(S[r], count, rho[r], L, d, p) for r in range(S.shape[0])]
