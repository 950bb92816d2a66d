"""Attention over selected key clusters, with optional stripe-mean
compensation, and dense attention (fp64), one head.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64


def softmax_attend(logits: np.ndarray, values: np.ndarray):
    """o = sum_j softmax(logits)_j v_j per row; also the natural-log
    normaliser lse = log sum_j exp(logits_j)."""
    mx = np.max(logits, axis=1, keepdims=True)
    w = np.exp(logits - mx)
    den = np.sum(w, axis=1, keepdims=True)
    return (w @ values) / den, (mx + np.log(den))[:, 0]


def dense_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, rows: np.ndarray, scale: float):
    """Full attention for the given query rows (AdaCluster Algorithm 3, F
    branch).  Q, K, V are fp64 [L, d]."""
    return softmax_attend((Q[rows] @ K.T) * scale, V)


def sparse_rows(Q, K, V, rows, q_labels, k_labels, selection, scale, compensate=False,
                count=None, kmean=None, vmean=None):
    """Attention of each query row over the keys of its query cluster's
    selected key clusters (AdaCluster Algorithm 3, K* = K[Index];
    ClusterAttention §1.2 eq. (2): softmax normalised over the selected set).

    With ``compensate`` every non-empty excluded cluster c also enters as one
    pseudo-key: logit q.mean(K_c)*scale + ln n_c and value mean(V_c).  This
    is the stripe-mean compensation of ClusterAttention §1.2 eq. (5), with
    the weight ||c|| read as the cluster size n_c (under that reading eq. (5)
    is an exact identity; see the oracle tests).

    Q, K, V fp64 [L, d]; q_labels / k_labels int [L]; selection[r] the
    selected cluster ids of query cluster r.  Returns (O [len(rows), d], lse).
    """
    rows = np.asarray(rows)
    O = np.zeros((rows.size, Q.shape[1]))
    lse = np.zeros(rows.size)
    rq = q_labels[rows]
    for r in np.unique(rq):
        sel = np.asarray(selection[r], dtype=np.int64)
        keymask = np.isin(k_labels, sel)
        kidx = np.nonzero(keymask)[0]
        at = np.nonzero(rq == r)[0]
        q = Q[rows[at]]
        logits = (q @ K[kidx].T) * scale
        vals = V[kidx]
        if compensate:
            m = count.shape[0]
            excl = np.ones(m, dtype=bool)
            excl[sel] = False
            excl &= count > 0
            ex = np.nonzero(excl)[0]
            if ex.size:
                pl = (q @ kmean[ex].T) * scale + np.log(count[ex].astype(np.float64))[None, :]
                logits = np.concatenate([logits, pl], axis=1)
                vals = np.concatenate([vals, vmean[ex]], axis=0)
        O[at], lse[at] = softmax_attend(logits, vals)
    return O, lse


def subset_output(Q, K, V, row, subset, scale):
    """o_S of ClusterAttention §1.2 eq. (2) for one query row and a key
    subset S (indices), with its mass w_S under the full softmax."""
    logits = (Q[row] @ K.T) * scale
    w = np.exp(logits - np.max(logits))
    w = w / np.sum(w)
    wS = np.sum(w[subset])
    oS = (w[subset] @ V[subset]) / wS
    return oS, wS, w


def to_f64(bits):
    return bf16_to_f64(bits)
