"""Per-cluster statistics and the cluster-order permutation (fp64 / int).

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64


def counting_sort(labels: np.ndarray, m: int):
    """Stable sort of token indices by cluster label (the gather
    K* = K[Index] of AdaCluster Algorithm 3 needs each cluster's tokens
    contiguous).  Returns (perm, seg): perm[p] is the original index of the
    p-th token in cluster order, seg[c] the first position of cluster c
    (seg[m] = n)."""
    labels = np.asarray(labels, dtype=np.int64)
    perm = np.argsort(labels, kind="stable")
    cnt = np.bincount(labels, minlength=m)
    seg = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
    return perm, seg


def key_stats(Kbits: np.ndarray, Vbits: np.ndarray, labels: np.ndarray, cent: np.ndarray):
    """Statistics of the final key clusters of one head.

    count  n_c
    kmax   per-dimension max of member keys (AdaCluster eq. (1): max(K^d)),
           kmin per-dimension min; both are exact bf16 values (fp64 here)
    kmean  member mean of K, vmean member mean of V (the key and value
           centroids of ClusterAttention §1.2, used by stripe-mean
           compensation and by mean-based scoring)
    mse    (1/L) sum_i ||k_i - c(k_i)||^2 with c the assigned centre
           (AdaCluster §3.2.1, per head), and comp = 1/mse
    Empty clusters get count 0 and zeros elsewhere.
    """
    K = bf16_to_f64(Kbits)
    V = bf16_to_f64(Vbits)
    m, d = cent.shape
    cnt = np.bincount(labels, minlength=m)
    kmax = np.zeros((m, d))
    kmin = np.zeros((m, d))
    kmean = np.zeros((m, d))
    vmean = np.zeros((m, d))
    order = np.argsort(labels, kind="stable")
    starts = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    nz = np.nonzero(cnt)[0]
    if nz.size:
        Ks, Vs = K[order], V[order]
        kmax[nz] = np.maximum.reduceat(Ks, starts[nz], axis=0)
        kmin[nz] = np.minimum.reduceat(Ks, starts[nz], axis=0)
        kmean[nz] = np.add.reduceat(Ks, starts[nz], axis=0) / cnt[nz][:, None]
        vmean[nz] = np.add.reduceat(Vs, starts[nz], axis=0) / cnt[nz][:, None]
    diff = K - cent[labels]
    mse = float(np.sum(diff * diff) / K.shape[0])
    return dict(count=cnt, kmax=kmax, kmin=kmin, kmean=kmean, vmean=vmean, mse=mse,
                comp=(1.0 / mse if mse > 0 else np.inf))
