"""k-means pieces of the oracle (fp64), and query clustering.

Test infrastructure only (see the package docstring).

Readings where the pages are silent (AdaCluster names "KMeans" and
"standard KMeans" without details):
* Euclidean Lloyd iterations with arithmetic-mean centres; on normalised
  queries this is the angular clustering of AdaCluster §3.1 (centres are not
  re-normalised).
* Initialisation: k-means++ (D^2 sampling, Arthur and Vassilvitskii 2007)
  over a strided subsample {floor(j*n/s)} of s = min(n, init_sample*m)
  points (every point when init_sample is 0), driven by the counter-based
  stream of ``numerics.uniform01``.  When every subsample point already
  coincides with a chosen centre the pick falls back to floor(u*s).
* A fixed number of Lloyd iterations, then one final assignment to the last
  centres.  Ties go to the lowest centre index.  An empty cluster keeps its
  previous centre.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, bf16_to_f64, uniform01, stream_id


def normalize_queries(Qbits: np.ndarray) -> np.ndarray:
    """q_hat = q / ||q||_2 rounded to bfloat16 (AdaCluster §3.1 and Appendix
    A.2: the order of q.k over keys does not depend on ||q||).  The norm and
    quotient are taken in float64 and rounded once to bfloat16.  A zero query
    stays zero.  Returns bf16 bits [L, d]."""
    q = bf16_to_f64(Qbits)
    n = np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
    safe = np.where(n > 0, n, 1.0)
    qh = np.where(n > 0, q / safe, 0.0)
    return bf16_round(qh)


def sq_dist(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """||x_i - c_j||^2 for all pairs, via ||x||^2 - 2 x.c + ||c||^2 in fp64
    (checked against the direct difference form in the oracle's tests)."""
    xx = np.sum(X * X, axis=1)[:, None]
    cc = np.sum(C * C, axis=1)[None, :]
    return np.maximum(xx - 2.0 * (X @ C.T) + cc, 0.0)


def sq_dist_direct(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """The plain definition, sum_d (x_d - c_d)^2, for small inputs."""
    diff = X[:, None, :] - C[None, :, :]
    return np.sum(diff * diff, axis=2)


def assign(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Nearest centre of every point (ties -> lowest index)."""
    if C.shape[0] == 0:
        return np.zeros(X.shape[0], dtype=np.int64)
    out = np.empty(X.shape[0], dtype=np.int64)
    step = max(1, 4_000_000 // max(1, C.shape[0]))
    for s in range(0, X.shape[0], step):
        out[s:s + step] = np.argmin(sq_dist(X[s:s + step], C), axis=1)
    return out


def update(X: np.ndarray, labels: np.ndarray, C_prev: np.ndarray) -> np.ndarray:
    """Lloyd update: each centre becomes the mean of its members; an empty
    cluster keeps its previous centre."""
    m = C_prev.shape[0]
    cnt = np.bincount(labels, minlength=m)
    order = np.argsort(labels, kind="stable")
    starts = np.concatenate([[0], np.cumsum(cnt)[:-1]])
    C = C_prev.copy()
    nz = np.nonzero(cnt)[0]
    if nz.size:
        sums = np.add.reduceat(X[order], starts[nz], axis=0)
        C[nz] = sums / cnt[nz][:, None]
    return C


def inertia(X: np.ndarray, labels: np.ndarray, C: np.ndarray) -> float:
    diff = X - C[labels]
    return float(np.sum(diff * diff))


def subsample_index(n: int, m: int, init_sample: int) -> np.ndarray:
    s = n if init_sample <= 0 else min(n, init_sample * m)
    j = np.arange(s, dtype=np.int64)
    return (j * n) // s


def kmeanspp_init(X: np.ndarray, m: int, seed: int, stream: int, init_sample: int):
    """k-means++ seeding on the strided subsample of X (rows in order).

    Returns (centres [m, d] fp64, picked subsample rows as indices into X)."""
    n = X.shape[0]
    idx = subsample_index(n, m, init_sample)
    P = X[idx]
    s = P.shape[0]
    picks = []
    j0 = int(uniform01(seed, stream, 0) * s)
    picks.append(j0)
    diff = P - P[j0]
    D2 = np.sum(diff * diff, axis=1)
    for t in range(1, m):
        u = uniform01(seed, stream, t)
        total_prefix = np.cumsum(D2)
        total = total_prefix[-1]
        if total > 0.0:
            j = int(np.searchsorted(total_prefix, u * total, side="right"))
            j = min(j, s - 1)
        else:
            j = int(u * s)
        picks.append(j)
        diff = P - P[j]
        D2 = np.minimum(D2, np.sum(diff * diff, axis=1))
    picks = np.asarray(picks, dtype=np.int64)
    return P[picks].copy(), idx[picks]


def lloyd(X: np.ndarray, C0: np.ndarray, iters: int, trace: bool = False):
    """``iters`` Lloyd iterations from C0, then a final assignment.

    Returns (C, labels) or, with trace, (C, labels, [C after each update])."""
    C = C0.copy()
    hist = []
    for _ in range(iters):
        lab = assign(X, C)
        C = update(X, lab, C)
        if trace:
            hist.append(C.copy())
    lab = assign(X, C)
    return (C, lab, hist) if trace else (C, lab)


def kmeans(X: np.ndarray, m: int, seed: int, stream: int, iters: int, init_sample: int):
    """Cold k-means: k-means++ seeding, then ``lloyd``."""
    m = min(m, X.shape[0])
    C0, _ = kmeanspp_init(X, m, seed, stream, init_sample)
    return lloyd(X, C0, iters)


def cluster_queries(Qbits: np.ndarray, p, bh: int, warm_cent: np.ndarray | None = None):
    """Query side of Algorithm 3: A_q, C_q <- KMeans(Normalize(Q)) for one head.

    Returns a dict with
      qhat   bf16 bits [L, d] of the normalised queries
      cent   fp64 [m, d] centres (after the last update)
      labels int [L] final assignment
      rho    fp64 [m] mean ||q|| of each cluster's members (0 if empty); the
             top-p temperature uses it to restore the magnitude that
             normalisation removed
      count, perm, seg  (see ``stats.counting_sort``)
    Cold: k-means++ then p.iters iterations.  Warm (AdaCluster §3.2.2,
    "Efficient initialization"): p.iters_warm iterations from warm_cent.
    """
    from .stats import counting_sort
    qh_bits = normalize_queries(Qbits)
    X = bf16_to_f64(qh_bits)
    m = min(p.nq, X.shape[0])
    if warm_cent is None:
        C, lab = kmeans(X, m, p.seed, stream_id(bh, 0, 0), p.iters, p.init_sample)
    else:
        C, lab = lloyd(X, np.asarray(warm_cent, dtype=np.float64)[:m], p.iters_warm)
    qn = np.sqrt(np.sum(bf16_to_f64(Qbits) ** 2, axis=1))
    cnt = np.bincount(lab, minlength=m)
    rho = np.zeros(m)
    np.add.at(rho, lab, qn)
    rho = np.where(cnt > 0, rho / np.maximum(cnt, 1), 0.0)
    perm, seg = counting_sort(lab, m)
    return dict(qhat=qh_bits, cent=C, labels=lab, rho=rho, count=cnt, perm=perm, seg=seg, m=m)
