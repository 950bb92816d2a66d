"""Interaction-aware key clustering (fp64), one head.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "iCATS: Fast Video Generation via Interaction-Aware Sparse Attention
and Timestep-Adaptive Sparsity", method section, key design 1
(interaction-aware clustering): grouping keys should minimise the error of
the query-key products, sum over clusters t and members j of
||Q (k_j - mu_t)^T||^2 = (k_j - mu_t) Q^T Q (k_j - mu_t)^T, a quadratic
form in the d x d matrix Q^T Q, which the page replaces by the compact
M_Q = sum_r |A_r| mu_r^T mu_r over the query clusters A_r with centroids
mu_r.  Key k-means then assigns each key to the centre c minimising
(k - c) M_Q (k - c)^T.

Readings (the page leaves these open):

* mu_r is the mean of the raw (not normalised) member queries of query
  cluster r: the error concerns the products q.k the attention computes.
  Empty query clusters add nothing.
* The key clusters are a fixed number m of k-means clusters (the page's
  example fixes 1000 key clusters; there is no multi-stage loop and no
  fallback), seeded by the same Euclidean k-means++ as the other k-means
  (k-means++ under the metric is not described).
* The update keeps the member mean: for a positive semi-definite M the mean
  minimises sum_j (k_j - c) M (k_j - c)^T over c.
* Ties go to the lowest centre index; an empty cluster keeps its centre; a
  final assignment follows the last update (as the Euclidean k-means).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64, stream_id
from .kmeans import kmeanspp_init, update


def interaction_matrix(Qbits: np.ndarray, labels: np.ndarray, nq: int) -> np.ndarray:
    """M_Q = sum_r |A_r| mu_r^T mu_r (d x d) with mu_r the mean raw query of
    query cluster r."""
    Q = bf16_to_f64(Qbits)
    d = Q.shape[1]
    M = np.zeros((d, d))
    for r in range(nq):
        members = Q[labels == r]
        n = members.shape[0]
        if n == 0:
            continue
        mu = members.mean(axis=0)
        M += n * np.outer(mu, mu)
    return M


def metric_sq_dist(X: np.ndarray, C: np.ndarray, M: np.ndarray, chunk: int = 256) -> np.ndarray:
    """(x_i - c_j) M (x_i - c_j)^T for all pairs, the quadratic form as
    written (differences first: each difference times M, then its dot
    product with the difference), in row chunks."""
    out = np.empty((X.shape[0], C.shape[0]))
    for s in range(0, X.shape[0], chunk):
        diff = X[s:s + chunk, None, :] - C[None, :, :]
        out[s:s + chunk] = np.sum((diff @ M) * diff, axis=2)
    return out


def assign_metric(X: np.ndarray, C: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Centre minimising the quadratic form for every point (ties -> lowest)."""
    return np.argmin(metric_sq_dist(X, C, M), axis=1)


def lloyd_metric(X: np.ndarray, C0: np.ndarray, M: np.ndarray, iters: int, trace: bool = False):
    """``iters`` Lloyd iterations under the metric, then a final assignment."""
    C = C0.copy()
    hist = []
    for _ in range(iters):
        lab = assign_metric(X, C, M)
        C = update(X, lab, C)
        if trace:
            hist.append((lab.copy(), C.copy()))
    lab = assign_metric(X, C, M)
    return (C, lab, hist) if trace else (C, lab)


def objective(X: np.ndarray, labels: np.ndarray, C: np.ndarray, M: np.ndarray) -> float:
    diff = X - C[labels]
    return float(np.einsum("ik,kl,il->", diff, M, diff))


def cluster_keys_metric(Kbits: np.ndarray, p, bh: int, M: np.ndarray):
    """Fixed-count (m = min(m0, L)) interaction-aware k-means of one head's
    keys: Euclidean k-means++ seeding (stream of stage 0 of the keys), then
    p.iters Lloyd iterations under M, then the final assignment."""
    X = bf16_to_f64(Kbits)
    m = min(p.m0, X.shape[0])
    C0, _ = kmeanspp_init(X, m, p.seed, stream_id(bh, 1, 0), p.init_sample)
    C, lab = lloyd_metric(X, C0, M, p.iters)
    return dict(cent=C, labels=lab, nk=m, C0=C0)
