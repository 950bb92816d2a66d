"""ClusterAttention's clustering by recursive splitting along principal
components into clusters of a preset power-of-two size (fp64), one head.

Test infrastructure only (see the package docstring).

The page ("ClusterAttention: training-free acceleration of bidirectional
attention") states: the clustering is fast and recursive, runs per head and
separately for keys and queries, adapts to each head's geometry, lets the
cluster size be set freely, and the method fixes every cluster size to a
power of two so that block-sparse attention costs about what dense attention
costs per key-query interaction (abstract); it splits recursively along
principal components to produce clusters of a preset size (end of section 2);
the method section breaks off mid-sentence as it begins to describe an
approximate projection of the key or query set.  Readings taken here:

* A node of n > b points is cut in two by its leading principal direction:
  the points are ordered by their projection onto it (ties: lower token
  index first) and the first n_left = b * ceil(ceil(n / b) / 2) go left, the
  rest right; nodes of at most b points are clusters.  Every cluster then
  holds exactly b points except at most one (the last), and the tree's shape
  depends only on n and b.
* The direction is the leading right singular vector of the node's
  mean-centred points, taken on a strided subsample {floor(j n / s)} of
  s = min(n, sample) points (the approximation the page mentions; the GPU
  approximates this vector by power iteration).  Its sign makes the
  component of largest magnitude positive (lowest index among equal
  magnitudes).
* Children keep their parent's token order (the split is a stable
  partition), so each cluster lists its tokens in ascending index order and
  the cluster order is the tree's left-to-right leaf order.
"""
from __future__ import annotations

import math

import numpy as np


def split_sizes(n: int, b: int) -> tuple[int, int]:
    """(n_left, n_right) of a node of n > b points."""
    nb = -(-n // b)
    nl = b * -(-nb // 2)
    return nl, n - nl


def leaf_sizes(n: int, b: int) -> list[int]:
    """Cluster sizes of the whole tree, left to right (shape only)."""
    if n <= b:
        return [n] if n > 0 else []
    nl, nr = split_sizes(n, b)
    return leaf_sizes(nl, b) + leaf_sizes(nr, b)


def subsample(n: int, s: int) -> np.ndarray:
    s = min(n, s)
    return (np.arange(s, dtype=np.int64) * n) // s


def orient(v: np.ndarray) -> np.ndarray:
    """Sign convention: the component of largest magnitude is positive."""
    i = int(np.argmax(np.abs(v)))
    return v if v[i] >= 0 else -v


def principal_direction(P: np.ndarray) -> np.ndarray:
    """Leading right singular vector of the mean-centred rows of P (fp64)."""
    Y = P - P.mean(axis=0)
    if not np.any(Y):
        v = np.zeros(P.shape[1])
        v[0] = 1.0
        return v
    _, _, vt = np.linalg.svd(Y, full_matrices=False)
    return orient(vt[0])


def split_node(X: np.ndarray, idx: np.ndarray, b: int, v: np.ndarray):
    """Split the points idx (ascending token indices) of one node by the
    direction v: the n_left smallest projections (ties by token index) go
    left.  Both children keep ascending token order."""
    nl, _ = split_sizes(idx.size, b)
    p = X[idx] @ v
    order = np.lexsort((idx, p))
    left = np.zeros(idx.size, dtype=bool)
    left[order[:nl]] = True
    return idx[left], idx[~left]


def pca_split(X: np.ndarray, b: int, sample: int, trace: bool = False):
    """Cluster the rows of X (fp64 [n, d]) into power-of-two-sized clusters.

    Returns a dict: labels [n] (cluster id in left-to-right leaf order),
    perm / seg (tokens in cluster order, cluster starts), sizes, cent (member
    means), and with trace the list of internal nodes in breadth-first order,
    each (level, token indices, direction)."""
    n = X.shape[0]
    if b < 1 or (b & (b - 1)) != 0:
        raise ValueError("cluster size must be a power of two")
    leaves = []
    nodes = []

    def rec(idx, level):
        if idx.size <= b:
            if idx.size:
                leaves.append(idx)
            return
        v = principal_direction(X[idx[subsample(idx.size, sample)]])
        if trace:
            nodes.append((level, idx, v))
        lo, hi = split_node(X, idx, b, v)
        rec(lo, level + 1)
        rec(hi, level + 1)

    rec(np.arange(n, dtype=np.int64), 0)
    labels = np.empty(n, dtype=np.int64)
    for c, idx in enumerate(leaves):
        labels[idx] = c
    sizes = np.array([x.size for x in leaves], dtype=np.int64)
    perm = np.concatenate(leaves) if leaves else np.zeros(0, dtype=np.int64)
    seg = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    cent = np.stack([X[x].mean(axis=0) for x in leaves]) if leaves else np.zeros((0, X.shape[1]))
    out = dict(labels=labels, perm=perm, seg=seg, sizes=sizes, cent=cent, nclusters=len(leaves))
    if trace:
        nodes.sort(key=lambda t: t[0])
        out["nodes"] = nodes
    return out


def levels(n: int, b: int) -> int:
    """Number of split levels of the tree (0 when n <= b)."""
    return 0 if n <= b else 1 + max(levels(m, b) for m in split_sizes(n, b))


def n_clusters(n: int, b: int) -> int:
    return math.ceil(n / b) if n > 0 else 0
