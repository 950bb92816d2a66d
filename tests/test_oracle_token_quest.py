"""Pins of the oracle's per-token Quest scores (AdaCluster Algorithm 2 in its
literal shape: every query token against every key cluster, each entry
eq. (1)).  CPU only.

Quest is the maximum of the linear function k -> q.k over the axis-aligned
bounding box of the cluster's keys, which a linear function attains at a
corner of the box.  The corner brute force below is therefore an
independent definition of the same number; the member bound and the
singleton case tie it to the keys themselves."""
import itertools

import numpy as np

import csa_inputs as gen
from oracle import numerics as nm
from oracle import score as osc


def _clusters(K, labels, n):
    kmax = np.stack([K[labels == c].max(0) if np.any(labels == c) else np.zeros(K.shape[1]) for c in range(n)])
    kmin = np.stack([K[labels == c].min(0) if np.any(labels == c) else np.zeros(K.shape[1]) for c in range(n)])
    count = np.bincount(labels, minlength=n)
    return kmax, kmin, count


def test_token_quest_is_the_max_over_box_corners():
    rng = np.random.default_rng(31)
    d, n = 5, 6
    K = rng.normal(size=(90, d))
    labels = rng.integers(0, n, size=90)
    kmax, kmin, count = _clusters(K, labels, n)
    Q = rng.normal(size=(40, d)) * rng.lognormal(size=(40, 1))
    S = osc.token_quest_scores(Q, kmax, kmin, count, chunk=7)
    for c in range(n):
        corners = np.array([[kmax[c, j] if b[j] else kmin[c, j] for j in range(d)]
                            for b in itertools.product([0, 1], repeat=d)])
        brute = np.max(Q @ corners.T, axis=1)
        assert np.allclose(S[:, c], brute, rtol=1e-12, atol=1e-12)


def test_token_quest_bounds_every_member_and_is_exact_on_singletons():
    w = gen.get_workload("tiny")
    Qb, Kb, _ = gen.generate(w, heads=[0])
    Q = nm.bf16_to_f64(Qb.reshape(-1, w.L, w.d)[0][:300])
    K = nm.bf16_to_f64(Kb.reshape(-1, w.L, w.d)[0][:200])
    labels = np.arange(200) % 9
    labels[199] = 9  # a cluster of one key
    kmax, kmin, count = _clusters(K, labels, 10)
    S = osc.token_quest_scores(Q, kmax, kmin, count)
    dots = Q @ K.T
    for c in range(10):
        m = labels == c
        assert np.all(S[:, c] >= np.max(dots[:, m], axis=1) - 1e-12)
    assert np.allclose(S[:, 9], dots[:, 199], rtol=1e-13, atol=1e-13)


def test_token_quest_chunks_and_empty_clusters():
    rng = np.random.default_rng(5)
    d = 16
    K = rng.normal(size=(64, d))
    labels = rng.integers(0, 4, size=64) * 2  # clusters 1, 3, 5, 7 stay empty
    kmax, kmin, count = _clusters(K, labels, 8)
    Q = rng.normal(size=(130, d))
    a = osc.token_quest_scores(Q, kmax, kmin, count, chunk=64)
    b = osc.token_quest_scores(Q, kmax, kmin, count, chunk=1000)
    assert np.array_equal(a, b)
    assert np.all(np.isneginf(a[:, count == 0])) and np.all(np.isfinite(a[:, count > 0]))
    # the split form of eq. (2) with the max / min vectors gives the same numbers
    c = osc.quest_scores_split(Q, kmax, kmin)
    assert np.allclose(a[:, count > 0], c[:, count > 0], rtol=1e-12, atol=1e-12)
