"""Pins of the oracle's interaction-aware key clustering (CPU only): M_Q in
its two limiting cases, the page's identity between the quadratic form and
the query-key product error, and the metric k-means against plain k-means
(identity metric) and against Euclidean k-means on linearly transformed
keys (a metric A^T A), with the Lloyd objective never growing."""
import numpy as np

import csa_inputs as gen
from oracle import numerics as nm
from oracle import interaction as oia
from oracle import kmeans as okm


def _bits(x):
    return nm.bf16_round(x)


def test_interaction_matrix_limits():
    rng = np.random.default_rng(2)
    Qb = _bits(rng.normal(size=(40, 6)))
    Q = nm.bf16_to_f64(Qb)
    # every query its own cluster: Q^T Q
    M = oia.interaction_matrix(Qb, np.arange(40), 40)
    assert np.allclose(M, Q.T @ Q, rtol=1e-13, atol=1e-12)
    # one cluster: L mu mu^T
    M1 = oia.interaction_matrix(Qb, np.zeros(40, dtype=np.int64), 3)
    mu = Q.mean(axis=0)
    assert np.allclose(M1, 40 * np.outer(mu, mu), rtol=1e-13, atol=1e-12)
    # M_Q is symmetric positive semi-definite, and never above Q^T Q (Jensen per cluster)
    lab = rng.integers(0, 5, size=40)
    M5 = oia.interaction_matrix(Qb, lab, 5)
    assert np.allclose(M5, M5.T)
    assert np.min(np.linalg.eigvalsh(M5)) > -1e-9
    assert np.min(np.linalg.eigvalsh(Q.T @ Q - M5)) > -1e-9


def test_quadratic_form_is_the_product_error():
    rng = np.random.default_rng(4)
    Q = rng.normal(size=(30, 5))
    K = rng.normal(size=(12, 5))
    C = rng.normal(size=(3, 5))
    D = oia.metric_sq_dist(K, C, Q.T @ Q, chunk=5)
    direct = np.array([[np.sum((Q @ (k - c)) ** 2) for c in C] for k in K])
    assert np.allclose(D, direct, rtol=1e-12, atol=1e-12)


def test_identity_metric_is_plain_kmeans():
    w = gen.get_workload("tiny")
    _, Kb, _ = gen.generate(w, heads=[0])
    X = nm.bf16_to_f64(Kb[0, 0][:600])
    C0, _ = okm.kmeanspp_init(X, 12, 3, 7, 0)
    Ce, le = okm.lloyd(X, C0, 6)
    Cm, lm = oia.lloyd_metric(X, C0, np.eye(X.shape[1]), 6)
    assert np.array_equal(le, lm)
    assert np.allclose(Ce, Cm, rtol=1e-12, atol=1e-12)


def test_metric_equals_euclidean_on_transformed_keys():
    rng = np.random.default_rng(9)
    w = gen.get_workload("tiny")
    _, Kb, _ = gen.generate(w, heads=[1])
    X = nm.bf16_to_f64(Kb[0, 1][:500])
    d = X.shape[1]
    A = rng.normal(size=(d, d)) / np.sqrt(d) + np.eye(d)
    M = A.T @ A  # (x - c) M (x - c)^T = ||(x - c) A^T||^2
    C0 = X[rng.choice(X.shape[0], 10, replace=False)]
    Cm, lm, hist = oia.lloyd_metric(X, C0, M, 5, trace=True)
    Y = X @ A.T
    Ce, le = okm.lloyd(Y, C0 @ A.T, 5)
    assert np.array_equal(lm, le)
    assert np.allclose(Cm @ A.T, Ce, rtol=1e-9, atol=1e-9)
    # Lloyd never increases the objective
    objs = [oia.objective(X, lab, C, M) for lab, C in hist]
    assert all(b <= a * (1 + 1e-12) for a, b in zip(objs, objs[1:]))
