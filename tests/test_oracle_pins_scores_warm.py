"""Pins of the oracle's mean-based scores, the query-norm means rho, the
warm (later denoising step) paths, the top-p temperature and the
percentile rule for tau, against facts the pages and the mathematics fix.

Each test names the passage it follows.  CPU only."""
import math

import numpy as np

from oracle import numerics as nm
from oracle import kmeans as okm
from oracle import multistage as oms
from oracle import stats as ost
from oracle import score as osc
from oracle import layer as oly


def _rng(s):
    return np.random.default_rng(s)


def _bits(X):
    """fp64 values -> bf16 bit patterns (values already on the bf16 grid stay exact)."""
    return nm.bf16_round(X)


# ---------------------------------------------------------------- mean-based scores

def test_mean_scores_singletons_equal_quest_and_dot():
    """AdaCluster eq. (1) and the mean score of its "w/o Quest" ablation
    (§4.4): for a cluster of one key, max = min = mean = k, so both scores
    equal q.k exactly; an empty cluster scores -inf in both."""
    r = _rng(1)
    K = nm.bf16_to_f64(_bits(r.standard_normal((20, 16))))
    V = nm.bf16_to_f64(_bits(r.standard_normal((20, 16))))
    labels = np.arange(20)
    labels[7] = 6                               # cluster 7 empty, cluster 6 has two members
    cent = np.zeros((20, 16))
    kst = ost.key_stats(_bits(K), _bits(V), labels, cent)
    cq = r.standard_normal((3, 16))
    S_mean = osc.scores(nm.Params(score_mode=nm.SCORE_MEAN), cq, kst)
    S_quest = osc.scores(nm.Params(score_mode=nm.SCORE_QUEST), cq, kst)
    single = [c for c in range(20) if c not in (6, 7)]
    dots = cq @ K.T
    assert np.allclose(S_mean[:, single], dots[:, single], rtol=0, atol=1e-13)
    assert np.allclose(S_quest[:, single], dots[:, single], rtol=0, atol=1e-13)
    assert np.all(np.isneginf(S_mean[:, 7])) and np.all(np.isneginf(S_quest[:, 7]))
    # the two-member cluster: the mean score is the average of the two dot products
    assert np.allclose(S_mean[:, 6], 0.5 * (dots[:, 6] + dots[:, 7]), rtol=0, atol=1e-13)


def test_mean_scores_are_member_averages_not_centres():
    """The mean score uses each cluster's member mean of K (the key centroid
    of ClusterAttention §1.2), so by linearity S[r, c] is the average of
    q_r.k over the members.  The centres passed to key_stats are set far
    from the member means: a score built from them would fail."""
    r = _rng(2)
    n, d, m = 300, 12, 9
    K = nm.bf16_to_f64(_bits(r.standard_normal((n, d))))
    V = nm.bf16_to_f64(_bits(r.standard_normal((n, d))))
    labels = r.integers(0, m, n)
    labels[labels == 4] = 5                     # cluster 4 empty
    cent = 10.0 + r.standard_normal((m, d))     # not the member means
    kst = ost.key_stats(_bits(K), _bits(V), labels, cent)
    cq = r.standard_normal((5, d))
    S = osc.scores(nm.Params(score_mode=nm.SCORE_MEAN), cq, kst)
    for c in range(m):
        members = np.nonzero(labels == c)[0]
        if members.size == 0:
            assert np.all(np.isneginf(S[:, c]))
            continue
        for q in range(5):
            avg = sum(float(cq[q] @ K[i]) for i in members) / members.size
            assert abs(S[q, c] - avg) < 1e-12 * max(1.0, abs(avg))


# ---------------------------------------------------------------- rho: mean query norm per cluster

def test_rho_weighted_sum_is_total_query_norm():
    """rho_r is the mean ||q|| of cluster r's members (the magnitude that the
    normalisation of AdaCluster §3.1 removes), so sum_r n_r rho_r equals
    sum_i ||q_i|| and empty clusters carry 0."""
    r = _rng(3)
    L, d = 700, 16
    dirs = r.standard_normal((5, d))
    z = r.integers(0, 5, L)
    Q = (dirs[z] + 0.1 * r.standard_normal((L, d))) * r.lognormal(0, 0.5, (L, 1))
    Qb = _bits(Q)
    p = nm.Params(nq=8, iters=6, init_sample=0, seed=4)
    qc = okm.cluster_queries(Qb, p, 0)
    qn = np.linalg.norm(nm.bf16_to_f64(Qb), axis=1)
    cnt = np.bincount(qc["labels"], minlength=qc["m"])
    assert np.array_equal(cnt, qc["count"])
    assert abs(np.sum(cnt * qc["rho"]) - qn.sum()) < 1e-9 * qn.sum()
    assert np.all(qc["rho"][cnt == 0] == 0.0)
    for c in np.nonzero(cnt)[0]:
        assert qn[qc["labels"] == c].min() - 1e-12 <= qc["rho"][c] <= qn[qc["labels"] == c].max() + 1e-12


def test_rho_hand_built_two_directions():
    """Three queries along e1 with norms 1, 2, 3 and three along e2 with
    norms 4, 5, 6: two angular clusters whose mean norms are 2 and 5."""
    d = 8
    Q = np.zeros((6, d))
    Q[0:3, 0] = [1.0, 2.0, 3.0]
    Q[3:6, 1] = [4.0, 5.0, 6.0]
    p = nm.Params(nq=2, iters=3, init_sample=0, seed=1)
    qc = okm.cluster_queries(_bits(Q), p, 0)
    a, b = qc["labels"][0], qc["labels"][3]
    assert a != b and np.all(qc["labels"][:3] == a) and np.all(qc["labels"][3:] == b)
    assert qc["rho"][a] == 2.0 and qc["rho"][b] == 5.0
    assert np.array_equal(qc["cent"][a], np.eye(d)[0]) and np.array_equal(qc["cent"][b], np.eye(d)[1])


# ---------------------------------------------------------------- warm step

def _mixture(seed, n=600, d=8, k=6, spread=0.3):
    r = _rng(seed)
    mu = 3.0 * r.standard_normal((k, d))
    z = r.integers(0, k, n)
    return nm.bf16_to_f64(_bits(mu[z] + spread * r.standard_normal((n, d))))


def test_warm_keys_zero_iterations_nearest_to_carried_centres():
    """AdaCluster §3.2.2 "Efficient initialization": a later step keeps the
    cluster count and starts from the previous centres.  With no Lloyd
    iteration the centres are the carried ones and each key takes the
    nearest of them (plain difference form, ties to the lowest index)."""
    K = _mixture(5)
    r = _rng(6)
    C_prev = K[r.choice(K.shape[0], 9, replace=False)] + 0.05
    out = oms.warm_keys(_bits(K), nm.Params(iters_warm=0), C_prev)
    assert out["nk"] == 9 and np.array_equal(out["cent"], C_prev)
    d2 = okm.sq_dist_direct(K, C_prev)
    assert np.array_equal(out["labels"], np.argmin(d2, axis=1))


def test_warm_keys_one_iteration_is_member_mean():
    """One warm Lloyd iteration: every centre becomes the mean of the keys
    nearest to it among the carried centres; a centre nobody chose stays."""
    K = _mixture(7)
    C_prev = np.concatenate([K[:5] + 0.01, np.full((1, K.shape[1]), 1e3)])  # the last centre wins nothing
    out = oms.warm_keys(_bits(K), nm.Params(iters_warm=1), C_prev)
    near = np.argmin(okm.sq_dist_direct(K, C_prev), axis=1)
    for c in range(C_prev.shape[0]):
        mem = K[near == c]
        if mem.size == 0:
            assert np.array_equal(out["cent"][c], C_prev[c])
        else:
            ref = np.array([sum(mem[:, j]) / mem.shape[0] for j in range(K.shape[1])])
            assert np.allclose(out["cent"][c], ref, rtol=0, atol=1e-12)
    assert np.array_equal(out["labels"], np.argmin(okm.sq_dist_direct(K, out["cent"]), axis=1))


def test_warm_step_from_converged_state_is_a_fixed_point():
    """Lloyd's fixed point: from centres whose assignment no longer changes,
    warm iterations (keys and queries) return exactly those centres and
    labels, whatever iters_warm is."""
    K = _mixture(8)
    C = K[:7].copy()
    prev = None
    for _ in range(200):
        lab = okm.assign(K, C)
        if prev is not None and np.array_equal(lab, prev):
            break
        C, prev = okm.update(K, lab, C), lab
    else:
        raise AssertionError("no fixed point within 200 iterations")
    for it in (1, 3, 5):
        out = oms.warm_keys(_bits(K), nm.Params(iters_warm=it), C)
        assert np.array_equal(out["cent"], C) and np.array_equal(out["labels"], lab)
    # queries: converge cold, then warm from the converged centres
    Qb = _bits(_mixture(9, d=12) + 0.5)
    pc = nm.Params(nq=5, iters=200, init_sample=0, seed=2)
    cold = okm.cluster_queries(Qb, pc, 0)
    warm = okm.cluster_queries(Qb, nm.Params(nq=5, iters_warm=3), 0, warm_cent=cold["cent"])
    assert np.array_equal(warm["cent"], cold["cent"]) and np.array_equal(warm["labels"], cold["labels"])
    assert np.array_equal(warm["rho"], cold["rho"])


def test_warm_queries_zero_iterations_nearest_to_carried_centres():
    Qb = _bits(_mixture(10, d=12) + 0.5)
    X = nm.bf16_to_f64(okm.normalize_queries(Qb))
    C_prev = X[[3, 50, 99, 200]] * 0.9
    out = okm.cluster_queries(Qb, nm.Params(nq=4, iters_warm=0), 0, warm_cent=C_prev)
    assert np.array_equal(out["cent"], C_prev)
    assert np.array_equal(out["labels"], np.argmin(okm.sq_dist_direct(X, C_prev), axis=1))


def test_run_head_warm_carries_counts_flag_and_tau():
    """The warm step carries N_k, the fallback flag and tau from the cold
    step and runs no stage of Algorithm 1 (AdaCluster §3.2.2)."""
    import csa_inputs as gen
    w = gen.get_workload("tiny", H=1, L=512)
    Q, K, V = gen.generate(w)
    p = nm.Params(nq=8, m0=8, nmax=40, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, sel_mode=nm.SEL_TOPK, topk=4,
                  init_sample=0, iters=5, iters_warm=2)
    cold = oly.run_head(Q[0, 0], K[0, 0], V[0, 0], p, 0)
    warm = oly.run_head(Q[0, 0], K[0, 0], V[0, 0], p, 0, warm=cold["state"])
    assert warm["k"]["nk"] == cold["k"]["nk"] and warm["k"]["fallback"] == cold["k"]["fallback"]
    assert warm["k"]["tau"] == cold["k"]["tau"] and warm["k"]["stages"] == 0
    assert warm["q"]["m"] == cold["q"]["m"]


# ---------------------------------------------------------------- top-p temperature

def test_topp_mass_equals_attention_mass_of_each_cluster():
    """Top-p on softmaxed centroid scores (the Wan workload; iCATS's top-p):
    with pi_c = softmax(rho_r * S_rc * scale + ln n_c) and one query per
    query cluster along a coordinate axis (so the normalised query is exact),
    key clusters of n_c identical keys make pi_c exactly the attention
    probability mass the query puts on cluster c, computed here by brute
    force over every key.  The selection is the shortest score-ordered
    prefix whose attention mass reaches p.  A missing rho, scale or
    multiplicity term, or another log base, breaks the equality."""
    r = _rng(11)
    d, nk = 16, 12
    sizes = r.integers(1, 9, nk)
    sizes[4] = 0
    kc = nm.bf16_to_f64(_bits(0.8 * r.standard_normal((nk, d))))
    K = np.concatenate([np.repeat(kc[c:c + 1], sizes[c], axis=0) for c in range(nk)])
    klab = np.concatenate([np.full(sizes[c], c) for c in range(nk)])
    V = np.zeros_like(K)
    kst = ost.key_stats(_bits(K), _bits(V), klab, np.zeros((nk, d)))
    Qv = np.zeros((4, d))
    Qv[0, 0], Qv[1, 3], Qv[2, 7], Qv[3, 3] = 3.0, -2.5, 1.75, 0.5
    qc = okm.cluster_queries(_bits(Qv), nm.Params(nq=4, iters=2, init_sample=0, seed=3), 0)
    L = K.shape[0]
    scale = 1.0 / math.sqrt(d)
    for pv in (0.5, 0.8, 0.9, 0.99):
        p = nm.Params(sel_mode=nm.SEL_TOPP, sel_param=pv, score_mode=nm.SCORE_QUEST)
        S = osc.scores(p, qc["cent"], kst)
        sel = osc.select(S, kst["count"], qc["rho"], L, d, p)
        for i in range(4):
            r_ = qc["labels"][i]
            logits = (Qv[i] @ K.T) * scale                   # brute force over all keys
            w = np.exp(logits - logits.max())
            w /= w.sum()
            mass = np.bincount(klab, weights=w, minlength=nk)
            order = sorted([c for c in range(nk) if sizes[c] > 0], key=lambda c: (-S[r_, c], c))
            cum = np.cumsum(mass[order])
            k = int(np.searchsorted(cum, pv - 1e-12, side="left")) + 1
            assert sel[r_].tolist() == order[:k], (pv, i)


# ---------------------------------------------------------------- percentile rule of tau

def test_stage_tau_percentile_is_inverted_cdf():
    """The percentile threshold (CogVideoX workload, "95th-percentile
    distance") read as nearest rank: the smallest distance whose empirical
    CDF reaches the level, which is numpy's inverted-CDF percentile."""
    r = _rng(12)
    for n in (1, 2, 7, 100, 1001):
        dist = r.exponential(1.0, n)
        for q in (0.05, 0.5, 0.9, 0.95, 1.0):
            got = oms.stage_tau(dist, nm.TAU_PCTL, q)
            ref = float(np.percentile(dist, 100.0 * q, method="inverted_cdf"))
            assert got == ref, (n, q)
