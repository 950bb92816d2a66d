"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test names the passage (page title + section / equation) it checks.
These run on the CPU (no GPU marker)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import numerics as nm
from oracle import kmeans as okm
from oracle import multistage as oms
from oracle import stats as ost
from oracle import score as osc
from oracle import attention as oat
from oracle import layer as oly
import csa_inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(s):
    return np.random.default_rng(s)


# ---------------------------------------------------------------- numerics

def test_splitmix64_published_sequence():
    """SplitMix64 (Steele, Lea, Flood 2014) seeded with 0: the first three
    outputs of the public reference implementation."""
    s = 0
    outs = []
    for _ in range(3):
        s, z = nm.splitmix64_next(s)
        outs.append(z)
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_uniform01_range_and_spread():
    u = np.array([nm.uniform01(7, nm.stream_id(3, 1, 2), t) for t in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01
    h, _ = np.histogram(u, bins=10, range=(0, 1))
    assert h.min() > 1800 and h.max() < 2200
    # different streams give different sequences
    v = np.array([nm.uniform01(7, nm.stream_id(3, 1, 3), t) for t in range(100)])
    assert not np.allclose(u[:100], v)


def test_bf16_round_matches_torch_on_float32_values():
    """For float32-representable inputs, the oracle's direct float64 rounding
    equals torch's float32 -> bfloat16 conversion (round to nearest even)."""
    import torch
    x = _rng(0).standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # add exact ties: values halfway between two bf16 numbers
    base = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x[:1000]))
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1.0, -2.5])])
    ours = nm.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_float64_is_nearest():
    """Brute force: the result is the nearer of the two bracketing bf16
    values (ties to the even one) for float64 inputs that float32 cannot
    hold."""
    x = _rng(1).standard_normal(5000) * 2.0 + 1e-9 * _rng(2).standard_normal(5000)
    b = nm.bf16_round(x)
    v = nm.bf16_to_f64(b)
    up = nm.bf16_to_f64((b.astype(np.int64) + np.where(x >= 0, 1, -1)).astype(np.uint16))
    dn = nm.bf16_to_f64((b.astype(np.int64) - np.where(x >= 0, 1, -1)).astype(np.uint16))
    err = np.abs(x - v)
    assert np.all(err <= np.abs(x - up))
    assert np.all(err <= np.abs(x - dn))


# ---------------------------------------------------------------- query normalisation

def test_normalisation_order_invariance():
    """AdaCluster Appendix A.2: for ||q|| > 0, q.ka > q.kb iff q_hat.ka > q_hat.kb,
    so top-K over keys is the same for q and q/||q||."""
    r = _rng(3)
    K = r.standard_normal((500, 64))
    for _ in range(20):
        q = r.standard_normal(64) * r.lognormal(0, 1)
        qh = q / np.linalg.norm(q)
        a, b = np.argsort(-(K @ q), kind="stable"), np.argsort(-(K @ qh), kind="stable")
        assert np.array_equal(a[:50], b[:50])


def test_normalize_queries_unit_norm_and_zero():
    r = _rng(4)
    q = r.standard_normal((100, 128)) * r.lognormal(0, 0.5, (100, 1))
    q[7] = 0.0
    qb = nm.bf16_round(q)
    qh = nm.bf16_to_f64(okm.normalize_queries(qb))
    n = np.linalg.norm(qh, axis=1)
    assert np.all(np.abs(n[np.arange(100) != 7] - 1.0) < 2.0 ** -7)
    assert np.all(qh[7] == 0.0)
    # each element is the bf16 rounding of the exact quotient
    qq = nm.bf16_to_f64(qb)
    exact = qq[0] / np.linalg.norm(qq[0])
    assert np.array_equal(okm.normalize_queries(qb)[0], nm.bf16_round(exact))


# ---------------------------------------------------------------- k-means

def test_sq_dist_expansion_equals_direct():
    r = _rng(5)
    X, C = r.standard_normal((300, 64)), r.standard_normal((17, 64))
    assert np.allclose(okm.sq_dist(X, C), okm.sq_dist_direct(X, C), rtol=1e-12, atol=1e-10)
    lab = okm.assign(X, C)
    assert np.array_equal(lab, np.argmin(okm.sq_dist_direct(X, C), axis=1))


def test_assign_ties_lowest_index():
    X = np.array([[0.0, 0.0], [1.0, 0.0]])
    C = np.array([[1.0, 1.0], [1.0, -1.0], [1.0, 1.0]])
    assert list(okm.assign(X, C)) == [0, 0]


def test_lloyd_matches_sklearn_given_init():
    """Lloyd iterations from a fixed init equal scikit-learn's Lloyd KMeans
    (n_init=1, tol=0) when no cluster empties."""
    from sklearn.cluster import KMeans
    r = _rng(6)
    cen = r.standard_normal((6, 8)) * 4
    X = cen[r.integers(0, 6, 600)] + r.standard_normal((600, 8))
    C0 = X[[0, 100, 200, 300, 400, 500]].copy()
    C, lab = okm.lloyd(X, C0, 5)
    km = KMeans(n_clusters=6, init=C0, n_init=1, max_iter=5, tol=0.0, algorithm="lloyd").fit(X)
    assert np.array_equal(lab, km.predict(X))
    assert np.allclose(C, km.cluster_centers_, rtol=1e-10, atol=1e-10)


def test_lloyd_inertia_non_increasing():
    """Textbook Lloyd property: inertia never increases across iterations."""
    r = _rng(7)
    X = r.standard_normal((2000, 16)) + (r.integers(0, 10, (2000, 1)) * 0.7)
    C0, _ = okm.kmeanspp_init(X, 12, 1, 5, 0)
    C, lab, hist = okm.lloyd(X, C0, 10, trace=True)
    prev = okm.inertia(X, okm.assign(X, C0), C0)
    for Ck in hist:
        cur = okm.inertia(X, okm.assign(X, Ck), Ck)
        assert cur <= prev * (1 + 1e-12)
        prev = cur


def test_lloyd_fixed_point_once_labels_repeat():
    """Textbook Lloyd property the GPU loop relies on to let a head leave
    early: once an assignment equals the previous one, the update returns
    the same centres bit for bit (same members, same summation order, empty
    clusters keep theirs), so every later iteration is the same fixed point
    and stopping there gives exactly the full run's centres and labels."""
    r = _rng(11)
    for trial in range(6):
        n, d, m = int(r.integers(40, 400)), int(r.integers(2, 9)), int(r.integers(3, 25))
        X = r.standard_normal((n, d)) + r.integers(0, 6, (n, 1)) * 1.5
        C0, _ = okm.kmeanspp_init(X, min(m, n), trial, 3, 0)
        C_full, lab_full = okm.lloyd(X, C0, 10)
        C, prev, stopped = C0.copy(), None, None
        for it in range(10):
            lab = okm.assign(X, C)
            C_new = okm.update(X, lab, C)
            if prev is not None and np.array_equal(lab, prev):
                assert np.array_equal(C_new, C)  # the fixed point, exactly
                stopped = it
                break
            prev, C = lab, C_new
        lab_final = okm.assign(X, C)
        assert np.array_equal(C, C_full) and np.array_equal(lab_final, lab_full), (trial, stopped)


def test_update_empty_cluster_keeps_centre():
    X = np.array([[0.0], [1.0], [2.0]])
    C_prev = np.array([[0.5], [100.0]])
    C = okm.update(X, np.array([0, 0, 0]), C_prev)
    assert C[0, 0] == 1.0 and C[1, 0] == 100.0


def test_kmeanspp_second_pick_follows_d2():
    """k-means++ (Arthur and Vassilvitskii 2007): after the first centre, the
    next is drawn with probability proportional to D^2.  Empirical check
    over many streams on four points on a line."""
    X = np.array([[0.0], [1.0], [3.0], [7.0]])
    counts = np.zeros((4, 4))
    for s in range(12000):
        _, picks = okm.kmeanspp_init(X, 2, 11, s, 0)
        counts[picks[0], picks[1]] += 1
    for j0 in range(4):
        d2 = (X[:, 0] - X[j0, 0]) ** 2
        expect = d2 / d2.sum()
        got = counts[j0] / counts[j0].sum()
        assert counts[j0].sum() > 2500              # first pick uniform
        assert np.all(np.abs(got - expect) < 0.035)
        assert counts[j0, j0] == 0                  # never re-picks a centre


def test_kmeanspp_distinct_points_when_m_equals_n():
    r = _rng(8)
    X = r.standard_normal((40, 4))
    C, picks = okm.kmeanspp_init(X, 40, 3, 9, 0)
    assert len(set(picks.tolist())) == 40


def test_subsample_index_strided():
    idx = okm.subsample_index(100, 2, 8)
    assert idx.size == 16 and idx[0] == 0 and np.all(np.diff(idx) > 0) and idx[-1] < 100
    assert np.array_equal(okm.subsample_index(10, 5, 0), np.arange(10))


# ---------------------------------------------------------------- Algorithm 1

def _blobs(centres, per, spread, seed):
    r = _rng(seed)
    pts = [c + spread * r.standard_normal((per, len(c))) for c in centres]
    return np.concatenate(pts, 0)


def _keys_bits(X):
    return nm.bf16_round(X)


def test_alg1_single_stage_with_infinite_tau():
    p = nm.Params(m0=8, nmax=100, tau_rule=nm.TAU_INF, iters=3, init_sample=0)
    X = _rng(9).standard_normal((200, 16))
    out = oms.cluster_keys(_keys_bits(X), p, 0)
    assert out["stages"] == 1 and out["nk"] == 8 and not out["fallback"]


def test_alg1_identical_points_fall_back():
    """All keys equal: every distance is 0, tau = 1.5*mean = 0 and no key is
    strictly closer than tau, so stages continue until the cap: F = True."""
    p = nm.Params(m0=4, nmax=10, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, iters=2, init_sample=0)
    X = np.ones((50, 8))
    out = oms.cluster_keys(_keys_bits(X), p, 0)
    assert out["fallback"] and out["nk"] >= p.nmax and out["nk"] <= p.ncap_k()
    p2 = nm.Params(m0=4, nmax=10, tau_rule=nm.TAU_ABS, tau_param=1.0, iters=2, init_sample=0)
    out2 = oms.cluster_keys(_keys_bits(X), p2, 0)
    assert not out2["fallback"] and out2["stages"] == 1


def test_alg1_every_point_its_own_centre():
    p = nm.Params(m0=64, nmax=100, tau_rule=nm.TAU_ABS, tau_param=1e-3, iters=2, init_sample=0)
    X = _rng(10).standard_normal((30, 8)) * 5
    out = oms.cluster_keys(_keys_bits(X), p, 0)
    assert out["stages"] == 1 and out["nk"] == 30 and not out["fallback"]
    assert len(set(out["labels"].tolist())) == 30


def test_alg1_cap_forces_fallback_hand_case():
    """Eight far-apart keys, one cluster per stage (m0 = 1), tau = 0.5 and
    N_max = 3: each stage's single centre is the mean of all remaining
    keys, no key is within tau, so the loop stops at the cap after three
    stages with every key left: F = True, |C| = 3."""
    X = np.eye(8) * 10.0
    p = nm.Params(m0=1, nmax=3, tau_rule=nm.TAU_ABS, tau_param=0.5, iters=1, init_sample=0)
    out = oms.cluster_keys(_keys_bits(X), p, 0)
    assert out["fallback"] and out["nk"] == 3 and out["stages"] == 3


def test_alg1_two_blobs_hand_case():
    X = _blobs([np.zeros(4), np.full(4, 50.0)], 5, 0.01, 11)
    p = nm.Params(m0=2, nmax=10, tau_rule=nm.TAU_ABS, tau_param=0.5, iters=3, init_sample=0)
    out = oms.cluster_keys(_keys_bits(X), p, 0)
    assert out["stages"] == 1 and out["nk"] == 2 and not out["fallback"]
    lab = out["labels"]
    assert len(set(lab[:5])) == 1 and len(set(lab[5:])) == 1 and lab[0] != lab[5]


def test_alg1_invariants_multistage():
    """Algorithm 1 invariants: with F = 0 every key lies within tau of the
    centre it was removed with; the final labels are nearest-centre over all
    of C; |C| <= N_max - 1 + m0; F = 1 iff keys remained at the cap."""
    X = _blobs([np.full(16, float(i) * 3) for i in range(12)], 40, 0.3, 12)
    X = np.concatenate([X, _rng(13).uniform(-20, 20, (30, 16))], 0)
    for nmax in (200, 6):
        p = nm.Params(m0=6, nmax=nmax, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, iters=5, init_sample=0)
        out = oms.cluster_keys(_keys_bits(X), p, 0, trace=True)
        K = nm.bf16_to_f64(_keys_bits(X))
        assert out["nk"] <= p.ncap_k()
        assert np.array_equal(out["labels"], okm.assign(K, out["cent"]))
        left = out["trace"][-1]["U"][~out["trace"][-1]["removed"]]
        assert out["fallback"] == (left.size > 0)
        if not out["fallback"]:
            for st in out["trace"]:
                assert np.all(st["dist"][st["removed"]] < out["tau"])
            # every key is within tau of its removal centre, hence of its nearest centre
            d = np.sqrt(np.min(okm.sq_dist(K, out["cent"]), axis=1))
            assert np.all(d < out["tau"])
    # compact blobs only: eight far-apart blobs, six clusters per stage, so
    # stage 0 must merge blobs and the merged ones lie beyond 1.5x the mean
    # distance.  With a loose cap a later stage splits them and no fallback
    # happens; with N_max = 6 the cap is hit right after stage 0.
    Xb = _blobs(list(_rng(30).standard_normal((8, 16)) * 10), 30, 0.05, 31)
    p_loose = nm.Params(m0=6, nmax=200, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, iters=5, init_sample=0)
    p_tight = nm.Params(m0=6, nmax=6, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, iters=5, init_sample=0)
    lo = oms.cluster_keys(_keys_bits(Xb), p_loose, 0)
    assert not lo["fallback"] and lo["stages"] >= 2
    ti = oms.cluster_keys(_keys_bits(Xb), p_tight, 0)
    assert ti["fallback"] and ti["nk"] == 6 and ti["stages"] == 1


def test_stage_tau_rules():
    d = np.array([4.0, 1.0, 3.0, 2.0, 5.0])
    assert oms.stage_tau(d, nm.TAU_MEAN_X, 1.5) == 1.5 * 3.0
    assert oms.stage_tau(d, nm.TAU_PCTL, 0.95) == 5.0    # ceil(4.75) = 5th smallest
    assert oms.stage_tau(d, nm.TAU_PCTL, 0.4) == 2.0     # ceil(2.0) = 2nd smallest
    assert oms.stage_tau(d, nm.TAU_ABS, 0.7) == 0.7
    assert math.isinf(oms.stage_tau(d, nm.TAU_INF, 0))


def test_centroid_bound_and_tau_bound():
    """AdaCluster §3.2.1: q.c(k) - q.k <= ||q|| ||k - c(k)|| for every q, k;
    and with F = 0 every |q.c(k) - q.k| < ||q|| tau."""
    X = _blobs([np.full(8, float(i) * 4) for i in range(6)], 50, 0.4, 14)
    p = nm.Params(m0=4, nmax=100, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, iters=5, init_sample=0)
    out = oms.cluster_keys(_keys_bits(X), p, 0)
    K = nm.bf16_to_f64(_keys_bits(X))
    c = out["cent"][out["labels"]]
    Q = _rng(15).standard_normal((40, 8))
    lhs = Q @ c.T - Q @ K.T
    rhs = np.linalg.norm(Q, axis=1)[:, None] * np.linalg.norm(K - c, axis=1)[None, :]
    assert np.all(lhs <= rhs + 1e-9)
    assert not out["fallback"]
    assert np.all(np.abs(lhs) < np.linalg.norm(Q, axis=1)[:, None] * out["tau"])


# ---------------------------------------------------------------- statistics and permutation

def test_counting_sort_properties():
    lab = _rng(16).integers(0, 9, 500)
    lab[lab == 4] = 3          # cluster 4 empty
    perm, seg = ost.counting_sort(lab, 9)
    assert sorted(perm.tolist()) == list(range(500))
    assert seg[0] == 0 and seg[-1] == 500 and seg[4] == seg[5]
    for c in range(9):
        members = perm[seg[c]:seg[c + 1]]
        assert np.all(lab[members] == c)
        assert np.all(np.diff(members) > 0)          # stable: original order kept
    assert np.array_equal(np.diff(seg), np.bincount(lab, minlength=9))


def test_key_stats_properties_and_mse_closed_form():
    """max/min are attained member values bounding every member; means times
    counts give the sums; per-head MSE (AdaCluster §3.2.1) equals
    d*sigma^2*(1-1/n) in expectation for isotropic components whose centres
    are recovered."""
    d, sigma, per = 32, 0.5, 400
    cen = np.eye(d)[:8] * 1000.0
    X = _blobs(list(cen), per, sigma, 17)
    Kb = _keys_bits(X)
    Vb = _keys_bits(_rng(18).standard_normal(X.shape))
    p = nm.Params(m0=8, nmax=100, tau_rule=nm.TAU_INF, iters=5, init_sample=0)
    out = oms.cluster_keys(Kb, p, 0)
    st = ost.key_stats(Kb, Vb, out["labels"], out["cent"])
    K, V = nm.bf16_to_f64(Kb), nm.bf16_to_f64(Vb)
    assert np.all(st["count"] == per)
    for c in range(8):
        mem = out["labels"] == c
        assert np.array_equal(st["kmax"][c], K[mem].max(0))
        assert np.array_equal(st["kmin"][c], K[mem].min(0))
        assert np.allclose(st["kmean"][c] * per, K[mem].sum(0))
        assert np.allclose(st["vmean"][c] * per, V[mem].sum(0))
    expect = d * sigma ** 2 * (1 - 1 / per)
    assert abs(st["mse"] - expect) / expect < 0.05


# ---------------------------------------------------------------- scoring

def test_quest_is_upper_bound():
    """AdaCluster eq. (1) / Quest: the bound is >= q.k for every key of the cluster."""
    r = _rng(19)
    for _ in range(20):
        Kc = r.standard_normal((30, 16)) * r.uniform(0.1, 3)
        q = r.standard_normal(16)
        S = osc.quest_scores(q[None], Kc.max(0)[None], Kc.min(0)[None], np.array([30]))
        assert S[0, 0] >= np.max(Kc @ q) - 1e-12


def test_quest_split_form_equals_max_form():
    """The two-product form q+.max + q-.min equals the per-dimension max form
    (reading of AdaCluster eq. (2)).  A literal elementwise k+/k- reading does
    not: it is not even an upper bound on this example."""
    r = _rng(20)
    cq = r.standard_normal((7, 32))
    Kc = [r.standard_normal((r.integers(1, 20), 32)) for _ in range(11)]
    kmax = np.stack([k.max(0) for k in Kc])
    kmin = np.stack([k.min(0) for k in Kc])
    a = osc.quest_scores(cq, kmax, kmin, np.ones(11))
    b = osc.quest_scores_split(cq, kmax, kmin)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    literal = np.maximum(cq, 0) @ np.maximum(kmax, 0).T + np.minimum(cq, 0) @ np.minimum(kmin, 0).T
    assert not np.allclose(literal, a)


def test_quest_singletons_exact():
    """A cluster of one key: max = min = k, so Quest(q, {k}) = q.k exactly."""
    r = _rng(21)
    K = r.standard_normal((25, 16))
    q = r.standard_normal((3, 16))
    S = osc.quest_scores(q, K, K, np.ones(25))
    assert np.allclose(S, q @ K.T, atol=1e-13)


def test_selection_topk_matches_full_sort():
    r = _rng(22)
    S = np.round(r.standard_normal((5, 40)), 1)    # many exact ties
    cnt = r.integers(0, 50, 40)
    cnt[3] = 0
    p = nm.Params(sel_mode=nm.SEL_TOPK, topk=7)
    for row in range(5):
        got = osc.select_row(S[row], cnt, 1.0, 1000, 64, p)
        ref = sorted([c for c in range(40) if cnt[c] > 0], key=lambda c: (-S[row, c], c))[:7]
        assert got.tolist() == ref


def test_selection_density_and_topp_prefix_property():
    r = _rng(23)
    S = r.standard_normal((6, 50))
    cnt = r.integers(0, 300, 50)
    L = int(cnt.sum())
    for row in range(6):
        p = nm.Params(sel_mode=nm.SEL_DENSITY, sel_param=0.2)
        sel = osc.select_row(S[row], cnt, 1.0, L, 64, p)
        budget = math.ceil(0.2 * L)
        assert cnt[sel].sum() >= budget and cnt[sel[:-1]].sum() < budget
        order = osc.order_clusters(S[row], cnt)
        assert np.array_equal(sel, order[:sel.size])
        p2 = nm.Params(sel_mode=nm.SEL_TOPP, sel_param=0.9)
        sel2 = osc.select_row(S[row], cnt, 2.0, L, 64, p2)
        nzc = order
        z = 2.0 * S[row, nzc] / 8.0 + np.log(cnt[nzc])
        pi = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
        k = sel2.size
        assert pi[:k].sum() >= 0.9 - 1e-12 and pi[:k - 1].sum() < 0.9
        assert np.array_equal(sel2, order[:k])


def test_selection_scale_invariance_of_centre():
    """Quest is positively homogeneous in q, so scaling a query-cluster
    centre does not change TOPK / DENSITY selections (AdaCluster Appendix
    A.2 applied to the centre)."""
    r = _rng(24)
    kmax = r.standard_normal((30, 16)) + 1
    kmin = kmax - r.uniform(0, 2, (30, 16))
    cnt = r.integers(1, 100, 30)
    cq = r.standard_normal((4, 16))
    for mode in (nm.SEL_TOPK, nm.SEL_DENSITY):
        p = nm.Params(sel_mode=mode, topk=5, sel_param=0.3)
        a = osc.select(osc.quest_scores(cq, kmax, kmin, cnt), cnt, np.ones(4), int(cnt.sum()), 16, p)
        b = osc.select(osc.quest_scores(3.7 * cq, kmax, kmin, cnt), cnt, np.ones(4), int(cnt.sum()), 16, p)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ---------------------------------------------------------------- attention

def test_dense_matches_torch_sdpa_fp64():
    import torch
    r = _rng(25)
    Q, K, V = r.standard_normal((3, 64, 32))
    O, lse = oat.dense_rows(Q, K, V, np.arange(64), 1 / math.sqrt(32))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None])[0].numpy()
    assert np.allclose(O, ref, rtol=0, atol=1e-12)
    ref_lse = np.log(np.exp((Q @ K.T) / math.sqrt(32)).sum(1))
    assert np.allclose(lse, ref_lse, atol=1e-12)


def _toy_layer(seed, L=300, d=16, nk=12, nq=4):
    r = _rng(seed)
    Q, K, V = r.standard_normal((3, L, d))
    kl = r.integers(0, nk, L)
    ql = r.integers(0, nq, L)
    return Q, K, V, kl, ql


# every row (each query cluster gathers its selected keys) and a sparse
# sample (few rows a cluster: logits of every key, unselected ones at weight 0)
ROW_SETS = [np.arange(300), np.arange(3, 300, 37)]


@pytest.mark.parametrize("rows", ROW_SETS, ids=["all-rows", "sampled-rows"])
def test_all_selected_equals_dense(rows):
    Q, K, V, kl, ql = _toy_layer(26)
    sel = [np.arange(12)] * 4
    O, lse = oat.sparse_rows(Q, K, V, rows, ql, kl, sel, 0.25)
    Od, lsed = oat.dense_rows(Q, K, V, rows, 0.25)
    assert np.allclose(O, Od, atol=1e-12) and np.allclose(lse, lsed, atol=1e-12)


def test_error_identity_eq4():
    """ClusterAttention §1.2 eq. (4): o - o_S = (1 - w_S)(o_Sbar - o_S)."""
    r = _rng(27)
    Q, K, V = r.standard_normal((3, 200, 16))
    for row in range(5):
        S = np.nonzero(r.random(200) < 0.3)[0]
        Sb = np.setdiff1d(np.arange(200), S)
        oS, wS, w = oat.subset_output(Q, K, V, row, S, 0.25)
        oSb = (w[Sb] @ V[Sb]) / w[Sb].sum()
        o = w @ V
        assert np.allclose(o - oS, (1 - wS) * (oSb - oS), atol=1e-13)
        # the oracle's sparse path gives the same o_S
        kl = np.where(np.isin(np.arange(200), S), 0, 1)
        Os, _ = oat.sparse_rows(Q, K, V, np.array([row]), np.zeros(200, int), kl, [np.array([0])], 0.25)
        assert np.allclose(Os[0], oS, atol=1e-13)


@pytest.mark.parametrize("rows", ROW_SETS, ids=["all-rows", "sampled-rows"])
def test_compensation_identity_eq5(rows):
    """ClusterAttention §1.2 eq. (5), with ||c|| read as the cluster size:
    o - o_hat_S = (1/d_hat_S) sum_c n_c (delta_c (vbar_c - o) + Cov_c(w, v)),
    with delta_c >= 0 (Jensen) and d_hat_S <= 1."""
    Q, K, V, kl, ql = _toy_layer(28)
    scale = 0.25
    cnt = np.bincount(kl, minlength=12)
    kmean = np.stack([K[kl == c].mean(0) for c in range(12)])
    vmean = np.stack([V[kl == c].mean(0) for c in range(12)])
    sel = [np.array([0, 3, 5]), np.array([1]), np.array([2, 4, 6, 7]), np.array([11])]
    Oc, _ = oat.sparse_rows(Q, K, V, rows, ql, kl, sel, scale, True, cnt, kmean, vmean)
    for i, row in enumerate(rows):
        if i % 9:
            continue
        z = (Q[row] @ K.T) * scale
        Z = np.exp(z).sum()
        w = np.exp(z) / Z
        o = w @ V
        ex = np.setdiff1d(np.arange(12), sel[ql[row]])
        dhat = w[np.isin(kl, sel[ql[row]])].sum()
        rhs = np.zeros(16)
        for c in ex:
            m = kl == c
            wbar = w[m].mean()
            what = np.exp((Q[row] @ kmean[c]) * scale) / Z
            delta = wbar - what
            assert delta >= -1e-15
            cov = ((w[m] - wbar)[:, None] * (V[m] - vmean[c])).mean(0)
            rhs += cnt[c] * (delta * (vmean[c] - o) + cov)
            dhat += cnt[c] * what
        assert dhat <= 1 + 1e-12
        assert np.allclose(o - Oc[i], rhs / dhat, atol=1e-12)


@pytest.mark.parametrize("rows", [np.arange(60), np.arange(1, 60, 7)], ids=["all-rows", "sampled-rows"])
def test_singletons_compensation_is_dense(rows):
    """All clusters of size one: each pseudo-key is the key itself with weight
    ln 1 = 0, so sparse attention with compensation equals dense attention
    for any selection."""
    r = _rng(29)
    Q, K, V = r.standard_normal((3, 60, 8))
    kl = np.arange(60)
    ql = r.integers(0, 3, 60)
    sel = [np.array([1, 5]), np.array([7]), np.arange(30)]
    cnt = np.ones(60, int)
    O, _ = oat.sparse_rows(Q, K, V, rows, ql, kl, sel, 0.3, True, cnt, K, V)
    Od, _ = oat.dense_rows(Q, K, V, rows, 0.3)
    assert np.allclose(O, Od, atol=1e-12)


# ---------------------------------------------------------------- whole layer and pages' numbers

def test_tiny_layer_runs_and_is_consistent():
    w = gen.get_workload("tiny", L=1024)
    Q, K, V = gen.generate(w)
    p = nm.Params(nq=16, m0=32, nmax=64, tau_rule=nm.TAU_INF, sel_mode=nm.SEL_TOPK, topk=8,
                  init_sample=0, iters=10)
    out = oly.run_layer(Q, K, V, p)
    for h in out:
        assert h["O"].shape == (1024, 64) and np.all(np.isfinite(h["O"]))
        assert all(s.size == min(8, int((h["kstats"]["count"] > 0).sum())) for s in h["sel"])
        assert not h["dense"]
    # selecting every cluster reproduces dense attention
    p_all = nm.Params(nq=16, m0=32, nmax=64, tau_rule=nm.TAU_INF, sel_mode=nm.SEL_TOPK, topk=10 ** 6,
                      init_sample=0)
    h = oly.run_head(Q[0, 0], K[0, 0], V[0, 0], p_all, 0)
    Od, _ = oat.dense_rows(*(nm.bf16_to_f64(x[0, 0]) for x in (Q, K, V)), np.arange(1024), 1 / 8)
    assert np.allclose(h["O"], Od, atol=1e-12)


def test_page_token_grids():
    """AdaCluster §4.3 Table 2: tokens = 21 latent frames x (W/16) x (H/16)
    for the resolutions whose sides divide by 16; the workloads' grids give
    the token counts they name."""
    g = json.load(open(os.path.join(GOLDEN, "page_numbers.json")))
    t2 = g["table2_tokens"]
    f, p = g["latent_frames_81"]["frames"], g["latent_frames_81"]["patch"]
    for res in ("864x480", "1280x720", "1712x720"):
        wdt, hgt = map(int, res.split("x"))
        assert round(f * (wdt // p) * (hgt // p) / 1000, 1) == t2[res]
    # §2.1 names 1920x1120 for the 176.4K case
    assert round(f * (1920 // p) * (1120 // p) / 1000, 1) == t2["1912x1120"]
    assert gen.get_workload("wan").L == 21 * 60 * 60 == round(t2["1280x720"] * 1000)
    assert gen.get_workload("cogvideox").L == 13 * 75 * 72
    assert gen.get_workload("hunyuan").L == 33 * 45 * 80
    lat = g["figure1_latency_s"]
    assert round(lat["full"] / lat["adacluster"], 2) == g["table1_speedup_hunyuan"]["value"]
