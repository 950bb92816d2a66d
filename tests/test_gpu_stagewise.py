"""Stage-by-stage parity of the clustering at full sequence length.

ac_cluster_k_trace records every stage of Algorithm 1 (AdaCluster §3.2.2):
the unassigned set U_t, m_t, the centres after k-means++ seeding and after
each Lloyd update, the stage's final labels and the distances that set tau
and the removal.  ac_cluster_q_trace records the query centres the same way.
The oracle recomputes each step from the GPU's previous step (protocol
S1-S3): seeding picks bit-exact, each Lloyd update to fp32 rounding (clusters
touched by a near-tie label excluded), labels nearest-centre except near
ties, distances and tau to fp32 rounding, the removal set and the next U_t
exact except tau near ties, and the stage count, cluster count and fallback
flag from the recorded stages.  Heads are a few of each workload's own heads
at its real L (one GPU's share of heads does not change the per-head work)."""
import numpy as np
import pytest

import csa_inputs as gen
from oracle import numerics as nm
from oracle import kmeans as okm
from oracle import multistage as oms
from abi_helpers import Run, np_, near_tie_flips, workload_oracle_params

pytestmark = pytest.mark.gpu

REL_CENT = 1e-6    # a Lloyd update: fp64 sums rounded once to fp32
REL_DIST = 1e-6    # distances: fp64 accumulation stored in fp32
TAU_TIE = 1e-5     # removal decisions within this relative distance of tau are near ties


def _tie_clusters(X, C, rel=1e-5):
    """Clusters whose membership may differ at a near tie: the nearest and
    second-nearest centre of every point whose two squared distances are
    within rel of each other (relative to ||x||^2 + ||c||^2)."""
    if C.shape[0] < 2:
        return np.zeros(C.shape[0], dtype=bool)
    d2 = okm.sq_dist(X, C)
    two = np.argpartition(d2, 1, axis=1)[:, :2]
    a = np.take_along_axis(d2, two, axis=1)
    swap = a[:, 0] > a[:, 1]
    two[swap] = two[swap][:, ::-1]
    a[swap] = a[swap][:, ::-1]
    scale = np.sum(X * X, axis=1) + np.sum(C[two[:, 0]] ** 2, axis=1)
    tie = (a[:, 1] - a[:, 0]) < rel * scale
    out = np.zeros(C.shape[0], dtype=bool)
    out[two[tie, 0]] = True
    out[two[tie, 1]] = True
    return out


def _check_lloyd(X, cent_slots, m, iters, what):
    """Every recorded Lloyd update from the previous recorded centres."""
    skipped = 0
    for j in range(iters):
        Cj = cent_slots[j, :m].astype(np.float64)
        lab = okm.assign(X, Cj)
        ref = okm.update(X, lab, Cj)
        got = cent_slots[j + 1, :m].astype(np.float64)
        ok = ~_tie_clusters(X, Cj)
        skipped += int((~ok).sum())
        scale = max(1.0, float(np.max(np.abs(ref))))
        err = np.max(np.abs(got[ok] - ref[ok])) if ok.any() else 0.0
        assert err <= REL_CENT * scale, (what, "Lloyd update", j, err)
    return skipped


def _run_traced(Qb, Kb, Vb, p, max_stages):
    import torch
    import clustered_sparse_attention_amd as ac
    r = Run(Qb, Kb, Vb, p)
    dev = torch.device("cuda")
    tr = ac.KTrace(r.BH, r.L, max_stages, p.iters, p.m0, r.d, dev)
    ac.ac_cluster_k_trace(r.shape, r.cp, r.K, r.V, r.k, r.st, tr, r.ws)
    qtr = torch.zeros((r.BH, p.iters + 1, r.nq, r.d), dtype=torch.float32, device=dev)
    ac.ac_cluster_q_trace(r.shape, r.cp, r.Q, r.q, qtr, r.ws)
    torch.cuda.synchronize()
    return r, tr, qtr


def check_key_trace(r, tr, Kb, p, max_stages):
    """S1-S3 for every recorded stage of every head; returns a summary."""
    B, H, L, d = Kb.shape
    Kf = Kb.reshape(B * H, L, d)
    tn, tm, tu, tc, tl, td = (np_(x) for x in (tr.n, tr.m, tr.u, tr.cent, tr.labels, tr.dist))
    ncl, fb, stages, tau = np_(r.k.ncl), np_(r.st.fallback), np_(r.st.stages), np_(r.st.tau)
    out = dict(stages=[], tie_clusters=0, label_ties=0, tau_ties=0, fallback=fb.tolist())
    for h in range(B * H):
        K = nm.bf16_to_f64(Kf[h])
        U = np.arange(L)
        nC = 0
        ns = int(stages[h])
        assert 1 <= ns
        sizes = []
        exact = True  # U_t follows from the GPU's previous stage without a tau near tie
        for t in range(min(ns, max_stages)):
            n, m = int(tn[h, t]), int(tm[h, t])
            sizes.append(n)
            assert m == oms.next_m(n, p.m0), (h, t, "m_t")
            u = tu[h, t, :n]
            if exact:
                assert n == U.size and np.array_equal(u, U), (h, t, "U_t")
            X = K[u]
            # S1: seeding picks, bit-exact
            C0, _ = okm.kmeanspp_init(X, m, p.seed, nm.stream_id(h, 1, t), p.init_sample)
            assert np.array_equal(tc[h, t, 0, :m].astype(np.float64), C0), (h, t, "k-means++ picks")
            # S2: every Lloyd update
            out["tie_clusters"] += _check_lloyd(X, tc[h, t], m, p.iters, (h, t))
            # the stage's final labels
            Cf = tc[h, t, p.iters, :m].astype(np.float64)
            lab = tl[h, t, :n]
            bad, flips, _ = near_tie_flips(X, Cf, lab)
            assert bad == 0 and flips <= 0.001 * n, (h, t, "stage labels", bad, flips)
            out["label_ties"] += flips
            # S3: distances, tau (stage 0) and the removal set
            dref = np.linalg.norm(X - Cf[lab], axis=1)
            dg = td[h, t, :n].astype(np.float64)
            assert np.all(np.abs(dg - dref) <= REL_DIST * dref + 1e-7), (h, t, "distances")
            if t == 0:
                tref = oms.stage_tau(dg, p.tau_rule, p.tau_param)
                assert (np.isinf(tref) and np.isinf(tau[h])) or abs(float(tau[h]) - tref) <= REL_DIST * tref, \
                    (h, "tau", float(tau[h]), tref)
            removed = dg < float(tau[h])   # the GPU's decision (fp32 distances against fp32 tau)
            ref_removed = dref < float(tau[h])
            near = np.abs(dref - float(tau[h])) < TAU_TIE * float(tau[h])
            assert np.all((removed == ref_removed) | near), (h, t, "removal")
            if np.any(near & (removed != ref_removed)):
                out["tau_ties"] += 1
                exact = False  # the next U_t is the GPU's; checked as recorded from here on
            U = u[~removed]
            nC += m
        if ns <= max_stages and exact:
            # Algorithm 1's end: U empty, or the cap reached with keys left (fallback);
            # the cap is tested before each stage, so the last one started below it
            assert int(ncl[h]) == nC, (h, "cluster count")
            assert bool(fb[h]) == (U.size > 0), (h, "fallback flag")
            assert nC - m < p.nmax, (h, "a stage started at the cap")
            if fb[h]:
                assert nC >= p.nmax
        out["stages"].append(sizes)
    return out


def check_query_trace(r, qtr, Qb, p):
    B, H, L, d = Qb.shape
    Qf = Qb.reshape(B * H, L, d)
    cs = np_(qtr)
    skipped = 0
    for h in range(B * H):
        X = nm.bf16_to_f64(okm.normalize_queries(Qf[h]))
        C0, _ = okm.kmeanspp_init(X, r.nq, p.seed, nm.stream_id(h, 0, 0), p.init_sample)
        assert np.array_equal(cs[h, 0].astype(np.float64), C0), (h, "query k-means++ picks")
        skipped += _check_lloyd(X, cs[h], r.nq, p.iters, (h, "queries"))
        bad, flips, _ = near_tie_flips(X, cs[h, p.iters].astype(np.float64), np_(r.q.labels)[h])
        assert bad == 0 and flips <= 0.001 * L, (h, "query labels")
        assert np.array_equal(np_(r.q.cent)[h], cs[h, p.iters])
    return skipped


@pytest.mark.parametrize("name,H,overrides,max_stages", [
    ("wan", 2, {}, 12),                   # tau = 1.5 x mean; U_1 above the sort's one-group size
    ("cogvideox", 2, {}, 12),             # d = 64, percentile tau by radix select over 70,200 distances
    # the widest Student-t heads of the long workload: Algorithm 1 falls back
    ("long", 2, dict(key_sigma=(0.3, 0.3), key_outlier_scale=(0.70, 0.75)), 12),
    # absolute tau 5.5: a compact head finishes after 9 stages, a dispersed head with uniform
    # outliers keeps every key and falls back when the 15th stage reaches N_max
    ("hunyuan", 2, dict(key_sigma=(0.15, 0.8), outlier_heads=(1,)), 16),
])
def test_full_length_stagewise_clustering(name, H, overrides, max_stages):
    w = gen.get_workload(name, H=H, **overrides)
    Q, K, V = gen.generate(w)
    p = workload_oracle_params(name)
    r, tr, qtr = _run_traced(Q, K, V, p, max_stages)
    s = check_key_trace(r, tr, K, p, max_stages)
    print(f"\n[{name}] stage sizes {s['stages']}, fallback {s['fallback']}, tie clusters {s['tie_clusters']}, "
          f"label ties {s['label_ties']}, tau ties {s['tau_ties']}")
    assert len(s["stages"][0]) >= 2, "the workload should run several stages"
    if name == "long":
        assert any(s["fallback"]), "the widest heads should fall back"
    if name == "hunyuan":
        assert s["fallback"] == [0, 1], "the dispersed head, and only it, falls back"
        assert len(s["stages"][1]) == 15, "the dispersed head runs every stage up to N_max"
    skipped = check_query_trace(r, qtr, Q, p)
    print(f"[{name}] query tie clusters {skipped}")


def test_traced_clustering_equals_untraced():
    """The record is a copy: the traced entry points give bit-identical
    clusters and statistics to ac_cluster_k / ac_cluster_q."""
    import torch
    w = gen.get_workload("tiny", H=2, L=4096)
    Q, K, V = gen.generate(w)
    p = workload_oracle_params("tiny")
    p.tau_rule, p.tau_param, p.m0, p.nmax, p.init_sample = nm.TAU_MEAN_X, 1.5, 16, 64, 8
    r, tr, qtr = _run_traced(Q, K, V, p, 3)
    ref = Run(Q, K, V, p)
    ref.cluster_q()
    ref.cluster_k()
    torch.cuda.synchronize()
    for name in ("labels", "perm", "seg", "cent", "ncl"):
        assert torch.equal(getattr(ref.k, name), getattr(r.k, name)), f"k.{name}"
        assert torch.equal(getattr(ref.q, name), getattr(r.q, name)), f"q.{name}"
    for name in ("kmax", "kmin", "kmean", "vmean", "fallback", "tau", "stages", "mse"):
        assert torch.equal(getattr(ref.st, name), getattr(r.st, name)), f"stats.{name}"
    check_key_trace(r, tr, K, p, 3)
