"""GPU parity at the full sizes of the four large workloads, in the launch
configuration bench.py times: every stage of every head checked against the
oracle recomputing it from the GPU's previous stage; attention on a seeded
sample of 2048 query rows per head (for top-p selections, which keep most
keys, 128 rows from each of 16 seeded query clusters per head)."""
import numpy as np
import pytest

import csa_inputs as gen
from oracle import numerics as nm
from abi_helpers import (Run, workload_oracle_params, check_clusters_sampled, check_scores_selection,
                         check_attention_sampled, np_, bf16_dev_to_f64)

pytestmark = pytest.mark.gpu

ROW_SEED = {"cogvideox": 9002, "hunyuan": 9003, "wan": 9004, "long": 9005}
# top-p 0.9 keeps most keys of every query cluster here: its attention is
# checked on 128 rows from each of 16 seeded query clusters per head (2048
# rows, each sampled cluster's keys gathered once)
LARGE_SELECTION_SAMPLE = {"topp": dict(nrows=2048, clusters=16)}


@pytest.fixture(scope="module")
def wan_run():
    w = gen.get_workload("wan")
    Q, K, V = gen.generate(w)
    p = workload_oracle_params("wan")
    r = Run(Q, K, V, p)
    r.cluster_q()
    r.cluster_k()
    import torch
    torch.cuda.synchronize()
    return w, Q, K, V, r


def test_wan_clusters(wan_run):
    w, Q, K, V, r = wan_run
    out = check_clusters_sampled(r, Q, K, V, ROW_SEED["wan"])
    print("wan clusters:", out["fallback"], "fallback heads; key clusters", min(out["ncl"]), "-", max(out["ncl"]),
          "; near-tie label flips", out["label_flips"])


@pytest.mark.parametrize("variant,compensate", [("density", 0), ("density", 1), ("topp", 0), ("topp", 1)])
def test_wan_selection_and_attention(wan_run, variant, compensate):
    """The four measured variants of the Wan2.1-shaped layer: top-K at 15%
    density and top-p 0.9, each with and without stripe-mean compensation."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import abi_params
    w, Q, K, V, r = wan_run
    p = workload_oracle_params("wan", variant, compensate)
    r.p, r.cp = p, abi_params(p)
    r.score_select()
    r.attn()
    torch.cuda.synchronize()
    ties = check_scores_selection(r, p)
    worst = check_attention_sampled(r, Q, K, V, p, ROW_SEED["wan"], **LARGE_SELECTION_SAMPLE.get(variant, {}))
    print(f"wan {variant} comp={compensate}: selection near-tie rows {ties}; worst max-abs {worst[0]:.3g} "
          f"rel-L2 {worst[1]:.3g}")


def test_wan_layer_equals_entry_points(wan_run):
    """ac_layer, the call bench.py times (the query clustering beside the key
    clustering on a second stream, each stage's merge beside the next stage's
    seeding, statistics without the value rows when compensation is off), on
    the full Wan2.1-shaped layer: the same output, bit for bit, as the entry
    points one after another, whose every stage the tests above check against
    the oracle; and the same per-head cluster counts, flags, thresholds and
    stage counts."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import abi_params
    w, Q, K, V, r = wan_run
    p = workload_oracle_params("wan", "density", 0)
    r.p, r.cp = p, abi_params(p)
    r.score_select()
    r.attn()
    ws = ac.workspace(r.ws_bytes, torch.device("cuda"))
    state = ac.State(r.BH, r.nq, r.ncap_k, r.d, torch.device("cuda"))
    O = torch.empty_like(r.Q)
    hs = ac.ac_layer(r.shape, r.cp, r.Q, r.K, r.V, state, O, ws, host_stats=True)
    torch.cuda.synchronize()
    assert torch.equal(O, r.O)
    assert np.array_equal(hs["ncl_k"], np_(r.k.ncl)) and np.array_equal(hs["stages"], np_(r.st.stages))
    assert np.array_equal(hs["fallback"], np_(r.st.fallback)) and np.array_equal(hs["tau"], np_(r.st.tau))
    assert torch.equal(state.cent_q, r.q.cent)
    ck, ck0, ncl = np_(state.cent_k), np_(r.k.cent), np_(r.k.ncl)
    assert all(np.array_equal(ck[h, :ncl[h]], ck0[h, :ncl[h]]) for h in range(r.BH))  # slots past N_k are unused
    del ws


def test_wan_warm_layer_equals_entry_points(wan_run):
    """ac_layer's warm step (bench.py --warm: a cold call fills the state, then
    Q and K move by 2 %) on the full Wan2.1-shaped layer: bit-identical output
    and carried centres to the warm entry points from the same state."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import abi_params, to_dev
    w, Q, K, V, r = wan_run
    p = workload_oracle_params("wan", "density", 0)
    cp = abi_params(p)
    dev = torch.device("cuda")
    ws = ac.workspace(r.ws_bytes, dev)
    state = ac.State(r.BH, r.nq, r.ncap_k, r.d, dev)
    O = torch.empty_like(r.Q)
    ac.ac_layer(r.shape, cp, r.Q, r.K, r.V, state, O, ws)
    torch.cuda.synchronize()
    assert state.valid == 1
    start = ac.State(r.BH, r.nq, r.ncap_k, r.d, dev)
    for name in ("cent_q", "cent_k", "ncl_k", "fallback", "tau"):
        getattr(start, name).copy_(getattr(state, name))
    start.valid = 1
    Q2, K2 = to_dev(gen.perturb(Q, 1103)), to_dev(gen.perturb(K, 1104))
    Ow = torch.empty_like(r.Q)
    ac.ac_layer(r.shape, cp, Q2, K2, r.V, state, Ow, ws)
    r2 = Run(gen.perturb(Q, 1103), gen.perturb(K, 1104), V, p)
    r2.cluster_q(warm_cent=start.cent_q)
    r2.cluster_k(warm=start)
    r2.score_select()
    r2.attn()
    torch.cuda.synchronize()
    assert torch.equal(Ow, r2.O)
    assert torch.equal(state.cent_q, r2.q.cent)
    ck, ck0, ncl = np_(state.cent_k), np_(r2.k.cent), np_(r2.k.ncl)
    assert np.array_equal(np_(state.ncl_k), ncl)
    assert all(np.array_equal(ck[h, :ncl[h]], ck0[h, :ncl[h]]) for h in range(r.BH))
    del ws, r2


@pytest.mark.parametrize("variant", ["density", "topp"])
def test_wan_tail_merge(wan_run, variant):
    """iCATS tail merging at full size: the merged clusters and selections of
    all 40 heads bit-identical to the oracle's, the query block count never
    larger, and the attention on the merged layout within tolerance."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import abi_params, check_tail_merge
    w, Q, K, V, r = wan_run
    p = workload_oracle_params("wan", variant, 0)
    r.p, r.cp = p, abi_params(p)
    r.score_select()
    torch.cuda.synchronize()
    qm, sm, before, after = check_tail_merge(r, 0)
    assert after <= before
    ac.ac_sparse_attn(r.shape, r.cp, r.Q, r.K, r.V, qm, r.k, r.st, sm, r.O, None, r.ws)
    torch.cuda.synchronize()
    worst = check_attention_sampled(r, Q, K, V, p, ROW_SEED["wan"], q=qm, sel=sm,
                                    **LARGE_SELECTION_SAMPLE.get(variant, {}))
    print(f"wan {variant} tail merge (256-row blocks): query blocks {before} -> {after}; worst max-abs "
          f"{worst[0]:.3g} rel-L2 {worst[1]:.3g}")


def test_wan_token_quest(wan_run):
    """Per-token Quest scores at full size (40 heads x 75,600 tokens against
    every key cluster), both engines, on a seeded sample of 256 query rows
    per head against the oracle's eq. (1)."""
    from abi_helpers import check_token_quest
    w, Q, K, V, r = wan_run
    ld = int(np_(r.k.ncl).max())
    rows = gen.row_sample(w.L, 256, ROW_SEED["wan"])
    worst = check_token_quest(r, Q, K, V, ld, rows=rows)
    print(f"wan token quest ld={ld}: max error / bound {worst}")


def test_wan_interaction_aware_keys(wan_run):
    """iCATS interaction-aware key clustering at full size: M_Q of all 40
    heads against the oracle (raw member means of the GPU's query clusters),
    the metric labels of a sample of keys against the metric argmin for the
    GPU's centres (up to near ties), the statistics of every cluster, and
    the layer's selection and attention on these clusters."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import abi_params
    from oracle import interaction as oia
    from oracle import stats as ost
    from test_gpu_tiny import _metric_label_check
    w, Q, K, V, r = wan_run
    p = workload_oracle_params("wan")
    r.p, r.cp = p, abi_params(p)
    k = ac.Clusters(r.BH, r.L, r.ncap_k, r.d, torch.device("cuda"), rho=False)
    st = ac.KStats(r.BH, r.ncap_k, r.d, torch.device("cuda"))
    M = torch.empty((r.BH, r.d, r.d), dtype=torch.float32, device="cuda")
    ac.ac_interaction_matrix(r.shape, r.cp, r.Q, r.q, M, r.ws)
    ac.ac_cluster_k_metric(r.shape, r.cp, r.K, r.V, M, k, st, r.ws)
    torch.cuda.synchronize()
    Mg = np_(M).astype(np.float64)
    qlab, lab, cent = np_(r.q.labels), np_(k.labels), np_(k.cent)
    kmax, kmin = bf16_dev_to_f64(st.kmax), bf16_dev_to_f64(st.kmin)
    m = min(p.m0, w.L)
    rows = gen.row_sample(w.L, 512, ROW_SEED["wan"])
    Qf, Kf, Vf = (x.reshape(r.BH, w.L, w.d) for x in (Q, K, V))
    flips = 0
    for h in range(r.BH):
        Mo = oia.interaction_matrix(Qf[h], qlab[h], r.nq)
        assert np.max(np.abs(Mg[h] - Mo)) <= 1e-6 * np.max(np.abs(Mo)), h
        C = cent[h, :m].astype(np.float64)
        bad, fl = _metric_label_check(nm.bf16_to_f64(Kf[h][rows]), C, Mg[h], lab[h][rows])
        assert bad == 0, (h, bad)
        flips += fl
        sto = ost.key_stats(Kf[h], Vf[h], lab[h], C)
        assert np.array_equal(kmax[h, :m], sto["kmax"]) and np.array_equal(kmin[h, :m], sto["kmin"]), h
    assert flips <= 0.001 * r.BH * rows.size
    # selection and attention on the metric key clusters
    saved_k, saved_st = r.k, r.st
    r.k, r.st = k, st
    try:
        r.score_select()
        r.attn()
        torch.cuda.synchronize()
        ties = check_scores_selection(r, p)
        worst = check_attention_sampled(r, Q, K, V, p, ROW_SEED["wan"])
    finally:
        r.k, r.st = saved_k, saved_st
    print(f"wan interaction-aware keys (m = {m}): label flips {flips}, selection ties {ties}, worst {worst}")


@pytest.mark.parametrize("name", ["cogvideox", "hunyuan", "long"])
def test_config_full_size(name):
    import torch
    w = gen.get_workload(name)
    Q, K, V = gen.generate(w)
    p = workload_oracle_params(name)
    r = Run(Q, K, V, p).all()
    out = check_clusters_sampled(r, Q, K, V, ROW_SEED[name])
    ties = check_scores_selection(r, p)
    worst = check_attention_sampled(r, Q, K, V, p, ROW_SEED[name])
    print(f"{name}: fallback heads {out['fallback']}, key clusters {min(out['ncl'])}-{max(out['ncl'])}, "
          f"label flips {out['label_flips']}, selection ties {ties}, worst {worst}")
    if name == "long":
        # the widest heavy-tailed heads cannot be covered by N_max centres: several fall back
        assert 2 <= out["fallback"] <= 8
    if name == "hunyuan":
        # absolute threshold 5.5: the compact heads (sigma 0.15) finish below N_max, the
        # dispersed ones (sigma 0.8 and 10% uniform outliers) keep every key and fall back
        assert set(np.flatnonzero(np_(r.st.fallback)).tolist()) == set(range(12, 24))


def test_hunyuan_warm_step():
    """Second denoising step (AdaCluster §3.2.2, efficient initialisation):
    after a 2% perturbation of Q and K the clusters are warm-started from the
    first step's centres with the counts, flags and tau kept."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import to_dev, Run
    from oracle import kmeans as okm
    w = gen.get_workload("hunyuan")
    Q, K, V = gen.generate(w)
    p = workload_oracle_params("hunyuan")
    r = Run(Q, K, V, p).all()
    state = ac.State(r.BH, r.nq, r.ncap_k, r.d, torch.device("cuda"))
    state.cent_q.copy_(r.q.cent)
    state.cent_k.copy_(r.k.cent)
    state.ncl_k.copy_(r.k.ncl)
    state.fallback.copy_(r.st.fallback)
    state.tau.copy_(r.st.tau)
    state.valid = 1
    ncl0, fb0, tau0 = np_(r.k.ncl), np_(r.st.fallback), np_(r.st.tau)
    assert set(np.flatnonzero(fb0).tolist()) == set(range(12, 24))  # the warm step covers fallback heads
    cent_q0, cent_k0 = np_(r.q.cent).astype(np.float64), np_(r.k.cent).astype(np.float64)
    Q2, K2 = gen.perturb(Q, 1103), gen.perturb(K, 1104)
    r2 = Run(Q2, K2, V, p)
    r2.cluster_q(warm_cent=state.cent_q)
    r2.cluster_k(warm=state)
    r2.score_select()
    r2.attn()
    torch.cuda.synchronize()
    assert np.array_equal(np_(r2.k.ncl), ncl0) and np.array_equal(np_(r2.st.fallback), fb0)
    assert np.array_equal(np_(r2.st.tau), tau0) and np.all(np_(r2.st.stages) == 0)
    # one warm Lloyd step from the first step's centres, on sampled rows
    out = check_clusters_sampled(r2, Q2, K2, V, 9103, tau_invariant=False)
    ties = check_scores_selection(r2, p)
    worst = check_attention_sampled(r2, Q2, K2, V, p, 9103)
    print(f"hunyuan warm: label flips {out['label_flips']}, selection ties {ties}, worst {worst}")
