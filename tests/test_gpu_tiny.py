"""GPU parity on the tiny workload (B=1, H=2, L=4096, d=64), stage by stage.

Each GPU stage is compared with the oracle recomputing that stage from the
GPU's own previous-stage outputs: k-means++ picks and normalised queries
bit-exact, Lloyd steps to fp32 rounding, labels identical except near ties,
permutations / segments / selections bit-exact, attention within
max-abs 2e-2 and relative-L2 5e-3 of fp64."""
import math

import numpy as np
import pytest

import csa_inputs as gen
from oracle import numerics as nm
from oracle import kmeans as okm
from oracle import multistage as oms
from oracle import stats as ost
from oracle import score as osc
from oracle import attention as oat
from oracle import layer as oly
from abi_helpers import (oracle_params, Run, np_, bf16_dev_to_f64, near_tie_flips, attn_error, ATTN_MAX_ABS,
                         ATTN_REL_L2, to_dev, check_clusters_sampled, check_scores_selection, check_attention_sampled,
                         selection_difference_is_near_tie)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    w = gen.get_workload("tiny")
    return gen.generate(w)


def P(**kw):
    base = dict(nq=16, m0=32, nmax=64, tau_rule=nm.TAU_INF, sel_mode=nm.SEL_TOPK, topk=8, init_sample=0,
                iters=10, seed=5)
    base.update(kw)
    return oracle_params(**base)


def _bits(x, bh):
    B, H, L, d = x.shape
    return x.reshape(B * H, L, d)[bh]


# ---------------------------------------------------------------- queries

@pytest.mark.parametrize("init_sample,L", [(0, None), (8, None), (0, 10000)])
def test_query_seeding_bit_exact(tiny, init_sample, L):
    """k-means++ picks equal the oracle's: the distance-matrix path (every
    point, s = 4096; s = 8 * 16 = 128) and the streamed path for subsamples
    above the matrix limit (every point of L = 10000)."""
    Q, K, V = tiny if L is None else gen.generate(gen.get_workload("tiny", H=1, L=L))
    p = P(iters=0, init_sample=init_sample)
    r = Run(Q, K, V, p)
    r.cluster_q()
    cent = np_(r.q.cent)
    for bh in range(r.BH):
        X = nm.bf16_to_f64(okm.normalize_queries(_bits(Q, bh)))
        C0, _ = okm.kmeanspp_init(X, 16, p.seed, nm.stream_id(bh, 0, 0), init_sample)
        assert np.array_equal(cent[bh].astype(np.float64), C0), f"head {bh}"


def test_query_lloyd_steps_and_labels(tiny):
    Q, K, V = tiny
    prev = None
    for it in range(0, 4):
        p = P(iters=it)
        r = Run(Q, K, V, p)
        r.cluster_q()
        cent = np_(r.q.cent).astype(np.float64)
        lab = np_(r.q.labels)
        for bh in range(r.BH):
            X = nm.bf16_to_f64(okm.normalize_queries(_bits(Q, bh)))
            if prev is not None:
                lab_o = okm.assign(X, prev[bh])
                ref = okm.update(X, lab_o, prev[bh])
                assert np.max(np.abs(ref - cent[bh])) < 1e-6, (it, bh)
            bad, flips, ties = near_tie_flips(X, cent[bh], lab[bh])
            assert bad == 0 and flips <= 0.001 * X.shape[0], (it, bh, bad, flips, ties)
        prev = cent


def test_query_perm_seg_rho(tiny):
    Q, K, V = tiny
    p = P()
    r = Run(Q, K, V, p)
    r.cluster_q()
    lab, perm, seg, rho, ncl = (np_(t) for t in (r.q.labels, r.q.perm, r.q.seg, r.q.rho, r.q.ncl))
    assert np.all(ncl == 16)
    for bh in range(r.BH):
        perm_o, seg_o = ost.counting_sort(lab[bh], 16)
        assert np.array_equal(perm[bh], perm_o)
        assert np.array_equal(seg[bh], seg_o)
        qn = np.linalg.norm(nm.bf16_to_f64(_bits(Q, bh)), axis=1)
        for c in range(16):
            m = lab[bh] == c
            ref = qn[m].mean() if m.any() else 0.0
            assert abs(rho[bh, c] - ref) <= 1e-5 * max(ref, 1.0)


# ---------------------------------------------------------------- keys

@pytest.mark.parametrize("init_sample", [0, 8, 64])
def test_key_seeding_and_single_stage(tiny, init_sample):
    Q, K, V = tiny
    p0 = P(iters=0, init_sample=init_sample)
    r0 = Run(Q, K, V, p0)
    r0.cluster_k()
    c0 = np_(r0.k.cent).astype(np.float64)
    for bh in range(r0.BH):
        Kx = nm.bf16_to_f64(_bits(K, bh))
        C0, _ = okm.kmeanspp_init(Kx, 32, p0.seed, nm.stream_id(bh, 1, 0), init_sample)
        assert np.array_equal(c0[bh, :32], C0), bh
    p = P()
    r = Run(Q, K, V, p)
    r.cluster_k()
    cent = np_(r.k.cent).astype(np.float64)
    lab, perm, seg, ncl = (np_(t) for t in (r.k.labels, r.k.perm, r.k.seg, r.k.ncl))
    fb, stages = np_(r.st.fallback), np_(r.st.stages)
    assert np.all(ncl == 32) and np.all(fb == 0) and np.all(stages == 1)
    for bh in range(r.BH):
        Kx = nm.bf16_to_f64(_bits(K, bh))
        bad, flips, ties = near_tie_flips(Kx, cent[bh, :32], lab[bh])
        assert bad == 0 and flips <= 0.001 * Kx.shape[0]
        perm_o, seg_o = ost.counting_sort(lab[bh], 32)
        assert np.array_equal(perm[bh], perm_o)
        assert np.array_equal(seg[bh, :33], seg_o) and np.all(seg[bh, 33:] == r.L)


def test_key_stats(tiny):
    Q, K, V = tiny
    p = P()
    r = Run(Q, K, V, p)
    r.cluster_k()
    cent = np_(r.k.cent).astype(np.float64)
    lab = np_(r.k.labels)
    kmax, kmin = bf16_dev_to_f64(r.st.kmax), bf16_dev_to_f64(r.st.kmin)
    kmean, vmean, mse = np_(r.st.kmean), np_(r.st.vmean), np_(r.st.mse)
    for bh in range(r.BH):
        st = ost.key_stats(_bits(K, bh), _bits(V, bh), lab[bh], cent[bh, :32])
        assert np.array_equal(kmax[bh, :32], st["kmax"])
        assert np.array_equal(kmin[bh, :32], st["kmin"])
        assert np.max(np.abs(kmean[bh, :32] - st["kmean"])) < 1e-5
        assert np.max(np.abs(vmean[bh, :32] - st["vmean"])) < 1e-5
        assert abs(mse[bh] - st["mse"]) <= 1e-4 * st["mse"]


@pytest.mark.parametrize("rule,param,init_sample", [(nm.TAU_MEAN_X, 1.5, 0), (nm.TAU_PCTL, 0.95, 0),
                                                    (nm.TAU_MEAN_X, 1.5, 8)])
def test_key_multistage_matches_oracle(tiny, rule, param, init_sample):
    Q, K, V = tiny
    p = P(m0=16, nmax=64, tau_rule=rule, tau_param=param, init_sample=init_sample)
    r = Run(Q, K, V, p)
    r.cluster_k()
    ncl, fb, stages, tau = np_(r.k.ncl), np_(r.st.fallback), np_(r.st.stages), np_(r.st.tau)
    cent = np_(r.k.cent).astype(np.float64)
    lab = np_(r.k.labels)
    for bh in range(r.BH):
        o = oms.cluster_keys(_bits(K, bh), p, bh)
        assert (ncl[bh], bool(fb[bh]), stages[bh]) == (o["nk"], o["fallback"], o["stages"]), bh
        assert abs(tau[bh] - o["tau"]) <= 1e-5 * o["tau"]
        Kx = nm.bf16_to_f64(_bits(K, bh))
        bad, flips, _ = near_tie_flips(Kx, cent[bh, :ncl[bh]], lab[bh])
        assert bad == 0 and flips <= 0.001 * r.L
        assert np.max(np.abs(cent[bh, :ncl[bh]] - o["cent"])) < 1e-4
        agree = np.mean(lab[bh] == o["labels"])
        assert agree >= 0.999, agree


# ---------------------------------------------------------------- scores and selection

def _sel_compare(S_gpu, sel_gpu, n_gpu, count, rho, L, d, p):
    """Rows whose GPU selection differs from the oracle's.  Returns
    (non-tie mismatches, tie mismatches)."""
    bad = ties = 0
    amax = np.max(np.abs(S_gpu[np.isfinite(S_gpu)]))
    for r in range(S_gpu.shape[0]):
        g = sel_gpu[r, :n_gpu[r]].tolist()
        o = osc.select_row(S_gpu[r].astype(np.float64), count, float(rho[r]), L, d, p).tolist()
        if g == o:
            continue
        # allowed only at a near tie of the cut (R15: scores within 1e-5 max|S|,
        # or, for top-p, cumulative mass within 1e-5 of p)
        if selection_difference_is_near_tie(S_gpu[r], count, rho[r], L, d, p, g, o, amax):
            ties += 1
        else:
            bad += 1
    return bad, ties


@pytest.mark.parametrize("mode,extra", [(nm.SEL_TOPK, {}), (nm.SEL_DENSITY, dict(sel_param=0.2)),
                                        (nm.SEL_TOPP, dict(sel_param=0.9)),
                                        (nm.SEL_TOPK, dict(score_mode=nm.SCORE_MEAN))])
def test_scores_and_selection(tiny, mode, extra):
    Q, K, V = tiny
    p = P(sel_mode=mode, **extra)
    r = Run(Q, K, V, p)
    r.cluster_q()
    r.cluster_k()
    r.score_select()
    cq = np_(r.q.cent).astype(np.float64)
    kmax, kmin = bf16_dev_to_f64(r.st.kmax), bf16_dev_to_f64(r.st.kmin)
    kmean = np_(r.st.kmean).astype(np.float64)
    seg = np_(r.k.seg)
    S = np_(r.sel.score)
    lst, n = np_(r.sel.list), np_(r.sel.n)
    rho = np_(r.q.rho)
    mask = np_(r.sel.mask).view(np.uint32)
    for bh in range(r.BH):
        count = np.diff(seg[bh])[:32]
        if p.score_mode == nm.SCORE_QUEST:
            So = osc.quest_scores(cq[bh], kmax[bh, :32], kmin[bh, :32], count)
        else:
            So = osc.mean_scores(cq[bh], kmean[bh, :32], count)
        fin = np.isfinite(So)
        assert np.array_equal(fin, np.isfinite(S[bh, :, :32]))
        assert np.all(np.isneginf(S[bh, :, 32:]))
        amax = np.max(np.abs(So[fin]))
        assert np.max(np.abs(S[bh, :, :32][fin] - So[fin])) <= 1e-5 * amax
        bad, ties = _sel_compare(S[bh, :, :32], lst[bh], n[bh], count, rho[bh], r.L, r.d, p)
        assert bad == 0, (bh, bad, ties)
        assert ties <= 0.001 * S.shape[1], (bh, "selection near ties", ties)
        for q in range(16):
            bits = np.unpackbits(mask[bh, q].view(np.uint8), bitorder="little")[:32]
            assert sorted(np.nonzero(bits)[0].tolist()) == sorted(lst[bh, q, :n[bh, q]].tolist())


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("mode,extra", [(nm.SEL_TOPK, {}), (nm.SEL_TOPK, dict(compensate=1)),
                                        (nm.SEL_DENSITY, dict(sel_param=0.15)),
                                        (nm.SEL_TOPP, dict(sel_param=0.9, compensate=1)),
                                        (nm.SEL_DENSE, {})])
def test_attention_given_gpu_selection(tiny, mode, extra):
    Q, K, V = tiny
    p = P(sel_mode=mode, **extra)
    r = Run(Q, K, V, p).all()
    O = bf16_dev_to_f64(r.O).reshape(r.BH, r.L, r.d)
    lse = np_(r.lse)
    qlab, klab, seg = np_(r.q.labels), np_(r.k.labels), np_(r.k.seg)
    lst, n = np_(r.sel.list), np_(r.sel.n)
    for bh in range(r.BH):
        Qx, Kx, Vx = (nm.bf16_to_f64(_bits(x, bh)) for x in (Q, K, V))
        rows = np.arange(r.L)
        if mode == nm.SEL_DENSE:
            Oo, lo = oat.dense_rows(Qx, Kx, Vx, rows, p.attn_scale(r.d))
        else:
            sel = [lst[bh, q, :n[bh, q]] for q in range(16)]
            st = ost.key_stats(_bits(K, bh), _bits(V, bh), klab[bh], np.zeros((32, r.d)))
            Oo, lo = oat.sparse_rows(Qx, Kx, Vx, rows, qlab[bh], klab[bh], sel, p.attn_scale(r.d), bool(p.compensate),
                                     st["count"], st["kmean"], st["vmean"])
        mx, rl2 = attn_error(O[bh], Oo)
        assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, (bh, mx, rl2)
        assert np.max(np.abs(lse[bh] - lo)) < 1e-2


def test_layer_end_to_end_against_independent_oracle(tiny):
    import torch
    import clustered_sparse_attention_amd as ac
    Q, K, V = tiny
    p = P(sel_mode=nm.SEL_TOPK, topk=8)
    r = Run(Q, K, V, p)
    state = ac.State(r.BH, r.nq, r.ncap_k, r.d, torch.device("cuda"))
    O = torch.empty_like(r.Q)
    hs = ac.ac_layer(r.shape, r.cp, r.Q, r.K, r.V, state, O, r.ws, host_stats=True)
    assert state.valid == 1
    Og = bf16_dev_to_f64(O).reshape(r.BH, r.L, r.d)
    ref = oly.run_layer(Q, K, V, p)
    for bh in range(r.BH):
        assert hs["ncl_k"][bh] == ref[bh]["k"]["nk"] and hs["fallback"][bh] == ref[bh]["k"]["fallback"]
        mx, rl2 = attn_error(Og[bh], ref[bh]["O"])
        assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, (bh, mx, rl2)
        assert hs["pairs"][bh] > 0


def test_query_and_key_clustering_side_by_side_share_a_workspace(tiny):
    """ac_cluster_q on a second stream beside ac_cluster_k, both on one
    workspace, gives bit-identical clusters, statistics and attention to the
    same calls made one after the other (the two use disjoint scratch)."""
    import torch
    import clustered_sparse_attention_amd as ac
    Q, K, V = tiny
    p = P(tau_rule=nm.TAU_MEAN_X, tau_param=1.5, m0=16, nmax=48, init_sample=8)
    seq = Run(Q, K, V, p).all()
    par = Run(Q, K, V, p)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for _ in range(2):  # the second round reuses the workspace left by the first
        side.wait_stream(main)
        ac.ac_cluster_q(par.shape, par.cp, par.Q, None, par.q, par.ws, stream=side.cuda_stream)
        par.cluster_k()
        main.wait_stream(side)
        par.score_select()
        par.attn()
    torch.cuda.synchronize()
    for name in ("labels", "perm", "seg", "cent", "ncl", "rho"):
        assert torch.equal(getattr(seq.q, name), getattr(par.q, name)), f"q.{name}"
    for name in ("labels", "perm", "seg", "cent", "ncl"):
        assert torch.equal(getattr(seq.k, name), getattr(par.k, name)), f"k.{name}"
    for name in ("kmax", "kmin", "kmean", "vmean", "fallback", "tau", "stages"):
        assert torch.equal(getattr(seq.st, name), getattr(par.st, name)), f"stats.{name}"
    assert torch.equal(seq.O, par.O)


# ---------------------------------------------------------------- tail merging (iCATS)

@pytest.mark.parametrize("block", [0, 64, 100, 1000])
def test_tail_merge_bit_exact(tiny, block):
    """ac_tail_merge against the oracle's pass 1 + pass 2 on the GPU's own
    clusters and selection: token order, segments, labels, masks, lists."""
    from abi_helpers import check_tail_merge
    Q, K, V = tiny
    for mode, extra in ((nm.SEL_TOPK, dict(topk=4)), (nm.SEL_TOPP, dict(sel_param=0.5))):
        r = Run(Q, K, V, P(sel_mode=mode, **extra)).all()
        _, _, before, after = check_tail_merge(r, block)
        assert after <= before


def test_attention_after_tail_merge(tiny):
    """The attention on merged clusters equals the oracle's attention over
    each token's merged key set; the same layer through ac_layer with
    tail_block gives the identical output."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import check_tail_merge
    Q, K, V = tiny
    block = 64
    p = P(sel_mode=nm.SEL_TOPK, topk=4, compensate=1)
    r = Run(Q, K, V, p).all()
    qm, sm, before, after = check_tail_merge(r, block)
    O = torch.empty_like(r.Q)
    ac.ac_sparse_attn(r.shape, r.cp, r.Q, r.K, r.V, qm, r.k, r.st, sm, O, None, r.ws)
    torch.cuda.synchronize()
    Og = bf16_dev_to_f64(O).reshape(r.BH, r.L, r.d)
    mlab, klab = np_(qm.labels), np_(r.k.labels)
    mlst, mn = np_(sm.list), np_(sm.n)
    for bh in range(r.BH):
        Qx, Kx, Vx = (nm.bf16_to_f64(_bits(x, bh)) for x in (Q, K, V))
        sel = [mlst[bh, c, :mn[bh, c]] for c in range(r.nq)]
        st = ost.key_stats(_bits(K, bh), _bits(V, bh), klab[bh], np.zeros((r.ncap_k, r.d)))
        Oo, _ = oat.sparse_rows(Qx, Kx, Vx, np.arange(r.L), mlab[bh], klab[bh], sel, p.attn_scale(r.d), True,
                                st["count"], st["kmean"], st["vmean"])
        mx, rl2 = attn_error(Og[bh], Oo)
        assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, (bh, mx, rl2)
    pl = P(sel_mode=nm.SEL_TOPK, topk=4, compensate=1, tail_block=block)
    rl = Run(Q, K, V, pl)
    state = ac.State(rl.BH, rl.nq, rl.ncap_k, rl.d, torch.device("cuda"))
    O2 = torch.empty_like(rl.Q)
    ac.ac_layer(rl.shape, rl.cp, rl.Q, rl.K, rl.V, state, O2, rl.ws)
    torch.cuda.synchronize()
    assert torch.equal(O2, O)


# ---------------------------------------------------------------- per-token Quest (Algorithm 2's literal shape)

@pytest.mark.parametrize("shape", [None, (3, 1000, 128)])
def test_token_quest_both_engines(tiny, shape):
    """ac_score_tokens on MFMA (TensorQuest) and on the vector ALUs against
    the oracle's eq. (1) for every query token: on the tiny layer, and on a
    ragged one (L = 1000, not a multiple of the 256-token block, d = 128);
    with ld past the last cluster (-inf fill) and ld cutting the clusters."""
    from abi_helpers import check_token_quest
    if shape is None:
        Q, K, V = tiny
    else:
        H, L, d = shape
        Q, K, V = gen.generate(gen.get_workload("tiny", H=H, L=L, d=d))
    r = Run(Q, K, V, P())
    r.cluster_k()
    for ld in (r.ncap_k + 5, 7):
        worst = check_token_quest(r, Q, K, V, ld)
        print(f"token quest shape={shape} ld={ld}: max error / bound {worst}")


# ---------------------------------------------------------------- multi-step, multi-layer policy

def test_multistep_driver_against_oracle():
    """Four denoising steps of two layers through ac_step_params and ac_layer:
    step 0 and layer 0 dense (warm-up), k_max calibrated on an uncapped first
    sparse step, SNR-guided top-p per step; the first sparse step of layer 1
    cold (counts and flags equal to the oracle's Algorithm 1 with that cap),
    later steps warm from the carried state.  Every output against the
    oracle's run of the same step (warm steps from the carried centres)."""
    import torch
    import clustered_sparse_attention_amd as ac
    from oracle import driver as odr
    from test_oracle_driver import _ell
    T, layers = 4, 2
    base = P(tau_rule=nm.TAU_MEAN_X, tau_param=1.5, m0=16, nmax=200, init_sample=8, sel_mode=nm.SEL_TOPP,
             sel_param=0.9)
    inputs = [gen.generate(gen.get_workload("tiny", seed=101 + 10 * l)) for l in range(layers)]
    topp = ac.ac_topp_schedule(_ell(T), 1, 0.6, 0.95)
    # calibration: the first sparse step uncapped, over the sparse layers' heads
    r = Run(*inputs[1], base)
    cal_state = ac.State(r.BH, r.nq, r.ncap_k, r.d, torch.device("cuda"))
    O = torch.empty_like(r.Q)
    hs = ac.ac_layer(r.shape, r.cp, r.Q, r.K, r.V, cal_state, O, r.ws, host_stats=True)
    kmax = ac.ac_kmax_calibrate(hs["ncl_k"], 0.5)
    assert kmax == odr.kmax_calibrate(hs["ncl_k"], 0.5) > 0
    sch = ac.Schedule(warmup_steps=1, warmup_layers=1, nmax=kmax, topp=topp)
    cbase = r.cp
    states = {}
    cur = [list(x) for x in inputs]
    for step in range(T):
        if step > 0:  # next-step inputs: 2% perturbations of Q and K
            for l in range(layers):
                cur[l][0] = gen.perturb(cur[l][0], 1103 + 7 * step + l)
                cur[l][1] = gen.perturb(cur[l][1], 2203 + 7 * step + l)
        for l in range(layers):
            cp = ac.ac_step_params(cbase, sch, step, l)
            po = odr.step_params(base, step, l, 1, 1, kmax, topp)
            assert (cp.sel_mode, cp.nmax) == (po.sel_mode, po.nmax)
            Qb, Kb, Vb = cur[l]
            rr = Run(Qb, Kb, Vb, po)
            # the state is laid out for the sparse steps' key capacity (k_max - 1 + m0)
            st = states.setdefault(l, ac.State(rr.BH, rr.nq, kmax - 1 + base.m0, rr.d, torch.device("cuda")))
            was_valid = st.valid
            prev = None if not was_valid else [dict(cent_q=np_(st.cent_q)[bh].astype(np.float64),
                                                      cent_k=np_(st.cent_k)[bh, :int(np_(st.ncl_k)[bh])].astype(
                                                          np.float64),
                                                      fallback=bool(np_(st.fallback)[bh]), tau=float(np_(st.tau)[bh]))
                                                 for bh in range(rr.BH)]
            Og = torch.empty_like(rr.Q)
            hs = ac.ac_layer(rr.shape, cp, rr.Q, rr.K, rr.V, st, Og, rr.ws, host_stats=True)
            Og = bf16_dev_to_f64(Og).reshape(rr.BH, rr.L, rr.d)
            dense = po.sel_mode == nm.SEL_DENSE
            assert st.valid == (0 if dense and not was_valid else 1)
            for bh in range(rr.BH):
                Qh, Kh, Vh = (_bits(x, bh) for x in (Qb, Kb, Vb))
                if dense:
                    Qx, Kx, Vx = (nm.bf16_to_f64(x) for x in (Qh, Kh, Vh))
                    Oo, _ = oat.dense_rows(Qx, Kx, Vx, np.arange(rr.L), po.attn_scale(rr.d))
                    assert hs["pairs"][bh] == rr.L * rr.L
                else:
                    ref = oly.run_head(Qh, Kh, Vh, po, bh, warm=None if prev is None else prev[bh])
                    Oo = ref["O"]
                    if prev is None:
                        assert hs["ncl_k"][bh] == ref["k"]["nk"] and hs["fallback"][bh] == ref["k"]["fallback"]
                mx, rl2 = attn_error(Og[bh], Oo)
                assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, (step, l, bh, mx, rl2)


# ---------------------------------------------------------------- interaction-aware key clustering (iCATS)

def _metric_label_check(X, C, M, lab_gpu):
    """GPU labels against the metric argmin for the GPU's centres; a mismatch
    is allowed only where the two best distances are within the rounding of
    the kernel's operands (x . M c with M c split into two bf16 parts)."""
    from oracle import interaction as oia
    Dm = oia.metric_sq_dist(X, C, M)
    lab_o = np.argmin(Dm, axis=1)
    srt = np.sort(Dm, axis=1)
    MC = C @ M  # rows M c (M is symmetric)
    scale = np.linalg.norm(X, axis=1) * np.max(np.linalg.norm(MC, axis=1)) + np.abs(srt[:, 0])
    tie = (srt[:, 1] - srt[:, 0]) < 1e-4 * scale
    bad = (lab_o != lab_gpu) & ~tie
    return int(bad.sum()), int(((lab_o != lab_gpu) & tie).sum())


@pytest.mark.parametrize("iters", [0, 1, 10])
def test_interaction_aware_key_clustering(tiny, iters):
    """iCATS interaction-aware clustering: M_Q from the GPU's query clusters
    against the oracle's (raw member means), then the metric k-means of the
    keys against the oracle's from the same k-means++ seeds: centres, labels
    (up to near ties), order and statistics."""
    import torch
    import clustered_sparse_attention_amd as ac
    from oracle import interaction as oia
    Q, K, V = tiny
    p = P(iters=iters, m0=24, nmax=64)
    r = Run(Q, K, V, p)
    r.cluster_q()
    M = torch.empty((r.BH, r.d, r.d), dtype=torch.float32, device="cuda")
    ac.ac_interaction_matrix(r.shape, r.cp, r.Q, r.q, M, r.ws)
    ac.ac_cluster_k_metric(r.shape, r.cp, r.K, r.V, M, r.k, r.st, r.ws)
    torch.cuda.synchronize()
    Mg = np_(M).astype(np.float64)
    qlab = np_(r.q.labels)
    cent, lab, perm, seg, ncl = (np_(t) for t in (r.k.cent, r.k.labels, r.k.perm, r.k.seg, r.k.ncl))
    kmax, kmin = bf16_dev_to_f64(r.st.kmax), bf16_dev_to_f64(r.st.kmin)
    assert np.all(ncl == 24) and np.all(np_(r.st.fallback) == 0) and np.all(np_(r.st.stages) == 1)
    for bh in range(r.BH):
        Mo = oia.interaction_matrix(_bits(Q, bh), qlab[bh], r.nq)
        assert np.max(np.abs(Mg[bh] - Mo)) <= 1e-6 * np.max(np.abs(Mo)), bh
        ref = oia.cluster_keys_metric(_bits(K, bh), p, bh, Mg[bh])
        C = cent[bh, :24].astype(np.float64)
        assert np.max(np.abs(C - ref["cent"])) <= 1e-5 * max(1.0, np.max(np.abs(ref["cent"]))), bh
        X = nm.bf16_to_f64(_bits(K, bh))
        bad, flips = _metric_label_check(X, C, Mg[bh], lab[bh])
        assert bad == 0 and flips <= 0.001 * r.L, (bh, bad, flips)
        perm_o, seg_o = ost.counting_sort(lab[bh], 24)
        assert np.array_equal(perm[bh], perm_o) and np.array_equal(seg[bh, :25], seg_o)
        st = ost.key_stats(_bits(K, bh), _bits(V, bh), lab[bh], C)
        assert np.array_equal(kmax[bh, :24], st["kmax"]) and np.array_equal(kmin[bh, :24], st["kmin"])
    # the metric clusters drive the rest of the layer like Algorithm 1's
    r.score_select()
    r.attn()
    torch.cuda.synchronize()
    from abi_helpers import check_attention_sampled
    check_attention_sampled(r, Q, K, V, p, 9001, nrows=512)


# ---------------------------------------------------------------- small, ragged and degenerate layers

@pytest.mark.parametrize("B,H,L,d,kw,zero_rows", [
    (1, 1, 1, 64, {}, 0),
    (1, 1, 1, 128, dict(sel_mode=nm.SEL_DENSITY, sel_param=0.5, compensate=1), 1),
    (1, 2, 37, 128, {}, 3),
    (1, 3, 300, 64, dict(tau_rule=nm.TAU_MEAN_X, tau_param=1.0, nmax=40), 0),
    (1, 3, 300, 64, dict(tau_rule=nm.TAU_MEAN_X, tau_param=0.8, nmax=70), 2),
    (1, 2, 513, 64, dict(sel_mode=nm.SEL_TOPP, sel_param=0.9, compensate=1), 0),
    (1, 1, 700, 128, dict(sel_mode=nm.SEL_DENSITY, sel_param=0.2, compensate=1, tau_rule=nm.TAU_PCTL,
                          tau_param=0.9), 5),
    (2, 2, 300, 128, {}, 0),
    (3, 1, 513, 64, dict(sel_mode=nm.SEL_DENSITY, sel_param=0.2, compensate=1), 4),
])
def test_small_ragged_and_degenerate_layers(B, H, L, d, kw, zero_rows):
    """Layers far from the kernels' tile sizes: a single token (one cluster on
    each side, the attention returns V), fewer tokens than centres, lengths
    that are not multiples of any block, rows of zero queries (their
    normalised query is 0), multi-stage keys with a low cap so that heads
    fall back to dense, and batches of several sequences.  Every stage is
    checked against the oracle given the GPU's earlier stages, the attention
    on every row."""
    Q, K, V = gen.generate(gen.get_workload("tiny", B=B, H=H, L=L, d=d))
    if zero_rows:
        Q = Q.copy()
        Q[:, :, :zero_rows, :] = 0
    p = P(**kw)
    r = Run(Q, K, V, p).all()
    out = check_clusters_sampled(r, Q, K, V, rows_seed=1, nrows=L)
    check_scores_selection(r, p)
    check_attention_sampled(r, Q, K, V, p, rows_seed=2, nrows=L)
    if L == 1:
        O = bf16_dev_to_f64(r.O).reshape(r.BH, 1, d)
        assert np.array_equal(O, nm.bf16_to_f64(V.reshape(r.BH, 1, d)))
        assert out["ncl"] == [1] * r.BH



def test_small_layer_rule_runs_dense():
    """min_sparse_gflop: a layer whose dense attention work 4*B*H*L^2*d is
    below the threshold runs the dense path (bit-identical to sel_mode DENSE,
    no clustering, the state left invalid); above it the layer runs sparse."""
    import torch
    import clustered_sparse_attention_amd as ac
    from abi_helpers import abi_params
    Q, K, V = gen.generate(gen.get_workload("tiny"))
    p = P(sel_mode=nm.SEL_TOPK, topk=8)
    r = Run(Q, K, V, p)
    dense_gflop = 4e-9 * r.BH * r.L * r.L * r.d        # 8.6 GFLOP
    dev = torch.device("cuda")
    outs = {}
    for name, thr, mode in (("rule", 10, nm.SEL_TOPK), ("dense", 0, nm.SEL_DENSE), ("sparse", 8, nm.SEL_TOPK)):
        cp = abi_params(P(sel_mode=mode, topk=8))
        cp.min_sparse_gflop = thr
        st = ac.State(r.BH, r.nq, r.ncap_k, r.d, dev)
        O = torch.empty_like(r.Q)
        hs = ac.ac_layer(r.shape, cp, r.Q, r.K, r.V, st, O, r.ws, host_stats=True)
        outs[name] = (O.clone(), st.valid, hs)
    assert 8 < dense_gflop < 10
    assert torch.equal(outs["rule"][0], outs["dense"][0])
    assert outs["rule"][1] == 0 and outs["dense"][1] == 0 and outs["sparse"][1] == 1
    assert np.all(outs["rule"][2]["pairs"] == r.L * r.L) and np.all(outs["rule"][2]["ncl_k"] == 0)
    assert np.all(outs["sparse"][2]["ncl_k"] == 32)
