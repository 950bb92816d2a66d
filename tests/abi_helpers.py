"""Shared helpers of the GPU tests: parameter mapping between the oracle and
the C ABI, device upload, and running the layer's entry points stage by
stage through the binding.  Not a test module."""
from __future__ import annotations

import math

import numpy as np

import csa_inputs as gen
from oracle import numerics as nm


def f32(x: float) -> float:
    """Round a Python float to float32 (the ABI carries float parameters)."""
    return float(np.float32(x))


def oracle_params(**kw) -> nm.Params:
    p = nm.Params(**kw)
    p.tau_param = f32(p.tau_param)
    p.sel_param = f32(p.sel_param)
    p.scale = f32(p.scale)
    return p


def abi_params(p: nm.Params):
    import clustered_sparse_attention_amd as ac
    return ac.params_default(nq=p.nq, iters=p.iters, iters_warm=p.iters_warm, m0=p.m0, nmax=p.nmax,
                             tau_rule=p.tau_rule, tau_param=p.tau_param, score_mode=p.score_mode,
                             sel_mode=p.sel_mode, topk=p.topk, sel_param=p.sel_param, compensate=p.compensate,
                             scale=p.scale, init_sample=p.init_sample, tail_block=p.tail_block, seed=p.seed)


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_(t):
    return t.detach().cpu().numpy()


class Run:
    """Runs the four entry points on one workload and keeps every output."""

    def __init__(self, Qb, Kb, Vb, p: nm.Params):
        import torch
        import clustered_sparse_attention_amd as ac
        B, H, L, d = Qb.shape
        self.B, self.H, self.L, self.d = B, H, L, d
        self.BH = B * H
        self.p = p
        self.cp = abi_params(p)
        self.shape = ac.Shape(B, H, L, d)
        self.ncap_k, self.ws_bytes = ac.ac_sizes(self.shape, self.cp)
        self.nq = min(p.nq, L)
        dev = torch.device("cuda")
        self.Q, self.K, self.V = to_dev(Qb), to_dev(Kb), to_dev(Vb)
        self.ws = ac.workspace(self.ws_bytes, dev)
        self.q = ac.Clusters(self.BH, L, self.nq, d, dev, rho=True)
        self.k = ac.Clusters(self.BH, L, self.ncap_k, d, dev, rho=False)
        self.st = ac.KStats(self.BH, self.ncap_k, d, dev)
        self.sel = ac.Selection(self.BH, self.nq, self.ncap_k, dev)
        self.O = torch.empty_like(self.Q)
        self.lse = torch.empty((self.BH, L), dtype=torch.float32, device=dev)

    def cluster_q(self, warm_cent=None):
        import clustered_sparse_attention_amd as ac
        ac.ac_cluster_q(self.shape, self.cp, self.Q, warm_cent, self.q, self.ws)

    def cluster_k(self, warm=None):
        import clustered_sparse_attention_amd as ac
        ac.ac_cluster_k(self.shape, self.cp, self.K, self.V, warm, self.k, self.st, self.ws)

    def score_select(self):
        import clustered_sparse_attention_amd as ac
        ac.ac_score_select(self.shape, self.cp, self.q, self.k, self.st, self.sel, self.ws)

    def attn(self):
        import clustered_sparse_attention_amd as ac
        ac.ac_sparse_attn(self.shape, self.cp, self.Q, self.K, self.V, self.q, self.k, self.st, self.sel, self.O,
                          self.lse, self.ws)

    def all(self):
        self.cluster_q()
        self.cluster_k()
        self.score_select()
        self.attn()
        import torch
        torch.cuda.synchronize()
        return self


def near_tie_flips(X, C, lab_gpu, rel=1e-5):
    """Compare GPU labels with the oracle's nearest centre (fp64, given the
    GPU's centres).  Returns (mismatches, near-tie mismatches, near ties)."""
    from oracle import kmeans as okm
    d2 = okm.sq_dist(X, C)
    lab_o = np.argmin(d2, axis=1)
    srt = np.sort(d2, axis=1)
    gap = (srt[:, 1] - srt[:, 0]) if C.shape[0] > 1 else np.full(X.shape[0], np.inf)
    scale = np.sum(X * X, axis=1) + np.sum(C[lab_o] ** 2, axis=1)
    tie = gap < rel * scale
    mism = lab_o != lab_gpu
    return int(np.sum(mism & ~tie)), int(np.sum(mism & tie)), int(np.sum(tie))


def attn_error(O_gpu: np.ndarray, O_ref: np.ndarray):
    """(max abs error, relative L2 error)."""
    diff = O_gpu - O_ref
    return float(np.max(np.abs(diff))), float(np.linalg.norm(diff) / max(np.linalg.norm(O_ref), 1e-30))


ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3


# ---------------------------------------------------------------- full-size sampled checks

def workload_oracle_params(name: str, variant: str = "density", compensate: int = 0) -> nm.Params:
    """The parameters bench.py times for a workload, as an oracle Params."""
    import bench
    kw = bench.workload_params(name, variant, compensate)
    kw = {k: v for k, v in kw.items() if k in nm.Params.__dataclass_fields__}
    return oracle_params(**kw)


def check_clusters_sampled(r: "Run", Qb, Kb, Vb, rows_seed: int, nrows: int = 2048, tau_invariant: bool = True):
    """Stage-wise checks of the clustering outputs of every head, given the
    GPU's own earlier stages.  Returns a summary dict; raises on a failure."""
    from oracle import kmeans as okm
    from oracle import stats as ost
    B, H, L, d = Qb.shape
    BH = B * H
    Qf, Kf, Vf = (x.reshape(BH, L, d) for x in (Qb, Kb, Vb))
    qlab, qperm, qseg, qcent = (np_(t) for t in (r.q.labels, r.q.perm, r.q.seg, r.q.cent))
    klab, kperm, kseg, kcent, ncl = (np_(t) for t in (r.k.labels, r.k.perm, r.k.seg, r.k.cent, r.k.ncl))
    fb, tau, mse = np_(r.st.fallback), np_(r.st.tau), np_(r.st.mse)
    kmax, kmin = bf16_dev_to_f64(r.st.kmax), bf16_dev_to_f64(r.st.kmin)
    kmean, vmean = np_(r.st.kmean), np_(r.st.vmean)
    rows = gen.row_sample(L, nrows, rows_seed)
    out = dict(label_flips=0, label_ties=0, fallback=int(fb.sum()), ncl=ncl.tolist())
    for h in range(BH):
        nk = int(ncl[h])
        assert 1 <= nk <= r.ncap_k
        # query labels: nearest centre of the sampled rows (normalised queries)
        Xq = nm.bf16_to_f64(okm.normalize_queries(Qf[h][rows]))
        bad, flips, ties = near_tie_flips(Xq, qcent[h].astype(np.float64), qlab[h][rows])
        assert bad == 0, (h, "query labels", bad)
        out["label_flips"] += flips
        out["label_ties"] += ties
        # key labels: nearest over all of C
        Xk = nm.bf16_to_f64(Kf[h][rows])
        C = kcent[h, :nk].astype(np.float64)
        bad, flips, ties = near_tie_flips(Xk, C, klab[h][rows])
        assert bad == 0, (h, "key labels", bad)
        out["label_flips"] += flips
        out["label_ties"] += ties
        # Algorithm 1 invariant: without fallback every key is within tau of a centre
        if tau_invariant and not fb[h]:
            dmin = np.sqrt(np.min(okm.sq_dist(Xk, C), axis=1))
            assert np.all(dmin < tau[h] * (1 + 1e-5)), (h, "tau invariant")
        elif fb[h]:
            assert nk >= r.p.nmax
        # permutations and segments: bit-exact
        for lab, perm, seg, m in ((qlab[h], qperm[h], qseg[h], r.nq), (klab[h], kperm[h], kseg[h], nk)):
            perm_o, seg_o = ost.counting_sort(lab, m)
            assert np.array_equal(perm, perm_o), (h, "perm")
            assert np.array_equal(seg[:m + 1], seg_o), (h, "seg")
        # statistics of every key cluster
        st = ost.key_stats(Kf[h], Vf[h], klab[h], C)
        assert np.array_equal(kmax[h, :nk], st["kmax"]) and np.array_equal(kmin[h, :nk], st["kmin"]), (h, "max/min")
        scale_k = max(1.0, float(np.max(np.abs(st["kmean"]))))
        assert np.max(np.abs(kmean[h, :nk] - st["kmean"])) <= 1e-5 * scale_k, (h, "kmean")
        assert np.max(np.abs(vmean[h, :nk] - st["vmean"])) <= 1e-5 * max(1.0, float(np.max(np.abs(st["vmean"])))), h
        assert abs(mse[h] - st["mse"]) <= 1e-4 * st["mse"], (h, "mse")
    assert out["label_flips"] <= 0.001 * 2 * BH * rows.size
    return out


TOPP_TIE = 1e-5  # |cumulative mass at the cut - p| below which a top-p cut is a near tie


def selection_difference_is_near_tie(S_row, count, rho_r, L, d, p: nm.Params, g, o, amax) -> bool:
    """Whether a GPU selection g that differs from the oracle's o (both in
    selection order, from the same fp32 scores) differs only at a near tie:
    for TOPK / DENSITY every differing cluster scores within 1e-5 * max|S| of
    the oracle's cut; for TOPP both are prefixes of the same score order and
    the oracle's cumulative mass is within 1e-5 of p at every cut between
    the two lengths."""
    from oracle import score as osc
    if p.sel_mode != nm.SEL_TOPP:
        diff = set(g) ^ set(o)
        cut = S_row[o[-1]]
        return all(abs(S_row[c] - cut) < 1e-5 * amax for c in diff)
    order = osc.order_clusters(np.asarray(S_row, dtype=np.float64), count).tolist()
    if order[:len(g)] != list(g) or order[:len(o)] != list(o):
        return False
    sc = np.asarray(S_row, dtype=np.float64)[order]
    z = float(rho_r) * sc * p.attn_scale(d) + np.log(np.asarray(count, dtype=np.float64)[order])
    w = np.exp(z - np.max(z))
    cum = np.cumsum(w / np.sum(w))
    lo, hi = min(len(g), len(o)), max(len(g), len(o))
    return all(abs(cum[k - 1] - p.sel_param) < TOPP_TIE for k in range(lo, hi))


def check_scores_selection(r: "Run", p: nm.Params):
    """Scores against the oracle's eq. (1) from the GPU's centres and
    statistics; selections against the oracle's selection from the GPU's
    scores (differences only between near-equal scores / masses)."""
    from oracle import score as osc
    BH = r.BH
    cq = np_(r.q.cent).astype(np.float64)
    kmax, kmin = bf16_dev_to_f64(r.st.kmax), bf16_dev_to_f64(r.st.kmin)
    kmean = np_(r.st.kmean).astype(np.float64)
    kseg, ncl, rho = np_(r.k.seg), np_(r.k.ncl), np_(r.q.rho)
    S = np_(r.sel.score)
    lst, n = np_(r.sel.list), np_(r.sel.n)
    ties = 0
    for h in range(BH):
        nk = int(ncl[h])
        count = np.diff(kseg[h])[:nk]
        if p.score_mode == nm.SCORE_QUEST:
            So = osc.quest_scores(cq[h], kmax[h, :nk], kmin[h, :nk], count)
        else:
            So = osc.mean_scores(cq[h], kmean[h, :nk], count)
        fin = np.isfinite(So)
        assert np.array_equal(fin, np.isfinite(S[h, :, :nk])), h
        amax = np.max(np.abs(So[fin]))
        assert np.max(np.abs(S[h, :, :nk][fin] - So[fin])) <= 1e-5 * amax, h
        for q in range(r.nq):
            g = lst[h, q, :n[h, q]].tolist()
            o = osc.select_row(S[h, q, :nk].astype(np.float64), count, float(rho[h, q]), r.L, r.d, p).tolist()
            if g != o:
                near = selection_difference_is_near_tie(S[h, q, :nk], count, rho[h, q], r.L, r.d, p, g, o, amax)
                assert near, (h, q, "selection", len(g), len(o))
                ties += 1
    assert ties <= 0.001 * BH * r.nq, ("selection near ties", ties)
    return ties


def cluster_rows(labels: np.ndarray, nclusters: int, per: int, seed: int) -> np.ndarray:
    """Seeded sample of query rows taken cluster by cluster: ``nclusters``
    distinct non-empty query clusters, up to ``per`` rows of each, ascending."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cand = np.unique(labels)
    pick = rng.choice(cand, size=min(nclusters, cand.size), replace=False)
    rows = [rng.choice(np.flatnonzero(labels == c), size=min(per, int(np.sum(labels == c))), replace=False)
            for c in pick]
    return np.sort(np.concatenate(rows))


def check_attention_sampled(r: "Run", Qb, Kb, Vb, p: nm.Params, rows_seed: int, nrows: int = 2048, q=None, sel=None,
                            clusters: int = 0):
    """Attention of a seeded sample of query rows per head against the fp64
    oracle given the GPU's clusters and selection (q / sel: other query
    clusters and selection than the Run's, e.g. tail-merged ones).  The
    sample is nrows rows drawn from the whole head, or with clusters > 0
    nrows / clusters rows from each of that many query clusters of the head
    (the oracle gathers a query cluster's selected keys once for all its
    sampled rows, which matters when selections keep most keys)."""
    from oracle import stats as ost
    from oracle import attention as oat
    B, H, L, d = Qb.shape
    BH = B * H
    Qf, Kf, Vf = (x.reshape(BH, L, d) for x in (Qb, Kb, Vb))
    O = bf16_dev_to_f64(r.O).reshape(BH, L, d)
    q = r.q if q is None else q
    sel_ = r.sel if sel is None else sel
    qlab, klab, ncl, fb = np_(q.labels), np_(r.k.labels), np_(r.k.ncl), np_(r.st.fallback)
    lst, n = np_(sel_.list), np_(sel_.n)
    head_rows = gen.row_sample(L, nrows, rows_seed)
    worst = (0.0, 0.0)
    for h in range(BH):
        rows = cluster_rows(qlab[h], clusters, nrows // clusters, rows_seed + h) if clusters else head_rows
        Qx, Kx, Vx = (nm.bf16_to_f64(x[h]) for x in (Qf, Kf, Vf))
        if fb[h] or p.sel_mode == nm.SEL_DENSE:
            Oo = np.concatenate([oat.dense_rows(Qx, Kx, Vx, rows[i:i + 256], p.attn_scale(d))[0]
                                 for i in range(0, rows.size, 256)])
        else:
            nk = int(ncl[h])
            cnt = kmean = vmean = None
            if p.compensate:
                st = ost.key_stats(Kf[h], Vf[h], klab[h], np.zeros((nk, d)))
                cnt, kmean, vmean = st["count"], st["kmean"], st["vmean"]
            sel = [lst[h, q, :n[h, q]] for q in range(r.nq)]
            Oo, _ = oat.sparse_rows(Qx, Kx, Vx, rows, qlab[h], klab[h], sel, p.attn_scale(d), bool(p.compensate),
                                    cnt, kmean, vmean)
        mx, rl2 = attn_error(O[h][rows], Oo)
        assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, (h, mx, rl2)
        worst = (max(worst[0], mx), max(worst[1], rl2))
    return worst


def unpack_masks(words: np.ndarray, nbits: int) -> np.ndarray:
    """[..., mwords] uint32 bitmasks -> [..., nbits] bool (bit c of word c // 32)."""
    w = words.astype(np.uint64)
    bits = (w[..., :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(*words.shape[:-1], -1)[..., :nbits].astype(bool)


def check_tail_merge(r, block, heads=None):
    """GPU ac_tail_merge of a Run's query clusters and selection against the
    oracle's tail_merge on the same inputs, bit for bit: new token order,
    segments, labels, masks, lists and counts.  Returns (q_out, sel_out,
    blocks before, blocks after) summed over the checked heads."""
    import torch
    import clustered_sparse_attention_amd as ac
    from oracle import tailmerge as tm
    dev = torch.device("cuda")
    qm = ac.Clusters(r.BH, r.L, r.nq, r.d, dev, rho=False)
    sm = ac.Selection(r.BH, r.nq, r.ncap_k, dev, score=False)
    ac.ac_tail_merge(r.shape, r.cp, block, r.q, r.sel, qm, sm, r.ws)
    torch.cuda.synchronize()
    b = block if block > 0 else (384 if r.d == 64 else 256)  # the attention's query block
    perm, seg = np_(r.q.perm), np_(r.q.seg)
    lst, n, mask = np_(r.sel.list), np_(r.sel.n), np_(r.sel.mask).view(np.uint32)
    mperm, mseg, mlab = np_(qm.perm), np_(qm.seg), np_(qm.labels)
    mlst, mn, mmask = np_(sm.list), np_(sm.n), np_(sm.mask).view(np.uint32)
    before = after = 0
    for bh in (range(r.BH) if heads is None else heads):
        sizes = np.diff(seg[bh][:r.nq + 1])
        masks = unpack_masks(mask[bh], r.ncap_k)
        lists = [lst[bh, c, :n[bh, c]] for c in range(r.nq)]
        pieces, nmask, nlist, nsize = tm.tail_merge(sizes, masks, lists, b)
        eperm, eseg = tm.apply(perm[bh], seg[bh], pieces)
        assert np.array_equal(mseg[bh][:r.nq + 1], eseg), f"head {bh}: segments"
        assert np.array_equal(mperm[bh], eperm), f"head {bh}: token order"
        for c in range(r.nq):
            assert np.all(mlab[bh][eperm[eseg[c]:eseg[c + 1]]] == c), f"head {bh}: labels of {c}"
            assert mn[bh, c] == len(nlist[c]) and np.array_equal(mlst[bh, c, :mn[bh, c]], nlist[c]), \
                f"head {bh}: list of {c}"
        assert np.array_equal(unpack_masks(mmask[bh], r.ncap_k), nmask), f"head {bh}: masks"
        before += tm.blocks(sizes, b)
        after += tm.blocks(nsize, b)
    return qm, sm, before, after


def check_token_quest(r, Qb, Kb, Vb, ld, rows=None, engines=(0, 1)):
    """ac_score_tokens (each engine) against the oracle's per-token Quest
    scores (eq. (1) in fp64, key max / min from the oracle's statistics of
    the GPU's key labels) on every head, on all query rows or a sample.
    Entries for non-empty clusters within 4 d 2^-24 sum_d |q_d| max(|kmax_d|,
    |kmin_d|) (fp32 summation of exact products); every other column of
    the ld written ones -inf.  Returns the largest error relative to that
    bound, per engine."""
    import torch
    import clustered_sparse_attention_amd as ac
    from oracle import stats as ost
    from oracle import score as osc
    B, H, L, d = Qb.shape
    BH = B * H
    Qf, Kf, Vf = (x.reshape(BH, L, d) for x in (Qb, Kb, Vb))
    klab, ncl = np_(r.k.labels), np_(r.k.ncl)
    rows = np.arange(L) if rows is None else rows
    S = torch.empty((BH, L, ld), dtype=torch.float32, device="cuda")
    worst = {}
    outs = {}
    for eng in engines:
        S.fill_(float("nan"))
        ac.ac_score_tokens(r.shape, r.cp, r.Q, r.k, r.st, eng, S, ld)
        torch.cuda.synchronize()
        outs[eng] = S[:, rows, :].cpu().numpy()
        worst[eng] = 0.0
    for h in range(BH):
        nk = int(ncl[h])
        st = ost.key_stats(Kf[h], Vf[h], klab[h], np.zeros((nk, d)))
        Qx = nm.bf16_to_f64(Qf[h][rows])
        So = osc.token_quest_scores(Qx, st["kmax"], st["kmin"], st["count"])
        bound = 4 * d * 2.0 ** -24 * (np.abs(Qx) @ np.maximum(np.abs(st["kmax"]), np.abs(st["kmin"])).T) + 1e-30
        m = min(nk, ld)
        live = np.zeros(ld, bool)
        live[:m] = st["count"][:m] > 0
        for eng in engines:
            Sg = outs[eng][h]
            assert np.all(np.isneginf(Sg[:, ~live])), (h, eng, "dead columns")
            err = np.abs(Sg[:, :m][:, live[:m]] - So[:, :m][:, live[:m]]) / bound[:, :m][:, live[:m]]
            assert err.size == 0 or np.max(err) <= 1.0, (h, eng, float(np.max(err)))
            worst[eng] = max(worst[eng], float(np.max(err)) if err.size else 0.0)
    return worst
