"""GPU parity of ClusterAttention's principal-component split (ac_cluster_q_pca,
ac_cluster_k_pca) against the oracle, split by split.

The trace gives each node's direction and the token order after each level.
For every internal node, given the GPU's order before the level: the node's
tokens are ascending (stable partitions), the direction is a unit vector
oriented as the reading fixes and captures the leading variance of the node's
subsample (Rayleigh quotient against the fp64 covariance's largest
eigenvalue), and the split the oracle makes along that direction equals the
GPU's except at projection near ties.  Then the clusters' shape (sizes, order,
labels, segments) is exact, centres and statistics match the oracle, and the
attention over PCA clusters matches the oracle given the GPU's selection."""
import numpy as np
import pytest

import csa_inputs as gen
from oracle import numerics as nm
from oracle import kmeans as okm
from oracle import pcasplit as ops
from oracle import stats as ost
from abi_helpers import Run, np_, bf16_dev_to_f64, oracle_params, check_scores_selection, check_attention_sampled

pytestmark = pytest.mark.gpu

RAYLEIGH_MIN = 0.9      # fraction of the leading eigenvalue the GPU direction must capture
PROJ_TIE = 1e-5         # projection near tie, relative to the node's largest row norm


def _nodes(L, b):
    """Internal nodes level by level, left to right: (level, start, count)."""
    out, cur, lvl = [], ([(0, L)] if L > b else []), 0
    while cur:
        nxt = []
        for st, n in cur:
            out.append((lvl, st, n))
            nl, nr = ops.split_sizes(n, b)
            if nl > b:
                nxt.append((st, nl))
            if nr > b:
                nxt.append((st + nl, nr))
        cur, lvl = nxt, lvl + 1
    return out


def check_pca_trace(X, b, dirs, perms):
    """Every split of one head; X fp64 [L, d] (the rows clustered)."""
    L = X.shape[0]
    nodes = _nodes(L, b)
    nlev = max((lv for lv, _, _ in nodes), default=-1) + 1
    assert perms.shape[0] >= nlev
    ties = 0
    for k, (lv, st, n) in enumerate(nodes):
        before = np.arange(L) if lv == 0 else perms[lv - 1]
        after = perms[lv]
        idx = before[st:st + n]
        assert np.all(np.diff(idx) > 0), (k, "node tokens not ascending")
        v = dirs[k].astype(np.float64)
        assert abs(np.linalg.norm(v) - 1) < 1e-4, (k, "direction norm")
        assert v[np.argmax(np.abs(v))] > 0, (k, "orientation")
        sub = idx[ops.subsample(n, 512)]
        Y = X[sub] - X[sub].mean(axis=0)
        C = Y.T @ Y
        lam = np.linalg.eigvalsh(C)[-1]
        if lam > 0:
            assert v @ C @ v >= RAYLEIGH_MIN * lam, (k, "direction quality", v @ C @ v / lam)
        nl, _ = ops.split_sizes(n, b)
        lo_g, hi_g = after[st:st + nl], after[st + nl:st + n]
        assert np.all(np.diff(lo_g) > 0) and np.all(np.diff(hi_g) > 0), (k, "children not stable")
        lo_o, hi_o = ops.split_node(X, idx, b, v)
        if not np.array_equal(lo_g, lo_o):
            p = X[idx] @ v
            thr = np.sort(p)[nl - 1:nl + 1].mean()
            tol = PROJ_TIE * max(1.0, float(np.max(np.linalg.norm(X[idx], axis=1))))
            moved = np.setxor1d(lo_g, lo_o)
            assert np.all(np.abs(X[moved] @ v - thr) < tol), (k, "split", moved.size)
            ties += 1
    return ties


def _check_clusters(X, b, lab, perm, seg, ncl, cent):
    L = X.shape[0]
    nc = -(-L // b)
    assert ncl == nc
    assert np.array_equal(seg[:nc + 1], np.minimum(np.arange(nc + 1) * b, L))
    assert np.array_equal(lab[perm], np.arange(L) // b)
    perm_o, seg_o = ost.counting_sort(lab, nc)
    assert np.array_equal(perm, perm_o) and np.array_equal(seg[:nc + 1], seg_o)
    for c in range(nc):
        ref = X[perm[seg[c]:seg[c + 1]]].mean(axis=0)
        assert np.max(np.abs(cent[c] - ref)) <= 1e-6 * max(1.0, float(np.max(np.abs(ref)))), c


def _run_pca(Q, K, V, p, bq, bk, trace=True):
    import torch
    import clustered_sparse_attention_amd as ac
    r = Run(Q, K, V, p)
    dev = torch.device("cuda")
    tq = ac.PcaTrace(r.BH, r.L, bq, ops.levels(r.L, bq), r.d, dev) if trace else None
    tk = ac.PcaTrace(r.BH, r.L, bk, ops.levels(r.L, bk), r.d, dev) if trace else None
    ac.ac_cluster_q_pca(r.shape, r.cp, r.Q, bq, r.q, r.ws, trace=tq)
    ac.ac_cluster_k_pca(r.shape, r.cp, r.K, r.V, bk, r.k, r.st, r.ws, trace=tk)
    torch.cuda.synchronize()
    return r, tq, tk


@pytest.mark.parametrize("L,d,bq,bk", [(4096, 64, 256, 64), (4133, 128, 256, 32), (700, 64, 64, 16), (20, 128, 16, 16)])
def test_pca_split_small(L, d, bq, bk):
    w = gen.get_workload("tiny", H=2, L=L, d=d)
    Q, K, V = gen.generate(w)
    p = oracle_params(nq=-(-L // bq), m0=32, nmax=max(64, -(-L // bk) + 1), sel_mode=nm.SEL_DENSITY, sel_param=0.2)
    r, tq, tk = _run_pca(Q, K, V, p, bq, bk)
    ties = 0
    for h in range(r.BH):
        Xq = nm.bf16_to_f64(okm.normalize_queries(Q.reshape(r.BH, L, d)[h]))
        Xk = nm.bf16_to_f64(K.reshape(r.BH, L, d)[h])
        if L > bq:
            ties += check_pca_trace(Xq, bq, np_(tq.dir)[h], np_(tq.perm)[h])
        if L > bk:
            ties += check_pca_trace(Xk, bk, np_(tk.dir)[h], np_(tk.perm)[h])
        _check_clusters(Xq, bq, np_(r.q.labels)[h], np_(r.q.perm)[h], np_(r.q.seg)[h], int(np_(r.q.ncl)[h]),
                        np_(r.q.cent)[h])
        _check_clusters(Xk, bk, np_(r.k.labels)[h], np_(r.k.perm)[h], np_(r.k.seg)[h], int(np_(r.k.ncl)[h]),
                        np_(r.k.cent)[h])
        qn = np.linalg.norm(nm.bf16_to_f64(Q.reshape(r.BH, L, d)[h]), axis=1)
        rho, qperm, qseg = np_(r.q.rho)[h], np_(r.q.perm)[h], np_(r.q.seg)[h]
        for c in range(int(np_(r.q.ncl)[h])):
            ref = qn[qperm[qseg[c]:qseg[c + 1]]].mean()
            assert abs(rho[c] - ref) <= 1e-5 * max(ref, 1.0)
        nk = int(np_(r.k.ncl)[h])
        st = ost.key_stats(K.reshape(r.BH, L, d)[h], V.reshape(r.BH, L, d)[h], np_(r.k.labels)[h],
                           np_(r.k.cent)[h, :nk].astype(np.float64))
        assert np.array_equal(bf16_dev_to_f64(r.st.kmax)[h, :nk], st["kmax"])
        assert np.array_equal(bf16_dev_to_f64(r.st.kmin)[h, :nk], st["kmin"])
        assert np.max(np.abs(np_(r.st.kmean)[h, :nk] - st["kmean"])) <= 1e-5 * max(1.0, np.max(np.abs(st["kmean"])))
        assert abs(np_(r.st.mse)[h] - st["mse"]) <= 1e-4 * st["mse"]
    assert np.all(np_(r.st.fallback) == 0)
    # the clusters drive scoring, selection and attention like Algorithm 1's
    r.score_select()
    r.attn()
    import torch
    torch.cuda.synchronize()
    check_scores_selection(r, p)
    check_attention_sampled(r, Q, K, V, p, rows_seed=3, nrows=min(L, 1024))
    print(f"\nL={L} d={d} bq={bq} bk={bk}: split near ties {ties}")


def test_pca_split_exact_on_an_axis_line():
    """Rows t e_0 + 1 with distinct integers 0 <= t < 256 (exact in bf16):
    the direction is e_0 at every node, so the GPU's clusters equal the
    oracle's exactly: runs of consecutive t."""
    L, d, b = 256, 64, 16
    r_ = np.random.default_rng(9)
    t = r_.permutation(L).astype(np.float64)
    X = np.ones((L, d))
    X[:, 0] = t
    bits = nm.bf16_round(X)[None, None]
    p = oracle_params(nq=L // b, m0=32, nmax=max(64, L // b + 1))
    r, _, tk = _run_pca(bits, bits, bits, p, b, b)
    ref = ops.pca_split(nm.bf16_to_f64(bits[0, 0]), b, 512)
    assert np.array_equal(np_(r.k.perm)[0], ref["perm"])
    assert np.array_equal(np_(r.k.labels)[0], ref["labels"])
    assert np.allclose(np_(tk.dir)[0][:, 0], 1.0) and np.allclose(np_(tk.dir)[0][:, 1:], 0.0)


@pytest.mark.parametrize("name", ["wan", "cogvideox"])
def test_pca_split_full_length(name):
    """Two heads at the workload's real L: every split of both sides, the
    exact cluster shape, then scores, selection and sampled attention rows
    against the oracle given the GPU's PCA clusters."""
    w = gen.get_workload(name, H=2)
    Q, K, V = gen.generate(w)
    bq, bk = 256, 64
    L, d = w.L, w.d
    p = oracle_params(nq=-(-L // bq), m0=200, nmax=-(-L // bk) + 1, sel_mode=nm.SEL_DENSITY, sel_param=0.15)
    r, tq, tk = _run_pca(Q, K, V, p, bq, bk)
    ties = 0
    for h in range(r.BH):
        Xq = nm.bf16_to_f64(okm.normalize_queries(Q.reshape(r.BH, L, d)[h]))
        Xk = nm.bf16_to_f64(K.reshape(r.BH, L, d)[h])
        ties += check_pca_trace(Xq, bq, np_(tq.dir)[h], np_(tq.perm)[h])
        ties += check_pca_trace(Xk, bk, np_(tk.dir)[h], np_(tk.perm)[h])
        _check_clusters(Xk, bk, np_(r.k.labels)[h], np_(r.k.perm)[h], np_(r.k.seg)[h], int(np_(r.k.ncl)[h]),
                        np_(r.k.cent)[h])
    r.score_select()
    r.attn()
    import torch
    torch.cuda.synchronize()
    check_scores_selection(r, p)
    worst = check_attention_sampled(r, Q, K, V, p, rows_seed=9004, nrows=1024)
    print(f"\n[{name}] PCA split near ties {ties}; attention worst max-abs {worst[0]:.3g} rel-L2 {worst[1]:.3g}")


def test_pca_split_tree_wider_than_one_block_holds():
    """261,144 queries in clusters of 16 (16,322 query clusters, which one
    k-means++ point per cluster allows): the widest level holds more internal
    nodes (8,130) than the one-block tree builder keeps in LDS (4,096), so the
    split tree comes from the sequential builder.  Every split of the query
    side against the oracle, then the exact cluster shape."""
    L, d, bq, bk = 261144, 64, 16, 4096
    counts = []
    cur = [L]
    while cur:
        counts.append(len(cur))
        nxt = []
        for n in cur:
            nl, nr = ops.split_sizes(n, bq)
            nxt += [c for c in (nl, nr) if c > bq]
        cur = nxt
    assert max(counts) > 4096
    w = gen.get_workload("tiny", H=1, L=L, d=d)
    Q, K, V = gen.generate(w)
    p = oracle_params(nq=-(-L // bq), m0=32, nmax=-(-L // bk) + 1, init_sample=1, sel_mode=nm.SEL_DENSITY,
                      sel_param=0.2)
    r, tq, _ = _run_pca(Q, K, V, p, bq, bk)
    Xq = nm.bf16_to_f64(okm.normalize_queries(Q.reshape(r.BH, L, d)[0]))
    ties = check_pca_trace(Xq, bq, np_(tq.dir)[0], np_(tq.perm)[0])
    _check_clusters(Xq, bq, np_(r.q.labels)[0], np_(r.q.perm)[0], np_(r.q.seg)[0], int(np_(r.q.ncl)[0]),
                    np_(r.q.cent)[0])
    print(f"\nL={L} bq={bq}: {len(counts)} levels, widest {max(counts)}; split near ties {ties}")


def test_pca_query_and_key_sides_overlap():
    """The query split and the key split have workspace scratch of their own:
    run on two streams over one workspace, in either order of enqueueing,
    every output equals that of the two calls one after the other, bit for
    bit."""
    import torch
    import clustered_sparse_attention_amd as ac
    w = gen.get_workload("wan", H=2)
    Q, K, V = gen.generate(w)
    bq, bk = 256, 64
    L = w.L
    p = oracle_params(nq=-(-L // bq), m0=200, nmax=-(-L // bk) + 1, sel_mode=nm.SEL_DENSITY, sel_param=0.15)
    r = Run(Q, K, V, p)

    def outputs():
        q, k, st = r.q, r.k, r.st
        return [t.clone() for t in (q.labels, q.perm, q.seg, q.cent, q.ncl, q.rho, k.labels, k.perm, k.seg, k.cent,
                                    k.ncl, st.kmax, st.kmin, st.kmean, st.vmean, st.mse, st.stages)]

    def clear():
        for t in (r.q.labels, r.q.perm, r.q.seg, r.q.ncl, r.k.labels, r.k.perm, r.k.seg, r.k.ncl):
            t.fill_(-7)
        for t in (r.q.cent, r.q.rho, r.k.cent, r.st.kmean, r.st.vmean, r.st.mse):
            t.fill_(-7.0)

    main = torch.cuda.current_stream()
    ac.ac_cluster_q_pca(r.shape, r.cp, r.Q, bq, r.q, r.ws)
    ac.ac_cluster_k_pca(r.shape, r.cp, r.K, r.V, bk, r.k, r.st, r.ws)
    torch.cuda.synchronize()
    ref = outputs()
    side = torch.cuda.Stream()  # default priority
    for query_first in (True, False):
        clear()
        torch.cuda.synchronize()
        side.wait_stream(main)
        calls = [lambda: ac.ac_cluster_q_pca(r.shape, r.cp, r.Q, bq, r.q, r.ws, stream=side.cuda_stream),
                 lambda: ac.ac_cluster_k_pca(r.shape, r.cp, r.K, r.V, bk, r.k, r.st, r.ws)]
        for c in (calls if query_first else calls[::-1]):
            c()
        main.wait_stream(side)
        torch.cuda.synchronize()
        for i, (a_, b_) in enumerate(zip(ref, outputs())):
            assert torch.equal(a_, b_), (query_first, i)


@pytest.mark.parametrize("L,d,bk", [(1793, 128, 512), (4396, 64, 4096), (768, 128, 256)])
def test_key_statistics_at_chunk_boundaries(L, d, bk):
    """The key statistics run in chunks of 256 members, one wave per chunk,
    and combine the chunks of larger clusters in order.  The PCA split makes
    clusters of exactly bk members (the last one L mod bk), so these cases
    hold clusters of 512 (two full chunks), 257 (a full chunk and a single
    member), 4096 (sixteen chunks), 300 and exactly 256 (one full chunk):
    counts, means, max/min and MSE against the oracle on every cluster."""
    from oracle import stats as ost
    w = gen.get_workload("tiny", H=2, L=L, d=d)
    Q, K, V = gen.generate(w)
    p = oracle_params(nq=-(-L // 256), m0=32, nmax=max(64, -(-L // bk) + 1))
    r, _, _ = _run_pca(Q, K, V, p, 256, bk, trace=False)
    sizes = np.diff(np_(r.k.seg), axis=1)
    for h in range(r.BH):
        nk = int(np_(r.k.ncl)[h])
        assert sizes[h, :nk].tolist() == ops.leaf_sizes(L, bk)
        st = ost.key_stats(K.reshape(r.BH, L, d)[h], V.reshape(r.BH, L, d)[h], np_(r.k.labels)[h],
                           np_(r.k.cent)[h, :nk].astype(np.float64))
        assert np.array_equal(bf16_dev_to_f64(r.st.kmax)[h, :nk], st["kmax"])
        assert np.array_equal(bf16_dev_to_f64(r.st.kmin)[h, :nk], st["kmin"])
        scale = max(1.0, float(np.max(np.abs(st["kmean"]))))
        assert np.max(np.abs(np_(r.st.kmean)[h, :nk] - st["kmean"])) <= 1e-5 * scale
        assert np.max(np.abs(np_(r.st.vmean)[h, :nk] - st["vmean"])) <= 1e-5 * max(1.0, float(np.max(np.abs(st["vmean"]))))
        assert abs(np_(r.st.mse)[h] - st["mse"]) <= 1e-4 * st["mse"]
        # clusters beyond the count are zeroed
        assert not np.any(np_(r.st.kmean)[h, nk:]) and not np.any(bf16_dev_to_f64(r.st.kmax)[h, nk:])
