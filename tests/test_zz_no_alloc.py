"""ac_score_select_noalloc: the scoring and selection with the library's fixed
scratch array instead of a workspace gives the same scores and selections as
ac_score_select, on two calls in a row (the second on a smaller layer, so the
array holds the first call's leftovers), with and without a caller score
buffer."""
import numpy as np
import pytest
import torch

import csa_inputs as gen
from oracle import numerics as nm
from abi_helpers import Run, oracle_params

pytestmark = pytest.mark.gpu


def _layer(H, L, d, mode, **kw):
    w = gen.get_workload("tiny", H=H, L=L, d=d)
    Q, K, V = gen.generate(w)
    p = oracle_params(nq=16, m0=32, nmax=64, tau_rule=nm.TAU_MEAN_X, tau_param=1.5, sel_mode=mode, topk=8,
                      sel_param=0.9 if mode == nm.SEL_TOPP else 0.2, init_sample=8, iters=10, seed=7, **kw)
    r = Run(Q, K, V, p)
    r.cluster_q()
    r.cluster_k()
    r.score_select()          # the workspace entry point
    torch.cuda.synchronize()
    return r


def _noalloc(r, with_score):
    import clustered_sparse_attention_amd as ac
    sel = ac.Selection(r.BH, r.nq, r.ncap_k, torch.device("cuda"), score=with_score)
    # leftovers of earlier calls must not show: fill the outputs with junk first
    sel.list.fill_(-7)
    sel.n.fill_(-7)
    sel.mask.fill_(-1)
    if with_score:
        sel.score.fill_(float("nan"))
    ac.ac_score_select_noalloc(r.shape, r.cp, r.q, r.k, r.st, sel)
    torch.cuda.synchronize()
    return sel


def _same(r, sel):
    n = r.sel.n
    assert torch.equal(sel.n, n)
    assert torch.equal(sel.mask, r.sel.mask)
    nn = n.cpu().numpy()
    lg, lr = sel.list.cpu().numpy(), r.sel.list.cpu().numpy()
    for h in range(r.BH):
        for q in range(r.nq):
            assert np.array_equal(lg[h, q, :nn[h, q]], lr[h, q, :nn[h, q]]), (h, q)
    if sel.score is not None:
        assert torch.equal(sel.score, r.sel.score)


@pytest.mark.parametrize("mode", [nm.SEL_TOPK, nm.SEL_DENSITY, nm.SEL_TOPP])
def test_noalloc_matches_workspace_entry_point_twice(mode):
    big = _layer(3, 4096, 128, mode, compensate=0)
    _same(big, _noalloc(big, with_score=True))
    _same(big, _noalloc(big, with_score=False))
    small = _layer(1, 700, 64, mode, score_mode=nm.SCORE_MEAN)
    _same(small, _noalloc(small, with_score=False))
    _same(small, _noalloc(small, with_score=True))


def test_noalloc_rejects_shapes_beyond_its_scratch():
    import clustered_sparse_attention_amd as ac
    r = _layer(1, 512, 64, nm.SEL_TOPK)
    big_shape = ac.Shape(1, 64, 75600, 128)
    cp = ac.params_default()
    ncap, _ = ac.ac_sizes(big_shape, cp)
    # argument checks need matching capacities; the scratch check comes before any device work
    q = ac.Clusters(1, 1, min(cp.nq, 75600), 128, torch.device("cuda"), rho=True)
    k = ac.Clusters(1, 1, ncap, 128, torch.device("cuda"), rho=False)
    st = ac.KStats(1, 1, 128, torch.device("cuda"))
    sel = ac.Selection(1, 1, ncap, torch.device("cuda"), score=False)
    with pytest.raises(ac.ACError) as e:
        ac.ac_score_select_noalloc(big_shape, cp, q, k, st, sel)
    assert e.value.status == ac.AC_E_UNSUPPORTED and "scratch" in str(e.value)
    # the array still works afterwards
    _same(r, _noalloc(r, with_score=True))
