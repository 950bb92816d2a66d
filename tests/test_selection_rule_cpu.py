"""The near-tie rule the GPU selection tests apply (CPU only): a GPU selection
that differs from the oracle's passes only when the cut lies at a near tie,
for top-p when the cumulative mass at the cut is within 1e-5 of p."""
import math

import numpy as np

from oracle import numerics as nm
from oracle import score as osc
from abi_helpers import selection_difference_is_near_tie


def _row(seed, nk=30):
    r = np.random.default_rng(seed)
    S = r.standard_normal(nk).astype(np.float32).astype(np.float64)
    cnt = r.integers(1, 60, nk)
    return S, cnt


def test_topp_wrong_cut_is_rejected():
    S, cnt = _row(1)
    p = nm.Params(sel_mode=nm.SEL_TOPP, sel_param=0.9)
    o = osc.select_row(S, cnt, 1.7, int(cnt.sum()), 64, p).tolist()
    order = osc.order_clusters(S, cnt).tolist()
    amax = float(np.max(np.abs(S)))
    for g in (o[:-1], order[:len(o) + 1], list(reversed(o))):
        assert not selection_difference_is_near_tie(S, cnt, 1.7, int(cnt.sum()), 64, p, g, o, amax)
    # another temperature (rho dropped) gives another cut, which the rule rejects
    g = osc.select_row(S, cnt, 1.0, int(cnt.sum()), 64, p).tolist()
    if g != o:
        assert not selection_difference_is_near_tie(S, cnt, 1.7, int(cnt.sum()), 64, p, g, o, amax)


def test_topp_cut_at_the_mass_boundary_is_a_near_tie():
    S, cnt = _row(2)
    L = int(cnt.sum())
    order = osc.order_clusters(S, cnt)
    z = 1.3 * S[order] / 8.0 + np.log(cnt[order].astype(np.float64))
    w = np.exp(z - z.max())
    cum = np.cumsum(w / w.sum())
    k = 7
    pv = float(cum[k - 1]) + 3e-6      # p just above the mass of the first k clusters
    p = nm.Params(sel_mode=nm.SEL_TOPP, sel_param=pv)
    o = osc.select_row(S, cnt, 1.3, L, 64, p).tolist()
    assert len(o) == k + 1
    assert selection_difference_is_near_tie(S, cnt, 1.3, L, 64, p, order[:k].tolist(), o, 1.0)
    assert not selection_difference_is_near_tie(S, cnt, 1.3, L, 64, p, order[:k - 1].tolist(), o, 1.0)


def test_topk_and_density_rule_uses_scores():
    S, cnt = _row(3)
    S[5] = S[6] = 0.25                 # an exact score tie
    p = nm.Params(sel_mode=nm.SEL_TOPK, topk=4)
    o = osc.select_row(S, cnt, 1.0, 100, 64, p).tolist()
    swapped = [c for c in o]
    if 5 in o and 6 not in o:
        swapped[o.index(5)] = 6
        assert selection_difference_is_near_tie(S, cnt, 1.0, 100, 64, p, swapped, o, float(np.max(np.abs(S))))
    far = osc.order_clusters(S, cnt)[-1]
    g = o[:-1] + [int(far)]
    assert not selection_difference_is_near_tie(S, cnt, 1.0, 100, 64, p, g, o, float(np.max(np.abs(S))))
    assert math.isfinite(float(np.max(np.abs(S))))
