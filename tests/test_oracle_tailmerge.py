"""Pins of the oracle's tail merging (iCATS method, tail-merging design and
its worked example): the page's numbers, conservation and superset
invariants, and brute force of the pass-2 pairing on small random cases."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import tailmerge as tm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _example():
    """400 query clusters over 1000 key clusters, built around the page's
    worked example: every other cluster is a whole number of blocks, so only
    the clusters of the example have tails."""
    g = json.load(open(os.path.join(GOLDEN, "tail_merge_example.json")))
    b, nq, nk = g["block"], g["nq"], g["nk"]
    rng = np.random.default_rng(7)
    masks = rng.random((nq, nk)) < 0.15
    sizes = np.full(nq, b, dtype=np.int64)
    e, t = g["exact_merge"], g["tail_remap"]
    a1, a2 = e["clusters"]
    masks[a2] = masks[a1]
    sizes[a1], sizes[a2] = e["sizes"]
    r, d = t["receiver"], t["donor"]
    sizes[r], sizes[d] = t["sizes"]
    masks[d] = masks[r].copy()
    masks[d][:3] = ~masks[r][:3]  # Hamming distance 3: far closer than any random pair
    lists = [np.flatnonzero(m) for m in masks]
    return g, b, sizes, masks, lists


def test_page_worked_example():
    g, b, sizes, masks, lists = _example()
    e, t = g["exact_merge"], g["tail_remap"]
    pieces, nm_, nl, ns = tm.tail_merge(sizes, masks, lists, b)
    a1, a2 = e["clusters"]
    assert ns[a1] == e["merged_size"] and ns[a2] == 0
    assert pieces[a1] == [(a1, 0, e["sizes"][0]), (a2, 0, e["sizes"][1])]
    r, d = t["receiver"], t["donor"]
    assert [sizes[r] % b, sizes[d] % b] == t["tails"] and sum(t["tails"]) == t["tail_sum"] <= b
    assert ns[r] == sizes[r] + t["moved"] and ns[d] == sizes[d] - t["moved"] and ns[d] % b == 0
    assert pieces[r] == [(r, 0, int(sizes[r])), (d, int(sizes[d]) - t["moved"], t["moved"])]
    assert np.array_equal(nm_[r], masks[r] | masks[d]) and np.array_equal(nm_[d], masks[d])
    # the receiver's list: its own, then the donor's extra clusters in the donor's order
    extra = [c for c in lists[d] if not masks[r][c]]
    assert list(nl[r]) == list(lists[r]) + extra
    assert tm.blocks(ns, b) < tm.blocks(sizes, b)


def _random_case(rng, nq, nk, b):
    sizes = rng.integers(0, 3 * b, size=nq)
    base = rng.random((4, nk)) < 0.3
    masks = base[rng.integers(0, 4, size=nq)].copy()
    flip = rng.random((nq, nk)) < 0.05
    masks ^= flip & (rng.random(nq) < 0.7)[:, None]
    lists = [rng.permutation(np.flatnonzero(m)) for m in masks]
    return sizes, masks, lists


@pytest.mark.parametrize("seed", range(20))
def test_conservation_and_supersets(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.choice([8, 16, 128]))
    nq, nk = int(rng.integers(2, 40)), int(rng.integers(1, 70))
    sizes, masks, lists = _random_case(rng, nq, nk, b)
    seg = np.concatenate([[0], np.cumsum(sizes)])
    perm = rng.permutation(int(seg[-1]))
    pieces, nm_, nl, ns = tm.tail_merge(sizes, masks, lists, b)
    newp, newseg = tm.apply(perm, seg, pieces)
    # a permutation of the same tokens, sizes consistent
    assert np.array_equal(np.sort(newp), np.sort(perm))
    assert np.array_equal(np.diff(newseg), ns)
    # every token keeps at least its key clusters, and lists match masks
    old_of = np.empty(int(seg[-1]), dtype=np.int64)
    for r in range(nq):
        old_of[perm[seg[r]:seg[r + 1]]] = r
    for c in range(nq):
        for tok in newp[newseg[c]:newseg[c + 1]]:
            assert np.all(nm_[c] >= masks[old_of[tok]])
        if ns[c] > 0:
            assert sorted(nl[c]) == list(np.flatnonzero(nm_[c]))
    # never more blocks
    assert tm.blocks(ns, b) <= tm.blocks(sizes, b)


@pytest.mark.parametrize("seed", range(20))
def test_pairing_by_brute_force(seed):
    """Pass 2 against an independent search: over the clusters with tails
    after pass 1, mutual nearest neighbours by a full Hamming matrix."""
    rng = np.random.default_rng(100 + seed)
    b = 16
    nq, nk = int(rng.integers(2, 24)), int(rng.integers(1, 40))
    sizes, masks, lists = _random_case(rng, nq, nk, b)
    pieces, nm_, nl, ns = tm.tail_merge(sizes, masks, lists, b)
    # pass 1 by itself: groups of identical masks among non-empty clusters
    s1 = sizes.copy()
    for r in range(nq):
        if s1[r] == 0:
            continue
        same = [q for q in range(r) if s1[q] > 0 and (masks[q] == masks[r]).all()]
        if same:
            s1[same[0]] += s1[r]
            s1[r] = 0
    cand = [r for r in range(nq) if s1[r] > 0 and s1[r] % b > 0]
    H = np.array([[np.sum(masks[i] != masks[j]) if i != j else 10 ** 9 for j in cand] for i in cand]).reshape(
        len(cand), len(cand))
    nn = {cand[i]: cand[int(np.argmin(H[i]))] for i in range(len(cand))} if len(cand) > 1 else {}
    expect = s1.copy()
    for i, j in itertools.combinations(cand, 2):
        if nn.get(i) == j and nn.get(j) == i and s1[i] % b + s1[j] % b <= b:
            ti, tj = s1[i] % b, s1[j] % b
            donor, recv = (i, j) if (ti < tj or (ti == tj and i > j)) else (j, i)
            t = s1[donor] % b
            expect[donor] -= t
            expect[recv] += t
    assert np.array_equal(ns, expect)
