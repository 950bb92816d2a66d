"""Tail merging of query clusters before block-sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "iCATS: Fast Video Generation via Interaction-Aware Sparse Attention
and Timestep-Adaptive Sparsity" (arXiv 2610.11302), method section, key
design 3 (tail merging) and its worked example: an attention kernel that
processes queries in blocks of b rows pays a whole block for the last,
partial block ("tail") of every query cluster, and pays it again for every
key block that cluster selects.  Two passes, per head:

1. Exact merge: query clusters whose key-cluster masks are identical are
   merged (token lists concatenated, sizes added); no selection changes.
2. Compatible tail remap: among the clusters that still have a tail
   tau = size mod b > 0, a pair that are each other's nearest neighbour in
   Hamming distance between masks, and whose tails add up to at most b,
   moves one cluster's tail tokens to the other, which then selects the
   union (bitwise OR) of both masks.

Readings (the page leaves these open):

* Empty clusters take part in neither pass.
* Pass 1 merges every cluster of an identical-mask group into the one with
  the lowest index, appending token lists in ascending cluster order.
* Pass 2 considers only clusters with a tail after pass 1; the nearest
  neighbour of r is the other such cluster at the smallest Hamming
  distance, ties to the lowest index; each mutual pair is examined once.
  The donor is the cluster with the smaller tail (ties: the higher index);
  its last tau tokens (in its token order) are appended to the receiver.
  Only the receiver's mask becomes the OR; the donor keeps its own.  The
  worked example (tails 44 and 42; cluster 18 gives 42 tokens to cluster 3)
  matches this.
* The receiver's selection list is its own list followed by the entries of
  the donor's list it did not have, in the donor's order.
* One application of each pass (the page: "two rounds of merging").
"""
from __future__ import annotations

import numpy as np


def tail_merge(sizes, masks, lists, b):
    """Merge query clusters of one head.

    sizes  : [nq] int, tokens per query cluster
    masks  : [nq, nk] bool, selected key clusters per query cluster
    lists  : list of nq int arrays, each cluster's selection in its order
    b      : query block size of the attention kernel

    Returns (pieces, new_masks, new_lists, new_sizes) where pieces[c] is the
    ordered list of (old cluster, start, length) runs of old token positions
    (offsets within the old cluster's token list) that make up new cluster
    c.  Clusters emptied by the merge have no pieces and size 0.
    """
    sizes = np.asarray(sizes, dtype=np.int64)
    masks = np.asarray(masks, dtype=bool)
    nq = sizes.shape[0]
    pieces = [[(r, 0, int(sizes[r]))] if sizes[r] > 0 else [] for r in range(nq)]
    new_masks = masks.copy()
    new_lists = [np.asarray(lst, dtype=np.int64).copy() for lst in lists]
    new_sizes = sizes.copy()

    # pass 1: identical masks
    for r in range(nq):
        if new_sizes[r] == 0:
            continue
        for q in range(r):
            if new_sizes[q] > 0 and np.array_equal(masks[q], masks[r]):
                pieces[q].extend(pieces[r])
                pieces[r] = []
                new_sizes[q] += new_sizes[r]
                new_sizes[r] = 0
                break

    # pass 2: compatible tails
    tails = new_sizes % b
    cand = [r for r in range(nq) if new_sizes[r] > 0 and tails[r] > 0]
    nn = {}
    for r in cand:
        best, best_d = -1, None
        for q in cand:
            if q == r:
                continue
            d = int(np.count_nonzero(new_masks[r] != new_masks[q]))
            if best_d is None or d < best_d:
                best, best_d = q, d
        nn[r] = best
    for r in cand:
        q = nn[r]
        if q < 0 or nn.get(q) != r or q < r:
            continue  # not mutual, or the pair is handled from its lower index
        if tails[r] + tails[q] > b:
            continue
        if tails[r] < tails[q] or (tails[r] == tails[q] and r > q):
            donor, recv = r, q
        else:
            donor, recv = q, r
        t = int(tails[donor])
        # cut the donor's last t tokens off its piece list
        moved, keep, rest = [], [], t
        for (o, st, ln) in reversed(pieces[donor]):
            if rest == 0:
                keep.append((o, st, ln))
            elif ln <= rest:
                moved.append((o, st, ln))
                rest -= ln
            else:
                keep.append((o, st, ln - rest))
                moved.append((o, st + ln - rest, rest))
                rest = 0
        pieces[donor] = list(reversed(keep))
        pieces[recv].extend(reversed(moved))
        new_sizes[donor] -= t
        new_sizes[recv] += t
        extra = [c for c in new_lists[donor] if not new_masks[recv][c]]
        new_masks[recv] = new_masks[recv] | new_masks[donor]
        new_lists[recv] = np.concatenate([new_lists[recv], np.asarray(extra, dtype=np.int64)])
    return pieces, new_masks, new_lists, new_sizes


def blocks(sizes, b):
    """Query blocks of b rows the attention launches for these clusters."""
    sizes = np.asarray(sizes, dtype=np.int64)
    return int(np.sum((sizes + b - 1) // b))


def apply(perm, seg, pieces):
    """New (perm, seg) of one head from the old ones and the pieces."""
    out, segs = [], [0]
    for pl in pieces:
        for (o, st, ln) in pl:
            out.extend(perm[seg[o] + st: seg[o] + st + ln])
        segs.append(len(out))
    return np.asarray(out, dtype=np.int64), np.asarray(segs, dtype=np.int64)
