"""The whole layer (AdaCluster Algorithm 3, with ClusterAttention's optional
compensation), cold and warm, one head at a time, in fp64.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .numerics import SEL_DENSE, bf16_to_f64
from .kmeans import cluster_queries
from .multistage import cluster_keys, warm_keys
from .stats import key_stats, counting_sort
from .score import scores, select
from .attention import dense_rows, sparse_rows
from . import tailmerge


def run_head(Qb, Kb, Vb, p, bh: int, rows=None, warm=None):
    """One head of the layer.

    Qb, Kb, Vb: bf16 bits [L, d].  rows: query rows whose output is computed
    (all rows when None).  warm: the state of the previous denoising step
    (dict with cent_q, cent_k, fallback, tau) or None for a cold step.

    Steps: queries KMeans(Normalize(Q)); keys MultiStageClustering (cold) or
    warm Lloyd from the previous centres; key statistics; scores; selection;
    attention (dense when the head fell back, or when sel_mode is DENSE).
    """
    L, d = Qb.shape
    if rows is None:
        rows = np.arange(L)
    qc = cluster_queries(Qb, p, bh, None if warm is None else warm["cent_q"])
    if warm is None:
        kc = cluster_keys(Kb, p, bh)
    else:
        kc = warm_keys(Kb, p, warm["cent_k"])
        kc["fallback"] = warm["fallback"]
        kc["tau"] = warm["tau"]
        kc["stages"] = 0
    kst = key_stats(Kb, Vb, kc["labels"], kc["cent"])
    kperm, kseg = counting_sort(kc["labels"], kc["nk"])
    S = scores(p, qc["cent"], kst)
    sel = select(S, kst["count"], qc["rho"], L, d, p)
    Q, K, V = bf16_to_f64(Qb), bf16_to_f64(Kb), bf16_to_f64(Vb)
    scale = p.attn_scale(d)
    dense = bool(kc["fallback"]) or p.sel_mode == SEL_DENSE
    merged = None
    q_labels = qc["labels"]
    if p.tail_block > 0 and not dense:
        merged = merge_queries(q_labels, len(sel), sel, kst["count"].shape[0], p.tail_block)
        q_labels, sel = merged["labels"], merged["sel"]
    if dense:
        O, lse = dense_rows(Q, K, V, rows, scale)
    else:
        O, lse = sparse_rows(Q, K, V, rows, q_labels, kc["labels"], sel, scale,
                             bool(p.compensate), kst["count"], kst["kmean"], kst["vmean"])
    return dict(q=qc, k=kc, kstats=kst, kperm=kperm, kseg=kseg, S=S, sel=sel, O=O, lse=lse,
                rows=rows, dense=dense, merged=merged,
                state=dict(cent_q=qc["cent"], cent_k=kc["cent"], fallback=kc["fallback"], tau=kc["tau"]))


def run_layer(Q, K, V, p, rows=None, warm=None):
    """All heads of a [B, H, L, d] layer.  Returns a list of per-head dicts
    (see ``run_head``).  ``warm`` is a list of per-head states or None."""
    B, H, L, d = Q.shape
    out = []
    for bh in range(B * H):
        b, h = divmod(bh, H)
        out.append(run_head(Q[b, h], K[b, h], V[b, h], p, bh, rows,
                            None if warm is None else warm[bh]))
    return out


def merge_queries(q_labels, nq, sel, nk, b):
    """Tail merging (iCATS, tail-merging design) of one head's query
    clusters: returns the merged clusters' token order (perm, seg), each
    token's new cluster and the new selections."""
    perm, seg = counting_sort(q_labels, nq)
    sizes = np.diff(seg)
    masks = np.zeros((nq, nk), dtype=bool)
    for r in range(nq):
        masks[r, np.asarray(sel[r], dtype=np.int64)] = True
    pieces, new_masks, new_lists, new_sizes = tailmerge.tail_merge(sizes, masks, sel, b)
    new_perm, new_seg = tailmerge.apply(perm, seg, pieces)
    labels = np.empty_like(q_labels)
    for c in range(nq):
        labels[new_perm[new_seg[c]:new_seg[c + 1]]] = c
    return dict(perm=new_perm, seg=new_seg, labels=labels, sel=new_lists, masks=new_masks, sizes=new_sizes,
                blocks_before=tailmerge.blocks(sizes, b), blocks_after=tailmerge.blocks(new_sizes, b))
