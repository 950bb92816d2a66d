"""Algorithm 1 of AdaCluster (§3.2.2, MultiStageClustering) in fp64, one head.

Test infrastructure only (see the package docstring).

Readings of the printed algorithm (its text is garbled in places):
* The unassigned set starts as all keys (the listing's initial set symbol is
  undefined), and the distance loop runs over the keys still in it, each
  measured to its own centre from the current stage.
* A key leaves the set when its distance is strictly below tau.
* The cap |C| >= N_max is tested at the top of the loop, before a stage, so
  the last stage may overshoot: |C| <= N_max - 1 + m0.  The fallback flag is
  per head, and is set exactly when the cap stops the loop with keys left.
* After the loop every key is assigned to its nearest centre over all of C;
  centres are not recomputed after this reassignment.
* tau is taken per head from the stage-0 distances (Euclidean, not
  squared): MEAN_X tau = param * mean (AdaCluster §4.1 uses 1.5x the mean
  token-to-centre distance); PCTL nearest-rank: the ceil(param*n)-th
  smallest; ABS tau = param; INF tau = +inf (one stage).
* m_t: every stage uses the same moderate count, m_t = min(|U_t|, m0).  The
  loop always ends: each stage adds at least one centre, so the cap is
  reached unless U empties first.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import TAU_MEAN_X, TAU_PCTL, TAU_ABS, TAU_INF, bf16_to_f64, stream_id
from .kmeans import kmeans, assign


def stage_tau(d: np.ndarray, rule: int, param: float) -> float:
    if rule == TAU_MEAN_X:
        return float(param * np.mean(d))
    if rule == TAU_PCTL:
        n = d.shape[0]
        r = min(max(int(math.ceil(param * n)), 1), n)
        return float(np.sort(d)[r - 1])
    if rule == TAU_ABS:
        return float(param)
    if rule == TAU_INF:
        return math.inf
    raise ValueError(rule)


def next_m(nU: int, m0: int) -> int:
    """Cluster count of a stage: the moderate count m0, or every remaining key."""
    return min(m0, nU)


def cluster_keys(Kbits: np.ndarray, p, bh: int, trace: bool = False):
    """Run Algorithm 1 on one head's keys (bf16 bits [L, d]).

    Returns a dict: cent [N_k, d] fp64, labels [L], nk, fallback (bool),
    tau, stages, and with trace a list of per-stage records
    (U indices, m_t, stage centres, stage labels, distances, removed mask).
    """
    K = bf16_to_f64(Kbits)
    L = K.shape[0]
    U = np.arange(L, dtype=np.int64)
    C = np.zeros((0, K.shape[1]))
    t = 0
    F = False
    tau = math.nan
    log = []
    while U.size > 0:
        if C.shape[0] >= p.nmax:
            F = True
            break
        m = next_m(U.size, p.m0)
        Ct, lab = kmeans(K[U], m, p.seed, stream_id(bh, 1, t), p.iters, p.init_sample)
        diff = K[U] - Ct[lab]
        dist = np.sqrt(np.sum(diff * diff, axis=1))
        if t == 0:
            tau = stage_tau(dist, p.tau_rule, p.tau_param)
        removed = dist < tau
        if trace:
            log.append(dict(U=U.copy(), m=m, cent=Ct.copy(), labels=lab.copy(), dist=dist.copy(),
                            removed=removed.copy()))
        U = U[~removed]
        C = np.concatenate([C, Ct], axis=0)
        t += 1
    labels = assign(K, C)
    out = dict(cent=C, labels=labels, nk=C.shape[0], fallback=F, tau=tau, stages=t)
    if trace:
        out["trace"] = log
    return out


def warm_keys(Kbits: np.ndarray, p, cent_prev: np.ndarray):
    """Later denoising step (AdaCluster §3.2.2, "Efficient initialization"):
    the number of centres is kept, and the previous centres seed
    p.iters_warm Lloyd iterations over all keys; then a final assignment."""
    from .kmeans import lloyd
    K = bf16_to_f64(Kbits)
    C, lab = lloyd(K, np.asarray(cent_prev, dtype=np.float64), p.iters_warm)
    return dict(cent=C, labels=lab, nk=C.shape[0])
