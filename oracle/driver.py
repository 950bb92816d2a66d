"""Multi-step, multi-layer policy of the sparse layer: which (denoising step,
layer) runs dense attention, the cap N_max (k_max) calibrated so that a
chosen fraction of the attention units falls back, and the SNR-guided
per-step top-p.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows:

* AdaCluster, §3.2.2 "Efficient initialization": the multi-stage clustering
  runs at the first (sparse) denoising step only; later steps keep the
  cluster counts and start from the previous step's centres (the warm step
  of ``layer.run_head``).
* AdaCluster, §4.1 "Platform and configurations": k_max is set so that the
  top 15% of layers (the least compact ones) use full attention.
* iCATS, method section, SNR-guided sparsity: top-p_t = p_min + (1 - p_min)
  (1 - sigmoid(k x_t)) with x_t = l_t - l_pivot, l_t = log SNR(t), a
  steepness k fixed by a saturation parameter tau; and its warm-up setting:
  the first denoising steps and the first layers stay dense.

Readings (the pages leave these open):

* An attention unit is one (layer, head) pair: the fallback flag of
  Algorithm 1 is per head here.  k_max is the cluster count of the unit
  ranked ceil(frac * units) by its uncapped count (largest first): the
  units at or above it are the target; Algorithm 1 then decides, with
  N_max = k_max, which of them fall back (a unit falls back only when a
  stage would start with N_max centres or more and keys are left, so the
  realised fraction can be lower).
* The pivot step is the sparse step where log SNR changes least (the
  smallest forward difference), unless given.
* tau fixes k through the last step: sigmoid(k x_last) = tau, i.e.
  k = logit(tau) / (l_last - l_pivot), so p falls from about 1 at the first
  sparse steps to p_min + (1 - p_min)(1 - tau) at the last.
* Warm-up steps get p = 1 and run dense attention; the schedule covers the
  remaining steps (t_sparse is the last step).
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import SEL_DENSE, SEL_TOPP


def pivot_step(log_snr, warmup_steps: int) -> int:
    """The sparse step at which log SNR is flattest (smallest forward
    difference; the last step counts with its backward difference)."""
    ell = np.asarray(log_snr, dtype=np.float64)
    T = ell.size
    best, best_d = warmup_steps, math.inf
    for t in range(warmup_steps, T):
        d = abs(ell[t + 1] - ell[t]) if t + 1 < T else abs(ell[t] - ell[t - 1])
        if d < best_d:
            best, best_d = t, d
    return best


def topp_schedule(log_snr, warmup_steps: int, p_min: float, tau: float, t_pivot: int = -1):
    """Per-step top-p of the SNR-guided schedule (1 for warm-up steps)."""
    ell = np.asarray(log_snr, dtype=np.float64)
    T = ell.size
    if t_pivot < 0:
        t_pivot = pivot_step(ell, warmup_steps)
    span = ell[T - 1] - ell[t_pivot]
    if not span > 0:
        raise ValueError("log SNR must grow from the pivot to the last step")
    k = math.log(tau / (1.0 - tau)) / span
    out = np.ones(T)
    for t in range(warmup_steps, T):
        x = ell[t] - ell[t_pivot]
        out[t] = p_min + (1.0 - p_min) * (1.0 - 1.0 / (1.0 + math.exp(-k * x)))
    return out


def kmax_calibrate(ncl, frac: float) -> int:
    """k_max: the uncapped cluster count of the unit ranked ceil(frac * units)
    from the top (0 when no unit is to fall back)."""
    n = np.sort(np.asarray(ncl, dtype=np.int64))[::-1]
    nd = int(math.ceil(frac * n.size - 1e-9))
    if nd <= 0:
        return 0
    return int(n[min(nd, n.size) - 1])


def step_params(base, step: int, layer: int, warmup_steps: int, warmup_layers: int, nmax: int = 0, topp=None):
    """Parameters of one (step, layer): dense attention during warm-up,
    the calibrated cap, and the step's top-p when a schedule is given."""
    import dataclasses
    p = dataclasses.replace(base)
    if step < warmup_steps or layer < warmup_layers:
        p.sel_mode = SEL_DENSE
        return p
    if nmax > 0:
        p.nmax = nmax
    if topp is not None:
        p.sel_mode = SEL_TOPP
        p.sel_param = float(np.float32(topp[step]))
    return p
