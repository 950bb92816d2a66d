"""Pins of the oracle's multi-step policy (CPU only): the SNR-guided top-p
schedule against the closed forms the sigmoid fixes, the pivot on sequences
whose flattest step is known, the k_max calibration on hand-counted cases,
and the per-(step, layer) parameters."""
import math

import numpy as np
import pytest

from oracle import driver as odr
from oracle import numerics as nm


def _ell(T=50, shift=5.0):
    # a flow-matching sampler's log SNR, log((1 - s)^2 / s^2), over shifted sigmas
    t = np.linspace(1.0, 0.0, T + 1)[:-1]
    s = shift * t / (1.0 + (shift - 1.0) * t)
    s = np.clip(s, 1e-4, 1 - 1e-4)
    return np.log(((1.0 - s) / s) ** 2)


def test_schedule_closed_forms():
    ell = _ell()
    p_min, tau, warm = 0.7, 0.999, 10
    piv = odr.pivot_step(ell, warm)
    p = odr.topp_schedule(ell, warm, p_min, tau)
    assert np.all(p[:warm] == 1.0)
    # sigmoid(0) = 1/2 at the pivot; sigmoid(k x_last) = tau at the last step
    assert abs(p[piv] - (p_min + (1 - p_min) / 2)) < 1e-12
    assert abs(p[-1] - (p_min + (1 - p_min) * (1 - tau))) < 1e-12
    # log SNR grows along the sampler, so p never grows after warm-up
    assert np.all(np.diff(p[warm:]) <= 1e-15)
    # 1 - sigmoid(z) + 1 - sigmoid(-z) = 1: p(x) + p(-x) = 1 + p_min
    k = math.log(tau / (1 - tau)) / (ell[-1] - ell[piv])
    for t in range(warm, len(ell)):
        x = ell[t] - ell[piv]
        mirror = p_min + (1 - p_min) * (1 - 1 / (1 + math.exp(k * x)))
        assert abs(p[t] + mirror - (1 + p_min)) < 1e-12
    assert np.all((p >= p_min) & (p <= 1.0))


def test_pivot_is_the_flattest_step():
    t = np.arange(30, dtype=np.float64)
    assert odr.pivot_step((t - 12.0) ** 3, 0) in (11, 12)
    ell = np.array([0.0, 5.0, 6.0, 6.5, 6.6, 8.0, 12.0])
    assert odr.pivot_step(ell, 0) == 3
    assert odr.pivot_step(ell, 5) == 5
    p = odr.topp_schedule(ell, 0, 0.6, 0.97, t_pivot=2)
    assert abs(p[2] - 0.8) < 1e-12
    with pytest.raises(ValueError):
        odr.topp_schedule(ell[::-1], 0, 0.6, 0.97)


def test_kmax_calibration_counts():
    ncl = [800, 1200, 950, 800, 1700, 600, 1000, 1100, 1300, 700]
    assert odr.kmax_calibrate(ncl, 0.15) == 1300   # ceil(1.5) = 2 units: 1700, 1300
    assert odr.kmax_calibrate(ncl, 0.10) == 1700
    assert odr.kmax_calibrate(ncl, 0.0) == 0
    assert odr.kmax_calibrate(ncl, 1.0) == 600
    # 40 heads, 15%: the 6th largest count
    rng = np.random.default_rng(3)
    n = rng.permutation(np.arange(500, 540))
    assert odr.kmax_calibrate(n, 0.15) == 534
    assert sum(int(v) >= 534 for v in n) == 6


def test_step_params():
    base = nm.Params(sel_mode=nm.SEL_DENSITY, sel_param=0.15, nmax=1500)
    topp = np.linspace(1.0, 0.7, 8)
    p = odr.step_params(base, 1, 3, warmup_steps=2, warmup_layers=1)
    assert p.sel_mode == nm.SEL_DENSE
    p = odr.step_params(base, 5, 0, warmup_steps=2, warmup_layers=1)
    assert p.sel_mode == nm.SEL_DENSE
    p = odr.step_params(base, 5, 2, warmup_steps=2, warmup_layers=1, nmax=900)
    assert (p.sel_mode, p.sel_param, p.nmax) == (nm.SEL_DENSITY, 0.15, 900)
    p = odr.step_params(base, 5, 2, warmup_steps=2, warmup_layers=1, topp=topp)
    assert p.sel_mode == nm.SEL_TOPP and p.sel_param == float(np.float32(topp[5])) and p.nmax == 1500
    assert base.sel_mode == nm.SEL_DENSITY  # the base is not modified
