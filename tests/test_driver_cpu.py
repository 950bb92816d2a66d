"""The C policy functions of the multi-step driver (host only, no GPU)
against the oracle's: SNR-guided top-p schedule, k_max calibration and the
per-(step, layer) parameters; and their argument checks."""
import numpy as np
import pytest

import clustered_sparse_attention_amd as ac
from oracle import driver as odr
from oracle import numerics as nm
from test_oracle_driver import _ell


@pytest.mark.parametrize("T,warm,p_min,tau,pivot", [(50, 10, 0.7, 0.999, -1), (50, 10, 0.65, 0.97, -1),
                                                    (30, 5, 0.7, 0.999, 12), (8, 0, 0.5, 0.9, -1)])
def test_topp_schedule_matches_oracle(T, warm, p_min, tau, pivot):
    ell = _ell(T)
    got = ac.ac_topp_schedule(ell, warm, p_min, tau, pivot)
    want = odr.topp_schedule(ell, warm, p_min, tau, pivot).astype(np.float32)
    # both evaluate in binary64 and round once to binary32: at most one binary32 ulp apart
    assert np.all(np.abs(got.view(np.int32) - want.view(np.int32)) <= 1)


def test_topp_schedule_rejects_bad_arguments():
    ell = _ell(20)
    for args in [(ell, 19, 0.7, 0.99), (ell, 0, 0.0, 0.99), (ell, 0, 0.7, 1.0), (ell, 0, 0.7, 0.3),
                 (ell[::-1].copy(), 0, 0.7, 0.99)]:
        with pytest.raises(ac.ACError):
            ac.ac_topp_schedule(*args)
    with pytest.raises(ac.ACError):
        ac.ac_topp_schedule(ell, 5, 0.7, 0.99, t_pivot=2)


def test_kmax_calibration_matches_oracle():
    rng = np.random.default_rng(11)
    for units in (1, 7, 40, 240):
        ncl = rng.integers(200, 1700, size=units)
        for frac in (0.0, 0.05, 0.15, 0.5, 1.0):
            assert ac.ac_kmax_calibrate(ncl, frac) == odr.kmax_calibrate(ncl, frac), (units, frac)
    with pytest.raises(ac.ACError):
        ac.ac_kmax_calibrate([800], 1.5)


def test_step_params_match_oracle():
    base = nm.Params(sel_mode=nm.SEL_DENSITY, sel_param=0.15, nmax=1500)
    cbase = ac.params_default(sel_mode=ac.AC_SEL_DENSITY, sel_param=0.15, nmax=1500)
    topp = odr.topp_schedule(_ell(12), 3, 0.7, 0.999)
    for nmax, sched in ((0, None), (900, None), (0, topp), (1100, topp)):
        s = ac.Schedule(warmup_steps=3, warmup_layers=1, nmax=nmax, topp=sched)
        for step in range(12):
            for layer in range(3):
                got = ac.ac_step_params(cbase, s, step, layer)
                want = odr.step_params(base, step, layer, 3, 1, nmax, None if sched is None else sched)
                assert (got.sel_mode, got.nmax) == (want.sel_mode, want.nmax), (step, layer)
                if want.sel_mode != nm.SEL_DENSE:
                    assert got.sel_param == np.float32(want.sel_param)
    s = ac.Schedule(topp=topp)
    with pytest.raises(ac.ACError):
        ac.ac_step_params(cbase, s, 12, 0)
