"""The C-ABI library loads, exports every symbol include/ac.h declares, and
rejects bad arguments before touching any device.  CPU only."""
import ctypes
import os
import re

import pytest

import clustered_sparse_attention_amd as ac

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ac.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ac_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ac.load()
    names = _declared()
    assert set(names) == set(ac.ENTRY_POINTS)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_c_layout():
    assert ctypes.sizeof(ac.Shape) == 16
    assert ctypes.sizeof(ac.Params) == 72
    assert ctypes.sizeof(ac.CClusters) == 56
    assert ctypes.sizeof(ac.CKStats) == 64
    assert ctypes.sizeof(ac.CSelection) == 40
    assert ctypes.sizeof(ac.CState) == 48
    assert ctypes.sizeof(ac.CSchedule) == 24
    assert ctypes.sizeof(ac.CKTrace) == 56
    assert ctypes.sizeof(ac.CPcaTrace) == 16


def test_defaults_and_status_strings():
    p = ac.params_default()
    assert (p.nq, p.iters, p.m0, p.nmax, p.tau_rule, p.sel_mode) == (65, 10, 200, 1500, ac.AC_TAU_MEAN_X,
                                                                    ac.AC_SEL_DENSITY)
    assert abs(p.tau_param - 1.5) < 1e-7 and abs(p.sel_param - 0.15) < 1e-7
    assert (p.tail_block, p.min_sparse_gflop) == (0, 0)
    lib = ac.load()
    assert lib.ac_status_str(ac.AC_E_WORKSPACE) == b"workspace too small"


def test_sizes_validation():
    p = ac.params_default()
    ncap, ws = ac.ac_sizes(ac.Shape(1, 40, 75600, 128), p)
    assert ncap == 1699 and ws > 40 * 75600 * 128 * 2
    for bad_shape, code in [((1, 2, 4096, 96), ac.AC_E_UNSUPPORTED), ((0, 2, 4096, 64), ac.AC_E_SHAPE),
                            ((1, 2, -5, 64), ac.AC_E_SHAPE), ((1, 2, 0, 64), ac.AC_E_SHAPE),
                            ((1, 0, 4096, 64), ac.AC_E_SHAPE), ((2, 32768, 64, 64), ac.AC_E_SHAPE)]:
        with pytest.raises(ac.ACError) as e:
            ac.ac_sizes(ac.Shape(*bad_shape), p)
        assert e.value.status == code
    ac.ac_sizes(ac.Shape(1, 65535, 64, 64), p)  # the most heads a call takes
    for kw in [dict(nq=0), dict(tau_rule=9), dict(sel_mode=7), dict(sel_mode=ac.AC_SEL_DENSITY, sel_param=1.5),
               dict(compensate=2), dict(tau_rule=ac.AC_TAU_PCTL, tau_param=0.0), dict(sel_mode=ac.AC_SEL_TOPK, topk=0),
               dict(min_sparse_gflop=-1)]:
        with pytest.raises(ac.ACError) as e:
            ac.ac_sizes(ac.Shape(1, 2, 4096, 64), ac.params_default(**kw))
        assert e.value.status == ac.AC_E_ARG, kw
    with pytest.raises(ac.ACError) as e:
        ac.ac_sizes(ac.Shape(1, 2, 4096, 64), ac.params_default(nmax=5000))
    assert e.value.status == ac.AC_E_UNSUPPORTED
    with pytest.raises(ac.ACError) as e:
        ac.ac_sizes(ac.Shape(1, 2, 100000, 64), ac.params_default(init_sample=0))
    assert e.value.status == ac.AC_E_UNSUPPORTED
    # one head's rows must be addressable with 32-bit byte offsets
    ac.ac_sizes(ac.Shape(1, 1, (1 << 24) - 1, 128), ac.params_default())
    for L, d in ((1 << 24, 128), (1 << 25, 64)):
        with pytest.raises(ac.ACError) as e:
            ac.ac_sizes(ac.Shape(1, 1, L, d), ac.params_default())
        assert e.value.status == ac.AC_E_UNSUPPORTED and b"4 GiB" in ac.load().ac_last_error()


def _fake_clusters(ncap):
    # aligned non-NULL addresses that are never dereferenced: every call below fails validation first
    a = 1 << 20
    return ac.CClusters(ncap, a, a, a, a, a, a)


def test_entry_points_reject_bad_arguments_before_any_device_work():
    lib = ac.load()
    shape = ac.Shape(1, 2, 4096, 64)
    p = ac.params_default(nq=16, m0=32, nmax=64)
    ncap, wsb = ac.ac_sizes(shape, p)
    q = _fake_clusters(16)
    k = _fake_clusters(ncap)
    ws = 1 << 24
    # NULL Q
    assert lib.ac_cluster_q(ctypes.byref(shape), ctypes.byref(p), None, None, ctypes.byref(q), ws, wsb, None) == ac.AC_E_ARG
    # workspace too small
    assert lib.ac_cluster_q(ctypes.byref(shape), ctypes.byref(p), 1 << 20, None, ctypes.byref(q), ws, wsb - 1,
                            None) == ac.AC_E_WORKSPACE
    # misaligned workspace
    assert lib.ac_cluster_q(ctypes.byref(shape), ctypes.byref(p), 1 << 20, None, ctypes.byref(q), ws + 8, wsb,
                            None) == ac.AC_E_ARG
    # wrong query capacity
    q_bad = _fake_clusters(15)
    assert lib.ac_cluster_q(ctypes.byref(shape), ctypes.byref(p), 1 << 20, None, ctypes.byref(q_bad), ws, wsb,
                            None) == ac.AC_E_ARG
    # key capacity must equal nmax - 1 + m0
    st = ac.CKStats(*([1 << 20] * 8))
    k_bad = _fake_clusters(ncap - 1)
    assert lib.ac_cluster_k(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, None, ctypes.byref(k_bad),
                            ctypes.byref(st), ws, wsb, None) == ac.AC_E_ARG
    # NULL stats array
    st_bad = ac.CKStats(*([1 << 20] * 7 + [0]))
    assert lib.ac_cluster_k(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, None, ctypes.byref(k),
                            ctypes.byref(st_bad), ws, wsb, None) == ac.AC_E_ARG
    # selection capacity mismatch
    sel = ac.CSelection(ncap + 1, 1 << 20, 1 << 20, 1 << 20, 0)
    assert lib.ac_score_select(ctypes.byref(shape), ctypes.byref(p), ctypes.byref(q), ctypes.byref(k),
                               ctypes.byref(st), ctypes.byref(sel), ws, wsb, None) == ac.AC_E_ARG
    assert b"ncap_k" in lib.ac_last_error()
    # NULL O
    sel_ok = ac.CSelection(ncap, 1 << 20, 1 << 20, 1 << 20, 0)
    assert lib.ac_sparse_attn(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, 1 << 20, ctypes.byref(q),
                              ctypes.byref(k), ctypes.byref(st), ctypes.byref(sel_ok), None, None, ws, wsb,
                              None) == ac.AC_E_ARG
    # per-token scores: bad engine, ld < 1, NULL S, key capacity
    for eng, ld, S, kk in [(2, 64, 1 << 20, k), (ac.AC_QUEST_MFMA, 0, 1 << 20, k), (ac.AC_QUEST_VALU, 64, None, k),
                           (ac.AC_QUEST_MFMA, 64, 1 << 20, k_bad)]:
        assert lib.ac_score_tokens(ctypes.byref(shape), ctypes.byref(p), 1 << 20, ctypes.byref(kk), ctypes.byref(st),
                                   eng, S, ld, None) == ac.AC_E_ARG, (eng, ld, S)
    # interaction-aware clustering: NULL M, wrong capacities
    assert lib.ac_interaction_matrix(ctypes.byref(shape), ctypes.byref(p), 1 << 20, ctypes.byref(q), None, ws, wsb,
                                     None) == ac.AC_E_ARG
    assert lib.ac_interaction_matrix(ctypes.byref(shape), ctypes.byref(p), 1 << 20, ctypes.byref(q_bad), 1 << 20, ws,
                                     wsb, None) == ac.AC_E_ARG
    assert lib.ac_cluster_k_metric(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, None, ctypes.byref(k),
                                   ctypes.byref(st), ws, wsb, None) == ac.AC_E_ARG
    assert lib.ac_cluster_k_metric(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, 1 << 20,
                                   ctypes.byref(k_bad), ctypes.byref(st), ws, wsb, None) == ac.AC_E_ARG
    # traced clustering: NULL trace, no stage to record
    assert lib.ac_cluster_k_trace(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, ctypes.byref(k),
                                  ctypes.byref(st), None, ws, wsb, None) == ac.AC_E_ARG
    tr0 = ac.CKTrace(0, 0, 0, 0, 0, 0, 0)
    assert lib.ac_cluster_k_trace(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, ctypes.byref(k),
                                  ctypes.byref(st), ctypes.byref(tr0), ws, wsb, None) == ac.AC_E_ARG
    assert lib.ac_cluster_q_trace(ctypes.byref(shape), ctypes.byref(p), 1 << 20, ctypes.byref(q), None, ws, wsb,
                                  None) == ac.AC_E_ARG
    # principal-component split: block not a power of two, too small, or more clusters than the capacity
    for blk in (48, 8, 8192):
        assert lib.ac_cluster_q_pca(ctypes.byref(shape), ctypes.byref(p), 1 << 20, blk, ctypes.byref(q), None, ws,
                                    wsb, None) == ac.AC_E_ARG, blk
    assert lib.ac_cluster_q_pca(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 128, ctypes.byref(q), None, ws, wsb,
                                None) == ac.AC_E_ARG  # 4096 / 128 = 32 clusters > nq = 16
    assert b"capacity" in lib.ac_last_error()
    assert lib.ac_cluster_k_pca(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, 32, ctypes.byref(k),
                                ctypes.byref(st), None, ws, wsb, None) == ac.AC_E_ARG  # 128 clusters > ncap 95
    # NULL state
    assert lib.ac_layer(ctypes.byref(shape), ctypes.byref(p), 1 << 20, 1 << 20, 1 << 20, None, 1 << 20, None, ws, wsb,
                        None) == ac.AC_E_ARG


def test_valid_arguments_without_device_report_device_error():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the no-device path")
    lib = ac.load()
    shape = ac.Shape(1, 2, 4096, 64)
    p = ac.params_default(nq=16, m0=32, nmax=64)
    ncap, wsb = ac.ac_sizes(shape, p)
    q = _fake_clusters(16)
    assert lib.ac_cluster_q(ctypes.byref(shape), ctypes.byref(p), 1 << 20, None, ctypes.byref(q), 1 << 24, wsb,
                            None) == ac.AC_E_DEVICE
    assert len(lib.ac_last_error()) > 0
