"""Python binding of the cluster-routed sparse attention library (libac.so).

Argument marshalling only: every step of the layer runs in the HIP kernels
of ``libac.so``.  PyTorch provides device memory and the stream.  The
functions carry the names of the C entry points declared in
``include/ac.h`` and raise ``ACError`` on a non-OK status.  There is no
fallback path: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libac.so")

# enums (values of include/ac.h)
AC_OK, AC_E_ARG, AC_E_SHAPE, AC_E_WORKSPACE, AC_E_UNSUPPORTED, AC_E_DEVICE = range(6)
AC_TAU_MEAN_X, AC_TAU_PCTL, AC_TAU_ABS, AC_TAU_INF = range(4)
AC_SCORE_QUEST, AC_SCORE_MEAN = range(2)
AC_SEL_TOPK, AC_SEL_DENSITY, AC_SEL_TOPP, AC_SEL_DENSE = range(4)
AC_QUEST_MFMA, AC_QUEST_VALU = range(2)

ENTRY_POINTS = ("ac_params_default", "ac_sizes", "ac_cluster_q", "ac_cluster_k", "ac_cluster_k_trace",
                "ac_cluster_q_trace", "ac_cluster_q_pca", "ac_cluster_k_pca", "ac_score_select",
                "ac_score_select_noalloc",
                "ac_sparse_attn", "ac_tail_merge", "ac_score_tokens", "ac_interaction_matrix",
                "ac_cluster_k_metric", "ac_layer", "ac_topp_schedule",
                "ac_kmax_calibrate", "ac_step_params", "ac_status_str", "ac_last_error")


class ACError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


# ---------------------------------------------------------------- C structs
P = ctypes.c_void_p


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("d", ctypes.c_int32)]


class Params(ctypes.Structure):
    _fields_ = [("nq", ctypes.c_int32), ("iters", ctypes.c_int32), ("iters_warm", ctypes.c_int32),
                ("m0", ctypes.c_int32), ("nmax", ctypes.c_int32), ("tau_rule", ctypes.c_int32),
                ("tau_param", ctypes.c_float), ("score_mode", ctypes.c_int32), ("sel_mode", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("sel_param", ctypes.c_float), ("compensate", ctypes.c_int32),
                ("scale", ctypes.c_float), ("init_sample", ctypes.c_int32), ("tail_block", ctypes.c_int32),
                ("min_sparse_gflop", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class CClusters(ctypes.Structure):
    _fields_ = [("ncap", ctypes.c_int32), ("labels", P), ("perm", P), ("seg", P), ("cent", P), ("ncl", P),
                ("rho", P)]


class CKStats(ctypes.Structure):
    _fields_ = [("kmax", P), ("kmin", P), ("kmean", P), ("vmean", P), ("fallback", P), ("tau", P), ("mse", P),
                ("stages", P)]


class CKTrace(ctypes.Structure):
    _fields_ = [("max_stages", ctypes.c_int32), ("n", P), ("m", P), ("u", P), ("cent", P), ("labels", P),
                ("dist", P)]


class CPcaTrace(ctypes.Structure):
    _fields_ = [("dir", P), ("perm", P)]


class CSelection(ctypes.Structure):
    _fields_ = [("ncap_k", ctypes.c_int32), ("list", P), ("n", P), ("mask", P), ("score", P)]


class CState(ctypes.Structure):
    _fields_ = [("cent_q", P), ("cent_k", P), ("ncl_k", P), ("fallback", P), ("tau", P), ("valid", ctypes.c_int32)]


class CSchedule(ctypes.Structure):
    _fields_ = [("warmup_steps", ctypes.c_int32), ("warmup_layers", ctypes.c_int32), ("nmax", ctypes.c_int32),
                ("steps", ctypes.c_int32), ("topp", P)]


class CLayerStats(ctypes.Structure):
    _fields_ = [("ncl_k", P), ("fallback", P), ("tau", P), ("mse", P), ("stages", P), ("pairs", P)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libac.so (built by ``clustered_sparse_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m clustered_sparse_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    vp = ctypes.c_void_p
    lib.ac_params_default.argtypes = [ctypes.POINTER(Params)]
    lib.ac_params_default.restype = st
    lib.ac_sizes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), ctypes.POINTER(ctypes.c_int32),
                             ctypes.POINTER(ctypes.c_size_t)]
    lib.ac_sizes.restype = st
    lib.ac_cluster_q.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp, ctypes.POINTER(CClusters),
                                 vp, ctypes.c_size_t, vp]
    lib.ac_cluster_q.restype = st
    lib.ac_cluster_k.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp, ctypes.POINTER(CState),
                                 ctypes.POINTER(CClusters), ctypes.POINTER(CKStats), vp, ctypes.c_size_t, vp]
    lib.ac_cluster_k.restype = st
    lib.ac_cluster_k_trace.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp,
                                       ctypes.POINTER(CClusters), ctypes.POINTER(CKStats), ctypes.POINTER(CKTrace),
                                       vp, ctypes.c_size_t, vp]
    lib.ac_cluster_k_trace.restype = st
    lib.ac_cluster_q_trace.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, ctypes.POINTER(CClusters),
                                       vp, vp, ctypes.c_size_t, vp]
    lib.ac_cluster_q_trace.restype = st
    lib.ac_cluster_q_pca.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, ctypes.c_int32,
                                     ctypes.POINTER(CClusters), ctypes.POINTER(CPcaTrace), vp, ctypes.c_size_t, vp]
    lib.ac_cluster_q_pca.restype = st
    lib.ac_cluster_k_pca.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp, ctypes.c_int32,
                                     ctypes.POINTER(CClusters), ctypes.POINTER(CKStats), ctypes.POINTER(CPcaTrace), vp,
                                     ctypes.c_size_t, vp]
    lib.ac_cluster_k_pca.restype = st
    lib.ac_score_select.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), ctypes.POINTER(CClusters),
                                    ctypes.POINTER(CClusters), ctypes.POINTER(CKStats), ctypes.POINTER(CSelection),
                                    vp, ctypes.c_size_t, vp]
    lib.ac_score_select.restype = st
    lib.ac_score_select_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), ctypes.POINTER(CClusters),
                                            ctypes.POINTER(CClusters), ctypes.POINTER(CKStats),
                                            ctypes.POINTER(CSelection), vp]
    lib.ac_score_select_noalloc.restype = st
    lib.ac_sparse_attn.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp, vp,
                                   ctypes.POINTER(CClusters), ctypes.POINTER(CClusters), ctypes.POINTER(CKStats),
                                   ctypes.POINTER(CSelection), vp, vp, vp, ctypes.c_size_t, vp]
    lib.ac_sparse_attn.restype = st
    lib.ac_tail_merge.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), ctypes.c_int32,
                                  ctypes.POINTER(CClusters), ctypes.POINTER(CSelection), ctypes.POINTER(CClusters),
                                  ctypes.POINTER(CSelection), vp, ctypes.c_size_t, vp]
    lib.ac_tail_merge.restype = st
    lib.ac_score_tokens.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, ctypes.POINTER(CClusters),
                                    ctypes.POINTER(CKStats), ctypes.c_int32, vp, ctypes.c_int32, vp]
    lib.ac_score_tokens.restype = st
    lib.ac_layer.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp, vp, ctypes.POINTER(CState), vp,
                             ctypes.POINTER(CLayerStats), vp, ctypes.c_size_t, vp]
    lib.ac_layer.restype = st
    lib.ac_interaction_matrix.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, ctypes.POINTER(CClusters),
                                          vp, vp, ctypes.c_size_t, vp]
    lib.ac_interaction_matrix.restype = st
    lib.ac_cluster_k_metric.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Params), vp, vp, vp,
                                        ctypes.POINTER(CClusters), ctypes.POINTER(CKStats), vp, ctypes.c_size_t, vp]
    lib.ac_cluster_k_metric.restype = st
    lib.ac_topp_schedule.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_int32, vp]
    lib.ac_topp_schedule.restype = st
    lib.ac_kmax_calibrate.argtypes = [vp, ctypes.c_int32, ctypes.c_double, ctypes.POINTER(ctypes.c_int32)]
    lib.ac_kmax_calibrate.restype = st
    lib.ac_step_params.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(CSchedule), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(Params)]
    lib.ac_step_params.restype = st
    lib.ac_status_str.argtypes = [st]
    lib.ac_status_str.restype = ctypes.c_char_p
    lib.ac_last_error.argtypes = []
    lib.ac_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != AC_OK:
        lib = load()
        raise ACError(status, f"{lib.ac_status_str(status).decode()}: {lib.ac_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libac must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------- parameter helpers
def params_default(**kw) -> Params:
    p = Params()
    _check(load().ac_params_default(ctypes.byref(p)))
    for k, v in kw.items():
        if not hasattr(p, k):
            raise AttributeError(k)
        setattr(p, k, v)
    return p


def ac_sizes(shape: Shape, params: Params):
    """(ncap_k, workspace bytes) for this shape and these parameters."""
    ncap = ctypes.c_int32()
    ws = ctypes.c_size_t()
    _check(load().ac_sizes(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(ncap), ctypes.byref(ws)))
    return ncap.value, ws.value


# ---------------------------------------------------------------- device buffers (torch)
class Clusters:
    """Device arrays of one side's clusters (see ac_clusters)."""

    def __init__(self, BH: int, L: int, ncap: int, d: int, device, rho: bool):
        import torch
        i32 = torch.int32
        self.ncap = ncap
        self.labels = torch.empty((BH, L), dtype=i32, device=device)
        self.perm = torch.empty((BH, L), dtype=i32, device=device)
        self.seg = torch.empty((BH, ncap + 1), dtype=i32, device=device)
        self.cent = torch.zeros((BH, ncap, d), dtype=torch.float32, device=device)
        self.ncl = torch.empty((BH,), dtype=i32, device=device)
        self.rho = torch.empty((BH, ncap), dtype=torch.float32, device=device) if rho else None

    def c(self) -> CClusters:
        return CClusters(self.ncap, _ptr(self.labels), _ptr(self.perm), _ptr(self.seg), _ptr(self.cent),
                         _ptr(self.ncl), _ptr(self.rho))


class KStats:
    def __init__(self, BH: int, ncap: int, d: int, device):
        import torch
        self.kmax = torch.empty((BH, ncap, d), dtype=torch.bfloat16, device=device)
        self.kmin = torch.empty((BH, ncap, d), dtype=torch.bfloat16, device=device)
        self.kmean = torch.empty((BH, ncap, d), dtype=torch.float32, device=device)
        self.vmean = torch.empty((BH, ncap, d), dtype=torch.float32, device=device)
        self.fallback = torch.empty((BH,), dtype=torch.uint8, device=device)
        self.tau = torch.empty((BH,), dtype=torch.float32, device=device)
        self.mse = torch.empty((BH,), dtype=torch.float32, device=device)
        self.stages = torch.empty((BH,), dtype=torch.int32, device=device)

    def c(self) -> CKStats:
        return CKStats(_ptr(self.kmax), _ptr(self.kmin), _ptr(self.kmean), _ptr(self.vmean), _ptr(self.fallback),
                       _ptr(self.tau), _ptr(self.mse), _ptr(self.stages))


class KTrace:
    """Device arrays of a key-clustering stage record (see ac_ktrace)."""

    def __init__(self, BH: int, L: int, max_stages: int, iters: int, m0: int, d: int, device):
        import torch
        i32 = torch.int32
        self.max_stages = max_stages
        self.n = torch.zeros((BH, max_stages), dtype=i32, device=device)
        self.m = torch.zeros((BH, max_stages), dtype=i32, device=device)
        self.u = torch.full((BH, max_stages, L), -1, dtype=i32, device=device)
        self.cent = torch.zeros((BH, max_stages, iters + 1, m0, d), dtype=torch.float32, device=device)
        self.labels = torch.full((BH, max_stages, L), -1, dtype=i32, device=device)
        self.dist = torch.zeros((BH, max_stages, L), dtype=torch.float32, device=device)

    def c(self) -> CKTrace:
        return CKTrace(self.max_stages, _ptr(self.n), _ptr(self.m), _ptr(self.u), _ptr(self.cent),
                       _ptr(self.labels), _ptr(self.dist))


class Selection:
    def __init__(self, BH: int, nq: int, ncap_k: int, device, score: bool = True):
        import torch
        self.ncap_k = ncap_k
        self.list = torch.empty((BH, nq, ncap_k), dtype=torch.int32, device=device)
        self.n = torch.empty((BH, nq), dtype=torch.int32, device=device)
        self.mask = torch.empty((BH, nq, (ncap_k + 31) // 32), dtype=torch.int32, device=device)
        self.score = torch.empty((BH, nq, ncap_k), dtype=torch.float32, device=device) if score else None

    def c(self) -> CSelection:
        return CSelection(self.ncap_k, _ptr(self.list), _ptr(self.n), _ptr(self.mask), _ptr(self.score))


class State:
    """Centres and flags carried from one denoising step to the next."""

    def __init__(self, BH: int, nq: int, ncap_k: int, d: int, device):
        import torch
        self.cent_q = torch.zeros((BH, nq, d), dtype=torch.float32, device=device)
        self.cent_k = torch.zeros((BH, ncap_k, d), dtype=torch.float32, device=device)
        self.ncl_k = torch.zeros((BH,), dtype=torch.int32, device=device)
        self.fallback = torch.zeros((BH,), dtype=torch.uint8, device=device)
        self.tau = torch.zeros((BH,), dtype=torch.float32, device=device)
        self.valid = 0
        self._c = None

    def c(self) -> CState:
        self._c = CState(_ptr(self.cent_q), _ptr(self.cent_k), _ptr(self.ncl_k), _ptr(self.fallback),
                         _ptr(self.tau), self.valid)
        return self._c


def workspace(nbytes: int, device):
    """A 256-byte aligned device byte buffer of at least nbytes."""
    import torch
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


# ---------------------------------------------------------------- entry points
def ac_cluster_q(shape, params, Q, warm_cent, q_out: Clusters, ws, stream=None):
    _check(load().ac_cluster_q(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(warm_cent),
                               ctypes.byref(q_out.c()), _ptr(ws), ws.numel(), _stream(stream)))


def ac_cluster_k(shape, params, K, V, warm: Optional[State], k_out: Clusters, stats: KStats, ws, stream=None):
    wc = ctypes.byref(warm.c()) if warm is not None else None
    _check(load().ac_cluster_k(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V), wc,
                               ctypes.byref(k_out.c()), ctypes.byref(stats.c()), _ptr(ws), ws.numel(),
                               _stream(stream)))


def ac_cluster_k_trace(shape, params, K, V, k_out: Clusters, stats: KStats, trace: KTrace, ws, stream=None):
    _check(load().ac_cluster_k_trace(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V),
                                     ctypes.byref(k_out.c()), ctypes.byref(stats.c()), ctypes.byref(trace.c()),
                                     _ptr(ws), ws.numel(), _stream(stream)))


def ac_cluster_q_trace(shape, params, Q, q_out: Clusters, cent_trace, ws, stream=None):
    """cent_trace: [BH, iters + 1, q_out.ncap, d] float32."""
    _check(load().ac_cluster_q_trace(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), ctypes.byref(q_out.c()),
                                     _ptr(cent_trace), _ptr(ws), ws.numel(), _stream(stream)))


class PcaTrace:
    """Device arrays of a principal-component split record (see ac_pca_trace)."""

    def __init__(self, BH: int, L: int, block: int, levels: int, d: int, device):
        import torch
        nint = max(1, -(-L // block) - 1)
        self.dir = torch.zeros((BH, nint, d), dtype=torch.float32, device=device)
        self.perm = torch.full((BH, max(levels, 1), L), -1, dtype=torch.int32, device=device)

    def c(self) -> CPcaTrace:
        return CPcaTrace(_ptr(self.dir), _ptr(self.perm))


def ac_cluster_q_pca(shape, params, Q, block: int, q_out: Clusters, ws, trace: Optional[PcaTrace] = None,
                     stream=None):
    tc = ctypes.byref(trace.c()) if trace is not None else None
    _check(load().ac_cluster_q_pca(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), int(block),
                                   ctypes.byref(q_out.c()), tc, _ptr(ws), ws.numel(), _stream(stream)))


def ac_cluster_k_pca(shape, params, K, V, block: int, k_out: Clusters, stats: KStats, ws,
                     trace: Optional[PcaTrace] = None, stream=None):
    tc = ctypes.byref(trace.c()) if trace is not None else None
    _check(load().ac_cluster_k_pca(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V), int(block),
                                   ctypes.byref(k_out.c()), ctypes.byref(stats.c()), tc, _ptr(ws), ws.numel(),
                                   _stream(stream)))


def ac_score_select(shape, params, q: Clusters, k: Clusters, stats: KStats, sel: Selection, ws, stream=None):
    _check(load().ac_score_select(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(q.c()),
                                  ctypes.byref(k.c()), ctypes.byref(stats.c()), ctypes.byref(sel.c()), _ptr(ws),
                                  ws.numel(), _stream(stream)))


def ac_score_select_noalloc(shape, params, q: Clusters, k: Clusters, stats: KStats, sel: Selection, stream=None):
    """ac_score_select with the library's fixed scratch array instead of a workspace."""
    _check(load().ac_score_select_noalloc(ctypes.byref(shape), ctypes.byref(params), ctypes.byref(q.c()),
                                          ctypes.byref(k.c()), ctypes.byref(stats.c()), ctypes.byref(sel.c()),
                                          _stream(stream)))


def ac_sparse_attn(shape, params, Q, K, V, q: Clusters, k: Clusters, stats: KStats, sel: Selection, O, lse=None,
                   ws=None, stream=None):
    _check(load().ac_sparse_attn(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(K), _ptr(V),
                                 ctypes.byref(q.c()), ctypes.byref(k.c()), ctypes.byref(stats.c()),
                                 ctypes.byref(sel.c()), _ptr(O), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))


def ac_tail_merge(shape, params, block: int, q_in: Clusters, sel_in: Selection, q_out: Clusters,
                  sel_out: Selection, ws, stream=None):
    _check(load().ac_tail_merge(ctypes.byref(shape), ctypes.byref(params), int(block), ctypes.byref(q_in.c()),
                                ctypes.byref(sel_in.c()), ctypes.byref(q_out.c()), ctypes.byref(sel_out.c()),
                                _ptr(ws), ws.numel(), _stream(stream)))


def ac_score_tokens(shape, params, Q, k: Clusters, stats: KStats, engine: int, S, ld: int, stream=None):
    """Per-token Quest scores into S ([BH, L, ld] float32)."""
    _check(load().ac_score_tokens(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), ctypes.byref(k.c()),
                                  ctypes.byref(stats.c()), int(engine), _ptr(S), int(ld), _stream(stream)))


def ac_interaction_matrix(shape, params, Q, q: Clusters, M, ws, stream=None):
    """M_Q of every head ([BH, d, d] float32) from the query clusters q."""
    _check(load().ac_interaction_matrix(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), ctypes.byref(q.c()),
                                        _ptr(M), _ptr(ws), ws.numel(), _stream(stream)))


def ac_cluster_k_metric(shape, params, K, V, M, k_out: Clusters, stats: KStats, ws, stream=None):
    _check(load().ac_cluster_k_metric(ctypes.byref(shape), ctypes.byref(params), _ptr(K), _ptr(V), _ptr(M),
                                      ctypes.byref(k_out.c()), ctypes.byref(stats.c()), _ptr(ws), ws.numel(),
                                      _stream(stream)))


def ac_layer(shape, params, Q, K, V, state: State, O, ws, host_stats: bool = False, stream=None):
    """Run the whole layer.  Returns a dict of per-head numpy arrays when
    host_stats is set (the call then waits for the stream), else None."""
    import numpy as np
    BH = shape.B * shape.H
    hs = None
    arrs = None
    if host_stats:
        arrs = dict(ncl_k=np.zeros(BH, np.int32), fallback=np.zeros(BH, np.uint8), tau=np.zeros(BH, np.float32),
                    mse=np.zeros(BH, np.float32), stages=np.zeros(BH, np.int32), pairs=np.zeros(BH, np.int64))
        hs = CLayerStats(*(a.ctypes.data for a in arrs.values()))
    cs = state.c()
    _check(load().ac_layer(ctypes.byref(shape), ctypes.byref(params), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(cs),
                           _ptr(O), ctypes.byref(hs) if hs is not None else None, _ptr(ws), ws.numel(),
                           _stream(stream)))
    state.valid = cs.valid
    return arrs


# ---------------------------------------------------------------- multi-step policy (host only)
def ac_topp_schedule(log_snr, warmup_steps: int, p_min: float, tau: float, t_pivot: int = -1):
    """Per-step top-p (numpy float32 array) of the SNR-guided schedule."""
    import numpy as np
    ell = np.ascontiguousarray(log_snr, dtype=np.float64)
    out = np.empty(ell.size, dtype=np.float32)
    _check(load().ac_topp_schedule(ell.ctypes.data, ell.size, int(warmup_steps), float(p_min), float(tau),
                                   int(t_pivot), out.ctypes.data))
    return out


def ac_kmax_calibrate(ncl, frac: float) -> int:
    import numpy as np
    n = np.ascontiguousarray(ncl, dtype=np.int32)
    k = ctypes.c_int32(0)
    _check(load().ac_kmax_calibrate(n.ctypes.data, n.size, float(frac), ctypes.byref(k)))
    return int(k.value)


class Schedule:
    """Holds an ac_schedule and the host array its topp points to."""

    def __init__(self, warmup_steps: int = 0, warmup_layers: int = 0, nmax: int = 0, topp=None):
        import numpy as np
        self.topp = None if topp is None else np.ascontiguousarray(topp, dtype=np.float32)
        self.s = CSchedule(warmup_steps, warmup_layers, nmax, 0 if self.topp is None else self.topp.size,
                           None if self.topp is None else self.topp.ctypes.data)


def ac_step_params(base: Params, sch: Schedule, step: int, layer: int) -> Params:
    out = Params()
    _check(load().ac_step_params(ctypes.byref(base), ctypes.byref(sch.s), int(step), int(layer), ctypes.byref(out)))
    return out
