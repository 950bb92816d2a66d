"""Shared helpers of the GPU tests: parameter mapping between the oracle and
the C ABI, device upload, and running the layer's entry points stage by
stage through the binding.  Not a test module."""
from __future__ import annotations

import math

import numpy as np

import csa_inputs as gen
from oracle import numerics as nm


def f32(x: float) -> float:
    """Round a Python float to float32 (the ABI carries float parameters)."""
    return float(np.float32(x))


def oracle_params(**kw) -> nm.Params:
    p = nm.Params(**kw)
    p.tau_param = f32(p.tau_param)
    p.sel_param = f32(p.sel_param)
    p.scale = f32(p.scale)
    return p


def abi_params(p: nm.Params):
    import clustered_sparse_attention_amd as ac
    return ac.params_default(nq=p.nq, iters=p.iters, iters_warm=p.iters_warm, m0=p.m0, nmax=p.nmax,
                             tau_rule=p.tau_rule, tau_param=p.tau_param, score_mode=p.score_mode,
                             sel_mode=p.sel_mode, topk=p.topk, sel_param=p.sel_param, compensate=p.compensate,
                             scale=p.scale, init_sample=p.init_sample, seed=p.seed)


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_(t):
    return t.detach().cpu().numpy()


class Run:
    """Runs the four entry points on one workload and keeps every output."""

    def __init__(self, Qb, Kb, Vb, p: nm.Params):
        import torch
        import clustered_sparse_attention_amd as ac
        B, H, L, d = Qb.shape
        self.B, self.H, self.L, self.d = B, H, L, d
        self.BH = B * H
        self.p = p
        self.cp = abi_params(p)
        self.shape = ac.Shape(B, H, L, d)
        self.ncap_k, self.ws_bytes = ac.ac_sizes(self.shape, self.cp)
        self.nq = min(p.nq, L)
        dev = torch.device("cuda")
        self.Q, self.K, self.V = to_dev(Qb), to_dev(Kb), to_dev(Vb)
        self.ws = ac.workspace(self.ws_bytes, dev)
        self.q = ac.Clusters(self.BH, L, self.nq, d, dev, rho=True)
        self.k = ac.Clusters(self.BH, L, self.ncap_k, d, dev, rho=False)
        self.st = ac.KStats(self.BH, self.ncap_k, d, dev)
        self.sel = ac.Selection(self.BH, self.nq, self.ncap_k, dev)
        self.O = torch.empty_like(self.Q)
        self.lse = torch.empty((self.BH, L), dtype=torch.float32, device=dev)

    def cluster_q(self, warm_cent=None):
        import clustered_sparse_attention_amd as ac
        ac.ac_cluster_q(self.shape, self.cp, self.Q, warm_cent, self.q, self.ws)

    def cluster_k(self, warm=None):
        import clustered_sparse_attention_amd as ac
        ac.ac_cluster_k(self.shape, self.cp, self.K, self.V, warm, self.k, self.st, self.ws)

    def score_select(self):
        import clustered_sparse_attention_amd as ac
        ac.ac_score_select(self.shape, self.cp, self.q, self.k, self.st, self.sel, self.ws)

    def attn(self):
        import clustered_sparse_attention_amd as ac
        ac.ac_sparse_attn(self.shape, self.cp, self.Q, self.K, self.V, self.q, self.k, self.st, self.sel, self.O,
                          self.lse, self.ws)

    def all(self):
        self.cluster_q()
        self.cluster_k()
        self.score_select()
        self.attn()
        import torch
        torch.cuda.synchronize()
        return self


def near_tie_flips(X, C, lab_gpu, rel=1e-5):
    """Compare GPU labels with the oracle's nearest centre (fp64, given the
    GPU's centres).  Returns (mismatches, near-tie mismatches, near ties)."""
    from oracle import kmeans as okm
    d2 = okm.sq_dist(X, C)
    lab_o = np.argmin(d2, axis=1)
    srt = np.sort(d2, axis=1)
    gap = (srt[:, 1] - srt[:, 0]) if C.shape[0] > 1 else np.full(X.shape[0], np.inf)
    scale = np.sum(X * X, axis=1) + np.sum(C[lab_o] ** 2, axis=1)
    tie = gap < rel * scale
    mism = lab_o != lab_gpu
    return int(np.sum(mism & ~tie)), int(np.sum(mism & tie)), int(np.sum(tie))


def attn_error(O_gpu: np.ndarray, O_ref: np.ndarray):
    """(max abs error, relative L2 error)."""
    diff = O_gpu - O_ref
    return float(np.max(np.abs(diff))), float(np.linalg.norm(diff) / max(np.linalg.norm(O_ref), 1e-30))


ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
