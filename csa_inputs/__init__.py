"""Seeded synthetic inputs for one cluster-routed sparse attention layer.

This module only draws inputs. It holds none of the method's arithmetic
(no clustering, scoring, selection or attention), so both the CPU oracle
and the HIP path can be fed from it without sharing any code with each
other.

Every tensor is drawn in float32 with numpy's PCG64 generator, one stream
per head (``SeedSequence(seed).spawn(B*H)``), and then rounded to bfloat16
with round-to-nearest-even.  Tensors are returned as ``uint16`` arrays of
bfloat16 bit patterns with layout ``[B, H, L, d]``.

The shapes and value distributions follow the five workloads the layer is
measured on (a tiny case, and CogVideoX-2B-, HunyuanVideo-, Wan2.1-14B- and
long-sequence-shaped layers).  Real DiT activations need model weights and
prompt sets that are not available, so these mixtures stand in for them.

Per-head draw order (fixed): key centres, key labels, key noise, extra key
draws of the config (outlier masks / values), query directions, query
labels, query noise, query norms, V.
"""
from __future__ import annotations

import dataclasses
import re
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "generate", "generate_head",
    "perturb", "f32_to_bf16_bits", "bf16_bits_to_f32", "row_sample",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    seed: int
    n_key_comp: int
    key_sigma: tuple          # per-head sigma (len H)
    key_weights: str          # "uniform" | "zipf1.1" | "pow0.62"
    key_outlier: str          # "" | "uniform3" | "student3"
    key_outlier_frac: float
    key_outlier_scale: tuple  # per-head scale for student-t outliers (len H) or ()
    outlier_heads: tuple      # heads that receive outliers
    n_query_dir: int
    query_noise: float = 0.2
    description: str = ""

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def dense_flops(self) -> float:
        """4*B*H*L^2*d: multiply-adds of QK^T and PV, dense."""
        return 4.0 * self.B * self.H * float(self.L) ** 2 * self.d


def _w(name, B, H, L, d, seed, ncomp, sig, weights, outlier, ofrac, oscale, oheads, ndir, desc):
    return Workload(name, B, H, L, d, seed, ncomp, tuple(float(s) for s in sig), weights, outlier,
                    ofrac, tuple(float(s) for s in oscale), tuple(oheads), ndir, 0.2, desc)


WORKLOADS = {
    # Tiny single layer: 32-component key mixture, 16 query directions.
    "tiny": _w("tiny", 1, 2, 4096, 64, 101, 32, [0.3] * 2, "uniform", "", 0.0, (), (), 16,
               "tiny layer H=2 L=4096 d=64"),
    # CogVideoX-2B-like: 13x75x72 grid, 400 components, sigma in [0.1, 0.6] across heads.
    "cogvideox": _w("cogvideox", 1, 30, 13 * 75 * 72, 64, 102, 400, np.linspace(0.1, 0.6, 30),
                    "uniform", "", 0.0, (), (), 100, "CogVideoX-2B-like H=30 L=70200 d=64"),
    # HunyuanVideo-like: 33x45x80 grid; heads 0-11 compact, 12-23 dispersed + 10% uniform outliers.
    "hunyuan": _w("hunyuan", 1, 24, 33 * 45 * 80, 128, 103, 400, [0.15] * 12 + [0.8] * 12,
                  "uniform", "uniform3", 0.10, (), range(12, 24), 100,
                  "HunyuanVideo-like H=24 L=118800 d=128"),
    # Wan2.1-14B-like: 21x60x60 grid, 500 components with Zipf(1.1) sizes.
    "wan": _w("wan", 1, 40, 21 * 60 * 60, 128, 104, 500, [0.3] * 40, "zipf1.1", "", 0.0, (), (), 100,
              "Wan2.1-14B-like H=40 L=75600 d=128"),
    # Long stress: 80% from 1000 components (weights j^-0.62), 20% Student-t(3) with per-head
    # scale in [0.15, 0.75]; the widest heads cannot be covered by N_max centres and fall back.
    "long": _w("long", 1, 24, 180000, 128, 105, 1000, [0.3] * 24, "pow0.62", "student3", 0.20,
               np.linspace(0.15, 0.75, 24), range(24), 100, "long-sequence H=24 L=180000 d=128"),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if overrides:
        if "H" in overrides and "key_sigma" not in overrides:
            H = overrides["H"]
            sig = list(w.key_sigma)[:H] + [w.key_sigma[-1]] * max(0, H - len(w.key_sigma))
            overrides["key_sigma"] = tuple(sig)
            if w.key_outlier_scale:
                sc = list(w.key_outlier_scale)[:H] + [w.key_outlier_scale[-1]] * max(0, H - len(w.key_outlier_scale))
                overrides["key_outlier_scale"] = tuple(sc)
            overrides.setdefault("outlier_heads", tuple(h for h in w.outlier_heads if h < H))
        w = dataclasses.replace(w, **overrides)
        # the description names the shape: keep it in step with overridden sizes
        desc = re.sub(r"\bH=\d+", f"H={w.H}", w.description)
        desc = re.sub(r"\bL=\d+", f"L={w.L}", desc)
        w = dataclasses.replace(w, description=desc)
    return w


def _comp_weights(kind: str, n: int) -> np.ndarray:
    j = np.arange(1, n + 1, dtype=np.float64)
    if kind == "uniform":
        p = np.ones(n)
    elif kind == "zipf1.1":
        p = j ** -1.1
    elif kind == "pow0.62":
        p = j ** -0.62
    else:
        raise ValueError(kind)
    return p / p.sum()


def _normalize_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return (x / n).astype(np.float32)


def generate_head(w: Workload, rng: np.random.Generator, h: int):
    """Draw (Q, K, V) of one head as float32 arrays [L, d] before bf16 rounding."""
    L, d = w.L, w.d
    # keys
    centres = rng.standard_normal((w.n_key_comp, d), dtype=np.float32)
    klab = rng.choice(w.n_key_comp, size=L, p=_comp_weights(w.key_weights, w.n_key_comp))
    knoise = rng.standard_normal((L, d), dtype=np.float32)
    K = centres[klab] + np.float32(w.key_sigma[h]) * knoise
    if w.key_outlier and h in w.outlier_heads:
        mask = rng.random(L) < w.key_outlier_frac
        cnt = int(mask.sum())
        if w.key_outlier == "uniform3":
            vals = rng.uniform(-3.0, 3.0, size=(cnt, d)).astype(np.float32)
        elif w.key_outlier == "student3":
            vals = (np.float32(w.key_outlier_scale[h]) *
                    rng.standard_t(3.0, size=(cnt, d)).astype(np.float32))
        else:
            raise ValueError(w.key_outlier)
        K[mask] = vals
    # queries
    dirs = _normalize_rows(rng.standard_normal((w.n_query_dir, d), dtype=np.float32))
    qlab = rng.integers(0, w.n_query_dir, size=L)
    qnoise = rng.standard_normal((L, d), dtype=np.float32)
    qn = rng.lognormal(0.0, 0.5, size=L).astype(np.float32)
    Q = _normalize_rows(dirs[qlab] + np.float32(w.query_noise / math.sqrt(d)) * qnoise) * qn[:, None]
    V = rng.standard_normal((L, d), dtype=np.float32)
    return Q, K, V


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(w: Workload, heads: Optional[list] = None):
    """Return (Q, K, V) as uint16 bf16 bit arrays of shape [B, H, L, d].

    ``heads`` restricts generation to a subset of flattened (b, h) indices;
    the other heads are left zero (each head has its own stream, so a
    subset draws exactly the same values as a full run).
    """
    BH = w.BH
    ss = np.random.SeedSequence(w.seed).spawn(BH)
    out = [np.zeros((BH, w.L, w.d), dtype=np.uint16) for _ in range(3)]
    todo = list(range(BH)) if heads is None else list(heads)

    def one(bh):
        rng = np.random.Generator(np.random.PCG64(ss[bh]))
        Q, K, V = generate_head(w, rng, bh % w.H)
        out[0][bh] = f32_to_bf16_bits(Q)
        out[1][bh] = f32_to_bf16_bits(K)
        out[2][bh] = f32_to_bf16_bits(V)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, todo))
    return tuple(o.reshape(w.B, w.H, w.L, w.d) for o in out)


def perturb(x_bits: np.ndarray, seed: int = 1103, rel: float = 0.02) -> np.ndarray:
    """Next-denoising-step stand-in: X' = bf16(X + rel * rms_h(X) * eps), eps ~ N(0,1).

    rms is taken per (b, h) head over all of its elements.  One stream per head.
    """
    B, H, L, d = x_bits.shape
    ss = np.random.SeedSequence(seed).spawn(B * H)
    flat = x_bits.reshape(B * H, L, d)
    out = np.empty_like(flat)

    def one(bh):
        x = bf16_bits_to_f32(flat[bh])
        rms = np.float32(np.sqrt(np.mean(x.astype(np.float64) ** 2)))
        eps = np.random.Generator(np.random.PCG64(ss[bh])).standard_normal((L, d), dtype=np.float32)
        out[bh] = f32_to_bf16_bits(x + np.float32(rel) * rms * eps)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(B * H)))
    return out.reshape(B, H, L, d)


def row_sample(L: int, n: int, seed: int) -> np.ndarray:
    """Seeded sample of ``n`` distinct query rows in [0, L), ascending."""
    n = min(n, L)
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(L, size=n, replace=False))
