"""Scalar helpers of the oracle: bfloat16 rounding, the counter-based random
stream used by k-means++, and the parameter record.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15

# parameter enums (values are part of the layer's interface)
TAU_MEAN_X, TAU_PCTL, TAU_ABS, TAU_INF = 0, 1, 2, 3
SCORE_QUEST, SCORE_MEAN = 0, 1
SEL_TOPK, SEL_DENSITY, SEL_TOPP, SEL_DENSE = 0, 1, 2, 3


@dataclasses.dataclass
class Params:
    """Hyperparameters of one layer.

    Defaults: 65 query clusters and tau = 1.5 x the mean token-to-centre
    distance of the first stage (AdaCluster §4.1 "Platform and
    configurations"); m0 = 200 initial key clusters and N_max = 1500 are
    readings (the pages give "moderate" and a calibrated cap).
    """
    nq: int = 65
    iters: int = 10
    iters_warm: int = 3
    m0: int = 200
    nmax: int = 1500
    tau_rule: int = TAU_MEAN_X
    tau_param: float = 1.5
    score_mode: int = SCORE_QUEST
    sel_mode: int = SEL_DENSITY
    topk: int = 8
    sel_param: float = 0.15
    compensate: int = 0
    scale: float = 0.0          # 0 -> 1/sqrt(d)
    init_sample: int = 8        # k-means++ subsample factor; 0 -> every point
    tail_block: int = 0         # query block of the tail merge (iCATS); 0 -> no merge
    seed: int = 0

    def attn_scale(self, d: int) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(d)

    def ncap_k(self) -> int:
        """Most key centres Algorithm 1 can hold: the cap is tested before a
        stage, so the last stage may add up to m0 centres on top of N_max-1."""
        return self.nmax - 1 + self.m0


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returning
    the bit patterns.  Works from the float64 value directly (one rounding,
    8 significant bits), via frexp: x = f * 2**e with 0.5 <= |f| < 1, so the
    bfloat16 spacing around x is 2**(e-8) (never below the subnormal spacing
    2**-133)."""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    spacing_exp = np.maximum(e - 8, -133)
    q = np.rint(np.ldexp(x, -spacing_exp))          # rint = round half to even
    r = np.ldexp(q, spacing_exp)
    r32 = r.astype(np.float32)                        # exact: r has <= 8 significant bits
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def splitmix64_next(state: int) -> tuple[int, int]:
    """One step of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014; the form
    in Vigna's public reference code): advance the state by the golden
    gamma, then apply the xor-shift-multiply finaliser.  Returns
    (new_state, output)."""
    state = (state + GOLDEN) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return state, z ^ (z >> 31)


def _mix(z: int) -> int:
    return splitmix64_next(z & MASK64)[1]


def stream_id(bh: int, role: int, stage: int) -> int:
    """Random stream of one k-means++ run: head bh, role 0 = queries,
    1 = keys, and the stage of Algorithm 1 (0 for queries)."""
    return ((bh & ((1 << 44) - 1)) << 20) | ((role & 0xF) << 16) | (stage & 0xFFFF)


def uniform01(seed: int, stream: int, counter: int) -> float:
    """Counter-based uniform in [0, 1): three chained SplitMix64 finalisers
    over (seed, stream, counter); the top 53 bits give the fraction."""
    x = _mix(seed & MASK64)
    x = _mix(x ^ (stream & MASK64))
    x = _mix(x ^ (counter & MASK64))
    return (x >> 11) * (1.0 / 9007199254740992.0)
