"""Seeded synthetic inputs for the fine-grained MoE feed-forward layer.

This module only draws random numbers and rounds them to the storage type.
It holds none of the layer's arithmetic, and it is the one piece shared by the
HIP path's callers (tests, bench) and by the CPU oracle's callers: both sides
receive the identical bits produced here.

Workload shapes follow the models on the pages:
  * Quartz Micro Preview Base model card (Architecture table) and the Vertex AGI
    research page (Architecture): hidden 1,024, 24 routed experts with 6 active,
    2 always-on shared experts, expert FFN width 640, load-balancing weight 0.01;
    one optimizer step is 4,096 tokens (Data section).
  * Moonfrost site (MoE card, stacking card): 32 routed experts, top 3, one shared
    expert, stacked (E, hidden, ffn) expert tensors with capacity-based routing.
  * Sutra-1.3B site ("48 + 1 experts" card): 48 routed experts, top 4, sigmoid
    scoring with bias-based load balancing, one shared expert.
  * dormouse site ("dropless MoE" and "TSCT low-rank experts" cards): 1,024
    experts, top-k 2, no capacity drops, each expert factorised as U diag(s) V^T
    of rank 64; training batch 24 x 1,024 bytes (terminal block).
Widths the pages do not give (Moonfrost expert width, Sutra and dormouse hidden
and expert widths) are fixed by the workload definitions below.

Draw order for every workload, from ``numpy.random.default_rng(seed)``:
  x, W_router, workload extras (logit offset / selection bias), the routed
  expert weights (gate, up, down; or U, s, V for gate, up, down in turn), then
  the shared expert weights (gate, up, down). Normal draws are float32
  ``standard_normal`` times the stated sigma; for bf16 workloads every drawn
  tensor is then rounded to bf16 (round to nearest, ties to even) so that both
  sides see exactly representable values. Biases stay float32.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from fractions import Fraction

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int                 # tokens (flattened batch-major)
    hidden: int            # d
    n_routed: int          # E
    top_k: int             # k
    n_shared: int          # S
    ffn: int               # F, width of every expert
    rank: int = 0          # 0: dense experts; r > 0: U diag(s) V^T factors
    score: str = "softmax"  # "softmax" | "sigmoid"
    renorm: int = 1        # softmax: renormalise gates over the top-k
    capacity_factor: str = ""  # "" dropless; else C = ceil(cf*T*k/E), e.g. "5/4"
    aux_coef: float = 0.01
    dtype: str = "bf16"    # "bf16" | "f32" for x and every weight; "fp8": bf16 draws,
                           # the expert products on fp8 codes of the same weights
    logit_offset_std: float = 0.0   # per-expert N(0, std) added to logits
    select_bias_std: float = 0.0    # per-expert N(0, std) selection-only bias
    zipf_s: float = 0.0             # logit offset -s*ln(i+1) by expert id
    x_std: float = 1.0
    w_std: float = 0.02
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def capacity(self) -> int:
        """Slots per expert; 0 means dropless."""
        if not self.capacity_factor:
            return 0
        return capacity_from_factor(Fraction(self.capacity_factor), self.T,
                                    self.top_k, self.n_routed)


def capacity_from_factor(factor: Fraction, T: int, k: int, E: int) -> int:
    """ceil(factor * T * k / E) in exact rational arithmetic."""
    q = Fraction(factor) * T * k / E
    return -((-q.numerator) // q.denominator)


TINY = Workload("tiny", T=64, hidden=128, n_routed=8, top_k=2, n_shared=1, ffn=64,
                dtype="f32")
QUARTZ = Workload("quartz", T=4096, hidden=1024, n_routed=24, top_k=6, n_shared=2,
                  ffn=640)
MOONFROST = Workload("moonfrost", T=16384, hidden=1024, n_routed=32, top_k=3,
                     n_shared=1, ffn=512, renorm=0, capacity_factor="5/4",
                     logit_offset_std=0.5)
SUTRA = Workload("sutra", T=32768, hidden=1536, n_routed=48, top_k=4, n_shared=1,
                 ffn=768, score="sigmoid", renorm=1, select_bias_std=0.1,
                 zipf_s=1.1)
DORMOUSE = Workload("dormouse", T=24576, hidden=768, n_routed=1024, top_k=2,
                    n_shared=0, ffn=512, rank=64, renorm=0)

WORKLOADS = {w.name: w for w in (TINY, QUARTZ, MOONFROST, SUTRA, DORMOUSE)}


def bf16_round_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even), as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _normal(rng, shape, std, bf16):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_round_f32(a) if bf16 else a


def _uniform(rng, shape, lo, hi, bf16):
    a = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return bf16_round_f32(a) if bf16 else a


def make_inputs(wl: Workload) -> dict:
    """Draw every input of one layer call. Returns float32 numpy arrays.

    Keys: x [T,d], w_router [d,E], logit_bias [E] or None, select_bias [E] or
    None; dense experts: w_gate, w_up [E,d,F], w_down [E,F,d]; low-rank experts:
    u_gate [E,d,r], s_gate [E,r], v_gate [E,F,r], the same for up, and
    u_down [E,F,r], s_down [E,r], v_down [E,d,r]; shared (S > 0): sh_gate,
    sh_up [S,d,F], sh_down [S,F,d].
    """
    rng = np.random.default_rng(wl.seed)
    bf = wl.dtype in ("bf16", "fp8")
    T, d, E, S, F, r = wl.T, wl.hidden, wl.n_routed, wl.n_shared, wl.ffn, wl.rank
    out: dict = {}
    out["x"] = _normal(rng, (T, d), wl.x_std, bf)
    out["w_router"] = _normal(rng, (d, E), wl.w_std, bf)
    logit_bias = None
    if wl.logit_offset_std > 0:
        logit_bias = rng.standard_normal(size=E, dtype=np.float32) * np.float32(
            wl.logit_offset_std)
    if wl.select_bias_std > 0:
        out["select_bias"] = rng.standard_normal(size=E, dtype=np.float32) * np.float32(
            wl.select_bias_std)
    else:
        out["select_bias"] = None
    if wl.zipf_s > 0:
        z = (-wl.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
        logit_bias = z if logit_bias is None else (logit_bias + z).astype(np.float32)
    out["logit_bias"] = logit_bias
    if r == 0:
        out["w_gate"] = _normal(rng, (E, d, F), wl.w_std, bf)
        out["w_up"] = _normal(rng, (E, d, F), wl.w_std, bf)
        out["w_down"] = _normal(rng, (E, F, d), wl.w_std, bf)
    else:
        for name, (din, dout) in (("gate", (d, F)), ("up", (d, F)), ("down", (F, d))):
            out["u_" + name] = _normal(rng, (E, din, r), wl.w_std, bf)
            out["s_" + name] = _uniform(rng, (E, r), 0.5, 1.5, bf)
            out["v_" + name] = _normal(rng, (E, dout, r), wl.w_std, bf)
    if S > 0:
        out["sh_gate"] = _normal(rng, (S, d, F), wl.w_std, bf)
        out["sh_up"] = _normal(rng, (S, d, F), wl.w_std, bf)
        out["sh_down"] = _normal(rng, (S, F, d), wl.w_std, bf)
    return out


def small_variant(wl: Workload, **kw) -> Workload:
    """A reduced-size copy of a workload for oracle-speed parity tests."""
    return wl.replace(**kw)


def make_upstream(wl: Workload, seed_offset: int = 1000) -> np.ndarray:
    """The loss gradient of the layer output for a backward call: float32
    standard normal [T, d] from ``default_rng(seed + seed_offset)`` (float32,
    like the layer output it stands for; not rounded)."""
    rng = np.random.default_rng(wl.seed + seed_offset)
    return rng.standard_normal(size=(wl.T, wl.hidden), dtype=np.float32)
