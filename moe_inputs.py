"""Seeded synthetic inputs for one MoE layer.

This module is shared by the CPU oracle side (tests, the CPU baseline) and the
GPU side (tests, bench).  It draws random numbers and rounds the draws that the
layer consumes in bfloat16; it holds none of the layer's arithmetic (no routing,
no quantisation, no expert maths).

Recipe (one ``numpy.random.PCG64`` stream per tensor, all spawned from
``SeedSequence(seed)``):

* ``x``      [T, d]   N(0, 1), rounded to bf16 (round-to-nearest-even)
* ``w_r``    [E, d]   N(0, 1/d), rounded to bf16 (the router weight)
* ``dy``     [T, d]   N(0, 1), rounded to bf16 (upstream gradient)
* ``w1[e]``  [2I, d]  N(0, 1/d) float32, gate rows 0..I-1 then up rows I..2I-1
* ``w2[e]``  [d, I]   N(0, 1/d) float32
* ``bias``   [E]      Zipf-shaped per-expert router bias (skewed workload only):
  ``-lam * s * ln(e + 1)`` with s = 1.1, so expert 0 is the hottest.

Expert weights come one expert at a time (``expert_weights``) so that a host
never needs more than one expert in float32.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# stream slots inside SeedSequence(seed).spawn(...)
_X, _WR, _DY, _BIAS, _EXPERT0 = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class LayerConfig:
    """Shape and routing of one MoE layer workload."""

    name: str
    T: int          # tokens in the batch
    d: int          # hidden size
    E: int          # routed experts
    k: int          # experts per token
    inter: int      # SwiGLU intermediate size I
    score: str      # "softmax" (softmax over the k selected logits) or "sigmoid" (sigmoid, normalised)
    seed: int
    n_shared: int = 0       # always-on shared experts (0 or 1)
    zipf_s: float = 0.0     # Zipf exponent of the router bias (0 = no bias)
    zipf_lam: float = 0.0   # scale of the Zipf bias
    backward: bool = False  # the workload includes the backward pass
    ring_rows: int = 0      # ring capacity the workload asks for (0 = library default)

    @property
    def rows(self) -> int:
        """Routed rows R = T*k plus one row per token for each shared expert."""
        return self.T * self.k + self.n_shared * self.T

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five workloads: a tiny layer, a Qwen3-30B-A3B-like layer, the DeepSeek-V3
# layer (forward), a Kimi-K2-shaped layer with a skewed router and a shared
# expert, and the DeepSeek-V3 layer forward + backward.
CONFIGS = {
    "tiny": LayerConfig("tiny", T=256, d=256, E=8, k=2, inter=128, score="softmax", seed=0),
    "qwen3_30b_a3b": LayerConfig("qwen3_30b_a3b", T=2048, d=2048, E=128, k=8, inter=768,
                                 score="softmax", seed=1),
    "dsv3_fwd": LayerConfig("dsv3_fwd", T=8192, d=7168, E=256, k=8, inter=2048,
                            score="sigmoid", seed=2),
    "kimi_k2_skew": LayerConfig("kimi_k2_skew", T=16384, d=7168, E=384, k=8, inter=2048,
                                score="sigmoid", seed=3, n_shared=1, zipf_s=1.1,
                                zipf_lam=0.21, ring_rows=2048),
    "dsv3_fwd_bwd": LayerConfig("dsv3_fwd_bwd", T=8192, d=7168, E=256, k=8, inter=2048,
                                score="sigmoid", seed=4, backward=True),
}


def _streams(cfg: LayerConfig) -> list[np.random.SeedSequence]:
    n_exp = cfg.E + cfg.n_shared
    return np.random.SeedSequence(cfg.seed).spawn(_EXPERT0 + 2 * n_exp)


def _normal(ss: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 draws to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """The float32 values of bfloat16 bit patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInputs:
    """Dense activations and router of one workload (expert weights are separate)."""

    cfg: LayerConfig
    x_bits: np.ndarray      # [T, d] uint16 (bf16)
    w_r_bits: np.ndarray    # [E, d] uint16 (bf16)
    bias: np.ndarray | None  # [E] float32 or None
    dy_bits: np.ndarray | None  # [T, d] uint16 (bf16) or None

    @property
    def x(self) -> np.ndarray:
        return bf16_values(self.x_bits)

    @property
    def w_r(self) -> np.ndarray:
        return bf16_values(self.w_r_bits)

    @property
    def dy(self) -> np.ndarray:
        return bf16_values(self.dy_bits)


def layer_inputs(cfg: LayerConfig, with_dy: bool | None = None) -> LayerInputs:
    """Draw x, the router weight, the optional Zipf bias and (for backward) dy."""
    s = _streams(cfg)
    x = bf16_bits(_normal(s[_X], (cfg.T, cfg.d), 1.0))
    w_r = bf16_bits(_normal(s[_WR], (cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d)))
    bias = None
    if cfg.zipf_s > 0.0:
        e = np.arange(cfg.E, dtype=np.float64)
        bias = (-cfg.zipf_lam * cfg.zipf_s * np.log(e + 1.0)).astype(np.float32)
    if with_dy is None:
        with_dy = cfg.backward
    dy = bf16_bits(_normal(s[_DY], (cfg.T, cfg.d), 1.0)) if with_dy else None
    return LayerInputs(cfg, x, w_r, bias, dy)


def expert_weights(cfg: LayerConfig, e: int) -> tuple[np.ndarray, np.ndarray]:
    """float32 (w1 [2I, d], w2 [d, I]) of expert e (e == E is the shared expert)."""
    s = _streams(cfg)
    std = 1.0 / math.sqrt(cfg.d)
    w1 = _normal(s[_EXPERT0 + 2 * e], (2 * cfg.inter, cfg.d), std)
    w2 = _normal(s[_EXPERT0 + 2 * e + 1], (cfg.d, cfg.inter), std)
    return w1, w2


def iter_expert_weights(cfg: LayerConfig, experts=None, threads: int = 8):
    """Yield (e, w1, w2) in expert order, drawing a few experts ahead on worker threads."""
    if experts is None:
        experts = range(cfg.E + cfg.n_shared)
    experts = list(experts)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        futs = {}
        ahead = max(1, threads)
        for i, e in enumerate(experts[:ahead]):
            futs[i] = ex.submit(expert_weights, cfg, e)
        for i, e in enumerate(experts):
            w1, w2 = futs.pop(i).result()
            nxt = i + ahead
            if nxt < len(experts):
                futs[nxt] = ex.submit(expert_weights, cfg, experts[nxt])
            yield e, w1, w2
