"""Seeded synthetic inputs for the DiT-MoE sparse MoE feed-forward layer.

This module only draws and stores inputs: layer shapes, seeds, normal draws
and the bf16 storage rounding of the drawn values.  None of the layer's
arithmetic (gate, softmax, selection, expert MLPs, combine, balance) lives
here.  Both the CPU oracle and the GPU path take their inputs from it.

Shapes follow the DiT-MoE model names (X/p-nEkA: p patch size, n routed
experts, k activated; "Scaling Diffusion Transformers to 16 Billion
Parameters", compute analysis) and the DiT width table and token counts
("Scalable Diffusion Models with Transformers (DiT)", model architecture:
T = (I/8/p)^2, so 256 tokens at 256x256 and 1024 at 512x512).  The input x
stands in for the layer's real input (a LayerNorm-modulated hidden state, so
roughly unit variance per feature), and N(0, 0.02) weights stand in for
trained weights.  A per-expert N(0, 1) logit bias stands in for the skewed
expert loads those pages report.

Recipe (every tensor):  numpy PCG64 ``default_rng([seed, j])`` with a fixed
sub-stream ``j`` per tensor, ``standard_normal(shape, dtype=float32)``, times
the standard deviation in fp32; for bf16 layers the product is rounded to
bf16 with round-to-nearest-even.  The gate weight and the logit bias stay
fp32 in every layer.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

# sub-stream ids, one per tensor
SUB_X, SUB_WG, SUB_BIAS, SUB_W1, SUB_W2, SUB_W1S, SUB_W2S = range(7)

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class LayerConfig:
    name: str
    B: int            # images (sequences)
    T: int            # tokens per image
    D: int            # hidden size
    H: int            # expert hidden width (4*D)
    E: int            # routed experts
    K: int            # activated routed experts per token (nominal for race)
    n_s: int          # shared experts
    dtype: str        # "f32" or "bf16": x, expert weights, outputs
    route: str = "topk"   # "topk" or "race"
    alpha: float = 0.01
    logit_bias: bool = False
    seed: int = 0

    @property
    def N(self) -> int:
        return self.B * self.T

    @property
    def Kmax(self) -> int:
        return self.E if self.route == "race" else self.K

    @property
    def A(self) -> int:
        """Routed rows: K*N in both routing modes."""
        return self.K * self.N

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    def flops_per_token(self) -> int:
        """Gate plus the K+n_s expert MLPs, 2 FLOP per multiply-add."""
        return 2 * self.D * self.E + 4 * self.D * self.H * (self.K + self.n_s)

    def gemm_flops(self) -> int:
        return 4 * self.D * self.H * (self.K + self.n_s) * self.N


# The five workloads: DiT-MoE-S/2 fp32, S/2-16E2A, B/2-8E2A with skewed loads,
# XL/2-8E2A at 512x512 (uniform and skewed), and the Expert-Race stress layer.
CONFIGS = {
    "s_8e2a_f32": LayerConfig("s_8e2a_f32", B=2, T=256, D=384, H=1536, E=8, K=2,
                              n_s=2, dtype="f32", seed=1001),
    "s_16e2a": LayerConfig("s_16e2a", B=32, T=256, D=384, H=1536, E=16, K=2,
                           n_s=2, dtype="bf16", seed=1002),
    "b_8e2a_skew": LayerConfig("b_8e2a_skew", B=64, T=256, D=768, H=3072, E=8,
                               K=2, n_s=2, dtype="bf16", logit_bias=True,
                               seed=1003),
    "xl_8e2a_512": LayerConfig("xl_8e2a_512", B=32, T=1024, D=1152, H=4608,
                               E=8, K=2, n_s=2, dtype="bf16", seed=1004),
    "xl_8e2a_512_skew": LayerConfig("xl_8e2a_512_skew", B=32, T=1024, D=1152,
                                    H=4608, E=8, K=2, n_s=2, dtype="bf16",
                                    logit_bias=True, seed=1014),
    "race_16e": LayerConfig("race_16e", B=16, T=1024, D=2048, H=8192, E=16,
                            K=2, n_s=2, dtype="bf16", route="race", seed=1005),
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the same values as fp32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed: int, sub: int, shape, std: float):
    rng = np.random.default_rng([seed, sub])
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


@dataclass
class LayerInputs:
    """One layer's inputs.  Floating tensors are fp32 arrays holding the exact
    stored values (bf16-representable for bf16 layers); ``*_bits`` hold the
    bf16 bit patterns the GPU receives."""
    cfg: LayerConfig
    x: np.ndarray                 # [N][D]
    w_gate: np.ndarray            # [E][D] fp32
    bias: Optional[np.ndarray]    # [E] fp32 or None
    w1: np.ndarray                # [E][H][D]
    w2: np.ndarray                # [E][D][H]
    w1s: np.ndarray               # [n_s][H][D]
    w2s: np.ndarray               # [n_s][D][H]

    def bits(self, name: str) -> np.ndarray:
        return bf16_bits(getattr(self, name))


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(a))
    return a


def make_inputs(cfg: LayerConfig, seed: Optional[int] = None) -> LayerInputs:
    """Draw every input of ``cfg`` from its seeded sub-streams."""
    s = cfg.seed if seed is None else seed
    N, D, H, E, n_s = cfg.N, cfg.D, cfg.H, cfg.E, cfg.n_s
    x = _store(_normal(s, SUB_X, (N, D), 1.0), cfg.dtype)
    w_gate = _normal(s, SUB_WG, (E, D), WEIGHT_STD)
    bias = _normal(s, SUB_BIAS, (E,), 1.0) if cfg.logit_bias else None
    w1 = _store(_normal(s, SUB_W1, (E, H, D), WEIGHT_STD), cfg.dtype)
    w2 = _store(_normal(s, SUB_W2, (E, D, H), WEIGHT_STD), cfg.dtype)
    w1s = _store(_normal(s, SUB_W1S, (n_s, H, D), WEIGHT_STD), cfg.dtype)
    w2s = _store(_normal(s, SUB_W2S, (n_s, D, H), WEIGHT_STD), cfg.dtype)
    return LayerInputs(cfg, x, w_gate, bias, w1, w2, w1s, w2s)


def small_config(name: str = "tiny", **kw) -> LayerConfig:
    """A small layer for tests: defaults span several tiles with ragged tails."""
    base = dict(B=2, T=40, D=128, H=256, E=8, K=2, n_s=2, dtype="bf16",
                seed=7)
    base.update(kw)
    return LayerConfig(name, **base)
