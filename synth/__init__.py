"""Seeded synthetic inputs for the dropless MoE expert-FFN layer.

This module is shared by the tests, the benchmark and the smoke check. It holds
only input generation: random tensors, the per-expert router bias that makes
the routing skewed, and the fp32 -> bf16 storage cast of the generated inputs.
It contains none of the layer's arithmetic (no routing, no GEMM, no activation).

The workloads stand in for the model shapes the pages talk about (DeepSeek-V3,
GPT-OSS and Mixtral-style expert FFNs); no dataset or trained weight is used.

Recipe (numpy ``default_rng``, one independent stream per tensor family):

* ``rng([seed, 0])``: a permutation ``perm`` of the experts; the router bias is
  ``-s * ln(perm + 1)`` (a Zipf(s) skew over the expert popularity ranks).
  Experts forced empty get bias ``-30`` so no token selects them.
* ``rng([seed, 1])``: logits ``= float32(N(0,1)[T,E] + bias)``.
* ``rng([seed, 2])``: ``x ~ N(0,1) [T,d]``.
* ``rng([seed, 3])``: ``W1 ~ N(0,1/d) [E,2f,d]`` then ``W2 ~ N(0,1/d) [E,d,f]``
  (``[E,f,d]`` for the non-gated squared-ReLU FFN).
* ``rng([seed, 4])``: ``b1 ~ N(0,1) [E,2f]`` then ``b2 ~ N(0,1) [E,d]`` (fp32).
* ``rng([seed, 5])``: ``dOut ~ N(0,1) [T,d]``.

Floating tensors are drawn as float32 and, for bf16 workloads, rounded to bf16
(round-to-nearest-even) and returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "MoEConfig", "WORKLOADS", "workload", "make_inputs", "f32_to_bf16_bits", "draw_router_weights",
    "bf16_bits_to_f32", "draw_router", "to_torch",
]


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Shape and options of one expert-FFN workload."""
    name: str
    T: int                    # tokens
    d: int                    # hidden size
    f: int                    # expert FFN size (per GLU half)
    E: int                    # experts (local to this GPU)
    k: int                    # experts per token
    dtype: str = "bf16"       # storage dtype of activations / weights: "bf16" | "f32"
    gemm: str = "bf16"        # GEMM operand precision: "bf16" | "f32" | "mxfp8" | "mxfp4"
    score: str = "softmax"    # "softmax" | "sigmoid"
    normalize: bool = True    # renormalise the selected gates to sum to 1
    act: str = "swiglu"       # "swiglu" | "geglu" | "srelu"
    clamp: float = 0.0        # <= 0: no clamp
    alpha: float = 1.0        # silu slope: silu_a(g) = g * sigmoid(a g)
    bias: bool = False        # b1 / b2 present
    zipf: float = 0.0         # Zipf exponent of the router bias
    forced_empty: int = 0     # experts forced to receive no token
    forced_mode: str = "top"  # "last": expert E-1; "top": largest perm values
    seed: int = 0
    backward: bool = False

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def gated(self) -> bool:
        return self.act in ("swiglu", "geglu")

    @property
    def n1(self) -> int:
        """Output width of FC1 (2f for gated activations, f for squared ReLU)."""
        return 2 * self.f if self.gated else self.f

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    def gemm_flops(self) -> int:
        """Algorithmic GEMM FLOP of one pass (forward, plus backward if set).

        Forward: FC1 2*R*d*n1 + FC2 2*R*d*f.  Backward: twice that
        (dgrad + wgrad of each of the two GEMMs)."""
        fwd = 2 * self.R * self.d * self.n1 + 2 * self.R * self.d * self.f
        return fwd * (3 if self.backward else 1)


WORKLOADS = {
    # fp32 correctness case; one expert forced empty.
    "tiny_fp32": MoEConfig("tiny_fp32", T=256, d=128, f=256, E=8, k=2, dtype="f32",
                           gemm="f32", score="softmax", zipf=0.0, forced_empty=1,
                           forced_mode="last", seed=1, backward=True),
    # Mixtral-like expert FFN, forward only.
    "mixtral_fwd": MoEConfig("mixtral_fwd", T=4096, d=4096, f=14336, E=8, k=2,
                             score="softmax", zipf=1.1, seed=2),
    # GPT-OSS-like expert FFN with clamp and biases, forward + backward.
    "gptoss_fwdbwd": MoEConfig("gptoss_fwdbwd", T=8192, d=2880, f=2880, E=32, k=4,
                               score="softmax", zipf=1.2, clamp=7.0, bias=True,
                               seed=3, backward=True),
    # DeepSeek-V3-like one-GPU expert shard (32 local experts), forward + backward.
    "dsv3_fwdbwd": MoEConfig("dsv3_fwdbwd", T=16384, d=7168, f=2048, E=32, k=8,
                             score="sigmoid", zipf=1.5, forced_empty=2, forced_mode="top",
                             seed=4, backward=True),
    # Same shard with MXFP8 GEMM operands.
    "dsv3_mxfp8_fwdbwd": MoEConfig("dsv3_mxfp8_fwdbwd", T=16384, d=7168, f=2048, E=32, k=8,
                                   gemm="mxfp8", score="sigmoid", zipf=1.5, forced_empty=2,
                                   forced_mode="top", seed=4, backward=True),
    # Same shard with MXFP4 GEMM operands.
    "dsv3_mxfp4_fwdbwd": MoEConfig("dsv3_mxfp4_fwdbwd", T=16384, d=7168, f=2048, E=32, k=8,
                                   gemm="mxfp4", score="sigmoid", zipf=1.5, forced_empty=2,
                                   forced_mode="top", seed=4, backward=True),
}


def workload(name: str, **overrides) -> MoEConfig:
    return WORKLOADS[name].replace(**overrides)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    # Process in slabs to bound temporary memory for multi-GiB weights.
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        v = flat_u[s:s + step]
        nan = (v & 0x7FFFFFFF) > 0x7F800000
        r = v + (np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1)))
        o = (r >> np.uint32(16)).astype(np.uint16)
        o[nan] = ((v[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
        flat_o[s:s + step] = o
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_router(cfg: MoEConfig, T: Optional[int] = None) -> np.ndarray:
    """Router logits [T,E] float32 with the Zipf per-expert bias of the recipe."""
    T = cfg.T if T is None else T
    E = cfg.E
    perm = np.random.default_rng([cfg.seed, 0]).permutation(E)
    bias = -cfg.zipf * np.log(perm + 1.0) if cfg.zipf > 0 else np.zeros(E)
    if cfg.forced_empty:
        if cfg.forced_mode == "last":
            empty = np.arange(E - cfg.forced_empty, E)
        else:
            empty = np.argsort(-perm, kind="stable")[:cfg.forced_empty]
        bias = bias.copy()
        bias[empty] = -30.0
    z = np.random.default_rng([cfg.seed, 1]).standard_normal((T, E), dtype=np.float32)
    return (z + bias).astype(np.float32)


def draw_router_weights(cfg: MoEConfig) -> np.ndarray:
    """Router weight [E, d] ~ N(0, 1/d) as bf16 bits (for layers that compute
    their own logits from x)."""
    a = _normal(np.random.default_rng([cfg.seed, 6]), (cfg.E, cfg.d), 1.0 / math.sqrt(cfg.d))
    return f32_to_bf16_bits(a)


def _normal(rng, shape, scale=1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def make_inputs(cfg: MoEConfig, parts=("x", "logits", "w", "b", "dout")) -> dict:
    """Generate the seeded inputs of ``cfg``.

    Returns a dict with float32 arrays (``dtype == "f32"``) or bf16 bit
    patterns as uint16 (``dtype == "bf16"``) for ``x``, ``W1``, ``W2``,
    ``dOut``; ``logits`` and biases are always float32.
    """
    T, d, f, E = cfg.T, cfg.d, cfg.f, cfg.E
    out = {"cfg": cfg}
    cast = (lambda a: a) if cfg.dtype == "f32" else f32_to_bf16_bits
    if "logits" in parts:
        out["logits"] = draw_router(cfg)
    if "x" in parts:
        out["x"] = cast(_normal(np.random.default_rng([cfg.seed, 2]), (T, d)))
    if "w" in parts:
        rw = np.random.default_rng([cfg.seed, 3])
        s = 1.0 / math.sqrt(d)
        out["W1"] = cast(_normal(rw, (E, cfg.n1, d), s))
        out["W2"] = cast(_normal(rw, (E, d, f), s))
    if "b" in parts and cfg.bias:
        rc = np.random.default_rng([cfg.seed, 4])
        out["b1"] = _normal(rc, (E, cfg.n1))
        out["b2"] = _normal(rc, (E, d))
    if "dout" in parts and cfg.backward:
        out["dOut"] = cast(_normal(np.random.default_rng([cfg.seed, 5]), (T, d)))
    return out


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """View generated storage (f32 array or bf16 bits) as float64 values."""
    if dtype == "bf16" or a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def to_torch(a: np.ndarray, device="cpu"):
    """numpy -> torch; uint16 arrays are reinterpreted as bfloat16."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)
