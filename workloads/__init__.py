"""Seeded synthetic inputs for the Switch FFN layer.

This module only draws random numbers and rounds them to bf16.  It holds none
of the layer's arithmetic (no routing, no softmax, no capacity, no FFN): both
the fp64 oracle and the HIP library receive what it produces, and neither is
imported here.

Shapes follow the layer sizes the pages discuss: 128 experts at capacity
factor 1.0 for Switch-Base (wq-win.github.io "042 Switch Transformer", section
four, Table 1), 64 experts (ai-papers.xuzou.cn paper card, "evidence", Fig. 5)
and 2048 experts (same card, Table 9, Switch-C).  Weight scales follow the
"reduced initialisation" remark of the pages (wq-win section two; lapla.si
"costs" section): router weights with variance 0.1/d, expert weights with a
truncated normal of standard deviation 0.1/sqrt(fan_in).

Random streams.  Every tensor has its own PCG64 stream keyed by
(config seed, tensor tag[, expert index]), so one expert's weights can be
drawn without drawing the others and experts can be drawn in parallel:

    x      : (seed, 0)        standard normal, float32, then bf16 (RNE)
    W_r    : (seed, 1)        normal, variance 0.1/d, float32
    W1[e]  : (seed, 2, e)     truncated normal (|z| <= 2, redrawn), scaled by
                              0.1/sqrt(d), bf16
    W2[e]  : (seed, 3, e)     same with fan_in = d_ff
    logits : (seed, 4)        tie-heavy dispatch-only logits (integers in
                              [-3, 3] divided by 4)
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Router-bias scale for the congested layer (configuration 3).  The bias of
# expert e is -1.1 * ln(e + 1) * ZIPF_BETA, a Zipf(1.1) profile with expert 0
# the most popular.  The value was found by bisection with
# oracle/calibrate_bias.py so that expert 0 receives 15 % (+-0.5 %) of the raw
# top-1 choices under the fp64 oracle router; tests/test_workloads.py checks it.
ZIPF_BETA = 0.11711645126342773


@dataclass(frozen=True)
class LayerConfig:
    index: int
    name: str
    T: int
    d: int
    d_ff: int
    E: int
    c: float
    alpha: float
    bias: str            # "plus2_expert0" | "zero" | "zipf"
    want_grad: bool      # whether the gradient of the aux loss is part of the workload

    @property
    def seed(self) -> int:
        return self.index


CONFIGS = {
    1: LayerConfig(1, "tiny_T512_d64_E4", 512, 64, 128, 4, 1.25, 0.01, "plus2_expert0", True),
    2: LayerConfig(2, "switch_base_T16384_d768_E128", 16384, 768, 3072, 128, 1.0, 0.01, "zero", False),
    3: LayerConfig(3, "congested_T16384_d768_E64_c2", 16384, 768, 3072, 64, 2.0, 0.01, "zipf", False),
    4: LayerConfig(4, "switch_large_T32768_d1024_E128", 32768, 1024, 4096, 128, 1.25, 0.01, "zero", True),
    5: LayerConfig(5, "many_small_T65536_d1024_E2048", 65536, 1024, 1024, 2048, 1.0, 0.01, "zero", False),
}


def custom_config(T, d, d_ff, E, c, alpha=0.01, bias="zero", index=101, name=None) -> LayerConfig:
    return LayerConfig(index, name or f"custom_T{T}_d{d}_F{d_ff}_E{E}", T, d, d_ff, E, c, alpha, bias, True)


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def _truncated_normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    flat = z.reshape(-1)
    bad = np.flatnonzero(np.abs(flat) > 2.0)
    while bad.size:
        flat[bad] = rng.standard_normal(bad.size, dtype=np.float32)
        bad = bad[np.abs(flat[bad]) > 2.0]
    z *= np.float32(scale)
    return z


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------- inputs
@dataclass
class LayerInputs:
    cfg: LayerConfig
    x_bits: np.ndarray                  # [T, d] uint16 (bf16)
    w_r: np.ndarray                     # [d, E] float32
    b_r: np.ndarray                     # [E] float32
    w1_bits: Optional[np.ndarray] = None  # [E, d_ff, d] uint16
    w2_bits: Optional[np.ndarray] = None  # [E, d, d_ff] uint16
    _x32: Optional[np.ndarray] = field(default=None, repr=False)

    @property
    def x(self) -> np.ndarray:
        if self._x32 is None:
            self._x32 = bf16_bits_to_f32(self.x_bits)
        return self._x32

    def w1(self, e: int) -> np.ndarray:
        return bf16_bits_to_f32(self.w1_bits[e])

    def w2(self, e: int) -> np.ndarray:
        return bf16_bits_to_f32(self.w2_bits[e])


def router_bias(cfg: LayerConfig, beta: float = ZIPF_BETA) -> np.ndarray:
    b = np.zeros(cfg.E, np.float32)
    if cfg.bias == "plus2_expert0":
        b[0] = 2.0
    elif cfg.bias == "zipf":
        e = np.arange(cfg.E, dtype=np.float64)
        b = (-1.1 * np.log(e + 1.0) * beta).astype(np.float32)
    elif cfg.bias != "zero":
        raise ValueError(cfg.bias)
    return b


def make_router_inputs(cfg: LayerConfig, beta: float = ZIPF_BETA) -> LayerInputs:
    x = _rng(cfg.seed, 0).standard_normal((cfg.T, cfg.d), dtype=np.float32)
    x_bits = f32_to_bf16_bits(x)
    w_r = (_rng(cfg.seed, 1).standard_normal((cfg.d, cfg.E), dtype=np.float32)
           * np.float32(math.sqrt(0.1 / cfg.d)))
    return LayerInputs(cfg, x_bits, w_r.astype(np.float32), router_bias(cfg, beta))


def expert_w1_bits(cfg: LayerConfig, e: int) -> np.ndarray:
    return f32_to_bf16_bits(_truncated_normal(_rng(cfg.seed, 2, e), (cfg.d_ff, cfg.d),
                                              0.1 / math.sqrt(cfg.d)))


def expert_w2_bits(cfg: LayerConfig, e: int) -> np.ndarray:
    return f32_to_bf16_bits(_truncated_normal(_rng(cfg.seed, 3, e), (cfg.d, cfg.d_ff),
                                              0.1 / math.sqrt(cfg.d_ff)))


def make_expert_weights(cfg: LayerConfig, threads: Optional[int] = None):
    """All experts' W1 [E, d_ff, d] and W2 [E, d, d_ff] as bf16 bits."""
    w1 = np.empty((cfg.E, cfg.d_ff, cfg.d), np.uint16)
    w2 = np.empty((cfg.E, cfg.d, cfg.d_ff), np.uint16)

    def one(e):
        w1[e] = expert_w1_bits(cfg, e)
        w2[e] = expert_w2_bits(cfg, e)

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(one, range(cfg.E)))
    return w1, w2


def make_layer_inputs(cfg: LayerConfig, with_experts: bool = True) -> LayerInputs:
    inp = make_router_inputs(cfg)
    if with_experts:
        inp.w1_bits, inp.w2_bits = make_expert_weights(cfg)
    return inp


def tie_heavy_logits(T: int, E: int, seed: int) -> np.ndarray:
    """Integers in [-3, 3] divided by 4, as float32: most rows hold exact ties."""
    return (_rng(seed, 4).integers(-3, 4, size=(T, E)).astype(np.float32) / np.float32(4.0))


def random_logits(T: int, E: int, seed: int, scale: float = 1.0) -> np.ndarray:
    return (_rng(seed, 5).standard_normal((T, E), dtype=np.float32) * np.float32(scale))


def random_bf16(shape, seed: int, tag: int = 6, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, scale^2) draws: generic operands for kernel-level tests."""
    return f32_to_bf16_bits(_rng(seed, tag).standard_normal(shape, dtype=np.float32) * np.float32(scale))
