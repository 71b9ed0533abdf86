"""Shared helpers of the GPU parity tests: device transfer of seeded inputs,
the oracle pieces each test compares against, and the tolerance checks."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import workloads
from oracle import switch_oracle as so

DEV = "cuda"

# Output tolerances of the layer: relative Frobenius error <= 5e-3 and max abs
# error <= 3e-2 * rms(ref) on the expert branch; aux loss and P within 1e-5
# relative; tokens whose top-2 logit margin is at most 1e-4 may route
# differently (they are resolved by re-running the oracle with the device's
# choice for them).
REL_FRO = 5e-3
MAX_ABS_RMS = 3e-2
AUX_REL = 1e-5
MARGIN = 1e-4
# gradient of the aux loss: relative Frobenius and max abs (relative to max |G|)
GRAD_REL = 1e-5


def say(*a):
    print(f"[{time.strftime('%H:%M:%S')}]", *a, flush=True)
    sys.stdout.flush()


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def dev_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def top2_margin(z: np.ndarray) -> np.ndarray:
    part = np.partition(z, z.shape[1] - 2, axis=1) if z.shape[1] > 1 else None
    if part is None:
        return np.full(z.shape[0], np.inf)
    return part[:, -1] - part[:, -2]


def rel_fro(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return np.linalg.norm(a - ref) / (n if n > 0 else 1.0)


def assert_branch_close(got, ref, what="branch"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rf = rel_fro(got, ref)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    mx = np.max(np.abs(got - ref)) if ref.size else 0.0
    assert rf <= REL_FRO, f"{what}: relative Frobenius {rf:.3e} > {REL_FRO}"
    assert mx <= MAX_ABS_RMS * rms + 1e-30, f"{what}: max abs {mx:.3e} > {MAX_ABS_RMS} * rms {rms:.3e}"
    return rf, mx / rms if rms else 0.0


# Gradients of the layer backward: relative Frobenius <= REL_FRO, and per
# element |got - ref| <= GRAD_ELEM_REL |ref| + MAX_ABS_RMS rms(ref).  The
# proportional term covers the large entries of heavy-tailed gradients, whose
# error scales with their own size (bf16 operands of the MFMA: 2^-9 relative).
GRAD_ELEM_REL = 1e-2


def assert_grad_close(got, ref, what="gradient"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rf = rel_fro(got, ref)
    assert rf <= REL_FRO, f"{what}: relative Frobenius {rf:.3e} > {REL_FRO}"
    if ref.size:
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(got - ref)
        bad = err > GRAD_ELEM_REL * np.abs(ref) + MAX_ABS_RMS * rms + 1e-30
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements off, worst {err.max():.3e} "
                               f"(rms {rms:.3e})")
    return rf


def assert_residual_close(out_bits, x, branch_ref, what="out"):
    """Residual mode: out = bf16(x + branch).  Allowed error per element: one
    bf16 ulp of the exact result plus the branch tolerance (MAX_ABS_RMS times
    the branch rms), so cancellation near zero is judged on absolute terms."""
    ref = np.asarray(x, np.float64) + np.asarray(branch_ref, np.float64)
    got = workloads.bf16_bits_to_f32(out_bits).astype(np.float64)
    mag = np.maximum(np.abs(ref), 1e-38)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    rms = np.sqrt(np.mean(np.asarray(branch_ref, np.float64) ** 2)) if branch_ref.size else 0.0
    err = np.abs(got - ref)
    bad = err > ulp + MAX_ABS_RMS * rms
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, worst {err.max():.3e}"


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """|a - b| in bf16 ulps (ordered-integer distance of the bit patterns)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


class DeviceInputs:
    """A config's seeded inputs, on the GPU and (as float views) on the host."""

    def __init__(self, cfg: workloads.LayerConfig, with_experts=True):
        say(f"generate inputs {cfg.name}")
        self.cfg = cfg
        self.inp = workloads.make_layer_inputs(cfg, with_experts=with_experts)
        self.x = bits_to_dev(self.inp.x_bits)
        self.w_r = f32_dev(self.inp.w_r)
        self.b_r = f32_dev(self.inp.b_r)
        if with_experts:
            self.w1 = bits_to_dev(self.inp.w1_bits)
            self.w2 = bits_to_dev(self.inp.w2_bits)
        self.C = so.capacity(cfg.T, cfg.E, cfg.c)
        self._z = None
        say(f"inputs ready {cfg.name} C={self.C}")

    @property
    def z(self) -> np.ndarray:
        """Oracle router logits (fp64), computed once."""
        if self._z is None:
            self._z = so.router_logits(self.inp.x, self.inp.w_r, self.inp.b_r)
        return self._z


def sample_kept_tokens(keep: np.ndarray, n: int, seed: int) -> np.ndarray:
    kept = np.flatnonzero(keep)
    if kept.size <= n:
        return kept
    rng = np.random.default_rng(seed)
    pick = rng.choice(kept, size=n, replace=False)
    return np.unique(np.concatenate([pick, kept[:4], kept[-4:]]))


def oracle_branch_rows(inp: workloads.LayerInputs, tokens: np.ndarray, expert: np.ndarray, gate: np.ndarray):
    """Oracle branch gate_t * expert_e(x_t) for the given tokens, one expert at a time."""
    out = np.zeros((tokens.size, inp.cfg.d))
    for e in np.unique(expert[tokens]):
        sel = np.flatnonzero(expert[tokens] == e)
        rows = inp.x[tokens[sel]]
        out[sel] = gate[tokens[sel], None] * so.expert_rows(rows, inp.w1(e), inp.w2(e))
    return out
