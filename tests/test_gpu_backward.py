"""GPU parity of the layer backward (switch_layer_bwd) against the fp64 oracle.

The forward runs on the device with its saved tensors requested; the oracle
backward is fed the device's choices (they match the oracle's except on
near-tie tokens, and the gradient holds the choices fixed anyway).  Every
gradient meets relative Frobenius <= 5e-3.  Per element: the weight and
router-weight gradients |got - ref| <= 1e-2 |ref| + 3e-2 rms(ref)
(tests/gpu_helpers.py); dgate and dz a per-token bound derived from the
precision of y (see check_bwd); dx, rounded to bf16 once, one bf16 ulp plus
the branch tolerance, like the forward output.  dy and dA are bf16 on the device (MFMA inputs)
and the forward's hidden activation is bf16, which is what these tolerances
absorb.
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_order_amd as sw
import workloads
from oracle import switch_oracle as so
from tests.gpu_helpers import (DeviceInputs, assert_grad_close, assert_residual_close, bits_to_dev, dev_bits,
                               f32_dev, rel_fro, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Small:
    def __init__(self, T, d, F, E, c, seed, bias0=0.0):
        self.cfg = workloads.custom_config(T, d, F, E, c, index=1300 + seed)
        self.inp = workloads.make_layer_inputs(self.cfg)
        self.inp.b_r = self.inp.b_r.copy()
        self.inp.b_r[0] += bias0
        self.x, self.w_r, self.b_r = bits_to_dev(self.inp.x_bits), f32_dev(self.inp.w_r), f32_dev(self.inp.b_r)
        self.w1, self.w2 = bits_to_dev(self.inp.w1_bits), bits_to_dev(self.inp.w2_bits)
        self.C = so.capacity(T, E, c)


def run_fwd_bwd(D, seed, z_beta=0.0, C=None):
    cfg = D.cfg
    T, d, F, E = cfg.T, cfg.d, cfg.d_ff, cfg.E
    C = D.C if C is None else C
    t = sw.layer_tensors(T, d, F, E, C, for_backward=True, z_loss=z_beta > 0)
    ws = t.pop("ws")
    a = sw.make_layer_args(D.x, D.w_r, D.b_r, D.w1, D.w2, t, T, d, F, E, C, cfg.alpha, residual=True, z_beta=z_beta)
    sw.switch_layer_fwd(a, ws)
    dout_bits = workloads.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32))
    dout = bits_to_dev(dout_bits)
    g = sw.layer_bwd_tensors(T, d, F, E, C, inspect=True)
    gws = g.pop("ws")
    for v in g.values():
        v.view(torch.uint8).fill_(0xFF)
    b = sw.make_layer_bwd_args(t, D.x, D.w_r, D.w1, D.w2, dout, g, T, d, F, E, C, cfg.alpha, z_beta=z_beta)
    sw.switch_layer_bwd(b, gws)
    # the same backward with the identity term of dx left out: dx_branch is
    # the expert and router terms alone, rounded to bf16 once
    g["dx_branch"] = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    gb = dict(g, dx=g["dx_branch"])
    b2 = sw.make_layer_bwd_args(t, D.x, D.w_r, D.w1, D.w2, dout, gb, T, d, F, E, C, cfg.alpha, z_beta=z_beta,
                                dx_branch_only=True)
    sw.switch_layer_bwd(b2, gws)
    torch.cuda.synchronize()
    return t, g, dout_bits


def check_bwd(D, t, g, dout_bits, z_beta=0.0, C=None, label="", dw_experts=None):
    """dw_experts: compare the weight gradients of these experts only (the
    fp64 weight gradients of every expert do not fit in host memory at
    E * d * d_ff = 2^31); every other gradient is compared in full."""
    cfg = D.cfg
    C = D.C if C is None else C
    e_dev = t["expert"].cpu().numpy().astype(np.int64)
    dout = workloads.bf16_bits_to_f32(dout_bits).astype(np.float64)
    say(f"backward {label}: oracle")
    L = so.layer_forward(D.inp.x, D.inp.w_r, D.inp.b_r, D.inp.w1, D.inp.w2, cfg.c, cfg.alpha, C=C,
                         expert_override=e_dev)
    # The ReLU derivative is a decision taken in floating point: away from zero
    # the device's mask (its saved activation is non-zero) must equal the
    # oracle's [a > 0] exactly; pre-activations within 1e-4 rms of zero take
    # the device's decision (as near-tie choices do).
    h_dev = dev_bits(t["h"]) if C > 0 else None
    n_near = [0]

    def relu_active(e, a):
        dev = (h_dev[e, :a.shape[0]] & 0x7FFF) != 0
        rms = np.sqrt(np.mean(a ** 2)) if a.size else 0.0
        near = np.abs(a) <= 1e-4 * rms
        np.testing.assert_array_equal(dev[~near], (a > 0)[~near], err_msg=f"{label} ReLU mask of expert {e}")
        n_near[0] += int(near.sum())
        return np.where(near, dev, a > 0)

    ref = so.layer_backward(D.inp.x, D.inp.w_r, D.inp.b_r, D.inp.w1, D.inp.w2, cfg.c, cfg.alpha, dout, beta=z_beta,
                            C=C, expert_override=e_dev, forward=L, relu_active=relu_active, dw_experts=dw_experts)
    say(f"backward {label}: {n_near[0]} pre-activations within rounding of zero")
    keep = t["keep"].cpu().numpy().astype(bool)
    np.testing.assert_array_equal(keep, L.slots.keep)
    # dgate_t = <dout_t, y_t> inherits the error of y_t (bf16 hidden activation,
    # about 2^-9 relative per element) without the cancellation of the dot
    # product: |error| <= 2^-7 |dout_t| |y_t| per token.  dz inherits it through
    # dgate_t gate_t (delta_je - p_tj).
    T, E = cfg.T, cfg.E
    y_tok = np.zeros((T, cfg.d))
    kt = np.flatnonzero(keep)
    y_tok[kt] = L.y[e_dev[kt], L.slots.position[kt]]
    bound = 2.0 ** -7 * np.linalg.norm(dout, axis=1) * np.linalg.norm(y_tok, axis=1)
    dg = g["dgate"].cpu().numpy().astype(np.float64)
    assert np.all(dg[~keep] == 0), "dropped tokens carry no gate gradient"
    err = np.abs(dg - ref.dgate)
    assert np.all(err <= bound + 1e-6 * np.abs(ref.dgate) + 1e-30), f"{label} dgate: worst {np.max(err - bound):.3e}"
    dz = g["dz"].cpu().numpy().astype(np.float64)
    gate = L.routing.gate
    onehot = np.zeros((T, E))
    onehot[np.arange(T), e_dev] = 1.0
    zb = (2.0 * bound * gate)[:, None] * np.abs(onehot - L.routing.p)
    zerr = np.abs(dz - ref.dz)
    rms = np.sqrt(np.mean(ref.dz ** 2)) if ref.dz.size else 0.0
    bad = zerr > zb + 1e-2 * np.abs(ref.dz) + 1e-3 * rms + 1e-30
    assert not bad.any(), f"{label} dz: {int(bad.sum())} elements off"
    assert rel_fro(dz, ref.dz) <= 5e-3, f"{label} dz: relative Frobenius {rel_fro(dz, ref.dz):.3e}"
    assert_grad_close(g["db_r"].cpu().numpy(), ref.db_r, f"{label} db_r")
    assert_grad_close(g["dw_r"].cpu().numpy(), ref.dw_r, f"{label} dW_r")
    if dw_experts is None:
        dw1 = g["dw1"].cpu().numpy()
        dw2 = g["dw2"].cpu().numpy()
        acc = t["accepted"].cpu().numpy()
    else:
        sel = torch.from_numpy(np.asarray(dw_experts, np.int64)).to(DEV)
        dw1 = g["dw1"].index_select(0, sel).cpu().numpy()
        dw2 = g["dw2"].index_select(0, sel).cpu().numpy()
        acc = t["accepted"].cpu().numpy()[np.asarray(dw_experts)]
    empty = acc == 0
    assert np.all(dw1[empty] == 0) and np.all(dw2[empty] == 0), "experts without tokens get zero gradients"
    if (~empty).any():
        assert_grad_close(dw1, ref.dw1, f"{label} dW1")
        assert_grad_close(dw2, ref.dw2, f"{label} dW2")
    # dx is bf16(dout + branch): one bf16 ulp of the exact value plus the branch tolerance
    assert_residual_close(dev_bits(g["dx"]), dout, ref.dx - dout, f"{label} dx")
    # the branch of dx alone (expert term dA W1 plus router term W_r dz), at
    # the gradient tolerance: it carries two bf16 roundings (dy and dA, the
    # MFMA inputs) where the forward output carries one; emulating exactly
    # those on the CPU gives relative Frobenius 2.8e-3 and max/rms up to 3.04e-2
    if "dx_branch" in g:
        br = workloads.bf16_bits_to_f32(dev_bits(g["dx_branch"]))
        rf = assert_grad_close(br, ref.dx - dout, f"{label} dx branch")
        say(f"backward {label}: dx branch rel fro {rf:.2e}")
    say(f"backward {label}: ok, kept {int(keep.sum())}/{cfg.T}")
    return ref


@pytest.mark.parametrize("shape", [
    (512, 64, 128, 4, 1.25, 2.0),      # the tiny layer: hot expert 0, 352 dropped tokens
    (1000, 128, 192, 5, 1.1, 0.0),     # ragged T, d_ff not a multiple of 128
    (777, 64, 128, 1, 1.0, 0.0),       # one expert: the dense MLP, no router gradient
    (600, 64, 128, 6, 1.0, 3.0),       # empty experts
    (2000, 64, 128, 16, 4.5, 0.0),     # C = 563: several token tiles per expert
])
def test_backward_small(shape):
    T, d, F, E, c, bias0 = shape
    D = Small(T, d, F, E, c, seed=hash(shape) % 997, bias0=bias0)
    t, g, dout_bits = run_fwd_bwd(D, seed=1)
    ref = check_bwd(D, t, g, dout_bits, label=f"shape {shape}")
    if E == 1:
        assert np.all(g["dw_r"].cpu().numpy() == 0) or np.abs(g["dw_r"].cpu().numpy()).max() < 1e-6


def test_backward_with_z_loss():
    D = Small(512, 64, 128, 8, 1.0, seed=5)
    t, g, dout_bits = run_fwd_bwd(D, seed=2, z_beta=0.01)
    check_bwd(D, t, g, dout_bits, z_beta=0.01, label="z-loss")


def test_backward_zero_capacity_and_empty_batch():
    D = Small(256, 64, 128, 4, 1.0, seed=6)
    t, g, dout_bits = run_fwd_bwd(D, seed=3, C=0)
    assert np.all(g["dw1"].cpu().numpy() == 0) and np.all(g["dw2"].cpu().numpy() == 0)
    check_bwd(D, t, g, dout_bits, C=0, label="C = 0")
    # T = 0: every gradient is zero
    g0 = sw.layer_bwd_tensors(0, 64, 128, 4, 3)
    ws = g0.pop("ws")
    for v in g0.values():
        v.view(torch.uint8).fill_(0xFF)
    f = torch.zeros(4, dtype=torch.float32, device=DEV)
    acc = torch.zeros(4, dtype=torch.int32, device=DEV)
    e = torch.empty(0, dtype=torch.float32, device=DEV)
    buf = torch.zeros((4, 3, 64), dtype=torch.bfloat16, device=DEV)
    h = torch.zeros((4, 3, 128), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((4, 3, 64), dtype=torch.float32, device=DEV)
    fwd = dict(accepted=acc, f=f, buf=buf, h=h, y=y)
    b = sw.make_layer_bwd_args(fwd, None, D.w_r, D.w1, D.w2, None, g0, 0, 64, 128, 4, 3, 0.01)
    sw.switch_layer_bwd(b, ws)
    for name in ("dw_r", "db_r", "dw1", "dw2"):
        assert torch.count_nonzero(g0[name]).item() == 0, name


@pytest.mark.parametrize("ci", [1, 2, 3, 4, 5])
def test_backward_layer_configs(ci):
    """The five layer shapes: every gradient in full, except at 2048 experts,
    whose fp64 weight gradients alone would take 34 GB of host memory: there
    dW1 and dW2 are compared on 32 experts (the fullest, the emptiest, the
    first, the last and 28 drawn at random) and dx, dz, dgate, dW_r and db_r
    in full."""
    D = DeviceInputs(workloads.CONFIGS[ci])
    say(f"backward cfg{ci}: run")
    t, g, dout_bits = run_fwd_bwd(D, seed=10 + ci)
    dw_experts = None
    if D.cfg.E * D.cfg.d * D.cfg.d_ff >= (1 << 31):
        acc = t["accepted"].cpu().numpy()
        rng = np.random.default_rng(50 + ci)
        dw_experts = np.unique(np.concatenate([[0, D.cfg.E - 1, np.argmax(acc), np.argmin(acc)],
                                               rng.choice(D.cfg.E, 28, replace=False)]))
    check_bwd(D, t, g, dout_bits, label=f"cfg{ci}", dw_experts=dw_experts)
    # determinism: a second backward is bitwise equal
    g2 = sw.layer_bwd_tensors(D.cfg.T, D.cfg.d, D.cfg.d_ff, D.cfg.E, D.C, inspect=True)
    ws = g2.pop("ws")
    b = sw.make_layer_bwd_args(t, D.x, D.w_r, D.w1, D.w2, bits_to_dev(dout_bits), g2, D.cfg.T, D.cfg.d, D.cfg.d_ff,
                               D.cfg.E, D.C, D.cfg.alpha)
    sw.switch_layer_bwd(b, ws)
    for name in ("dx", "dw_r", "db_r", "dw1", "dw2", "dz"):
        assert torch.equal(g[name], g2[name]), name
        del g2[name]
    del D, t, g, g2
    torch.cuda.empty_cache()
