"""GPU parity of the layer backward with routing groups and top-k choices
(switch_layer_bwd with k and group set) against the fp64 oracle.

The forward runs on the device (switch_layer_fwd with the same k, group and
priority, its saved tensors requested); the oracle backward is fed the
device's choices, which the gradient holds fixed.  Integer results of the
forward that the backward reads (keep masks, buffer rows) must equal the
oracle's exactly.  Tolerances are those of the Switch-layer backward
(tests/test_gpu_backward.py), applied per (token, choice): dgate_ti and dz
carry the bf16 error of y[e_ti, s_ti], the weight and router gradients meet
tests/gpu_helpers.py's gradient bound, dx one bf16 ulp plus the branch
tolerance.
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
        self.cfg = workloads.custom_config(T, d, F, E, c, index=1400 + seed)
        self.inp = workloads.make_layer_inputs(self.cfg)
        self.inp.b_r = self.inp.b_r.copy()
        self.inp.b_r[0] += bias0
        self.x, self.w_r, self.b_r = bits_to_dev(self.inp.x_bits), f32_dev(self.inp.w_r), f32_dev(self.inp.b_r)
        self.w1, self.w2 = bits_to_dev(self.inp.w1_bits), bits_to_dev(self.inp.w2_bits)


def run_fwd_bwd(D, k, G, Cg, priority, seed, z_beta=0.0):
    cfg = D.cfg
    T, d, F, E = cfg.T, cfg.d, cfg.d_ff, cfg.E
    t = sw.layer_tensors(T, d, F, E, Cg, for_backward=True, z_loss=z_beta > 0, k=k, group=G)
    ws = t.pop("ws")
    a = sw.make_layer_args(D.x, D.w_r, D.b_r, D.w1, D.w2, t, T, d, F, E, Cg, cfg.alpha, residual=True,
                           z_beta=z_beta, k=k, group=G, priority=priority)
    sw.switch_layer_fwd(a, ws)
    dout_bits = workloads.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((T, d)).astype(np.float32))
    dout = bits_to_dev(dout_bits)
    g = sw.layer_bwd_tensors(T, d, F, E, Cg, inspect=True, k=k, group=G)
    gws = g.pop("ws")
    for v in g.values():
        v.view(torch.uint8).fill_(0xFF)
    b = sw.make_layer_bwd_args(t, D.x, D.w_r, D.w1, D.w2, dout, g, T, d, F, E, Cg, cfg.alpha, z_beta=z_beta,
                               k=k, group=G)
    sw.switch_layer_bwd(b, gws)
    # again with the identity term of dx left out (its branch alone)
    dxb = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    b2 = sw.make_layer_bwd_args(t, D.x, D.w_r, D.w1, D.w2, dout, dict(g, dx=dxb), T, d, F, E, Cg, cfg.alpha,
                                z_beta=z_beta, k=k, group=G, dx_branch_only=True)
    sw.switch_layer_bwd(b2, gws)
    g["dx_branch"] = dxb
    torch.cuda.synchronize()
    return t, g, dout_bits, dout


def check_bwd_ex(D, t, g, dout_bits, k, G, Cg, priority, z_beta=0.0, label=""):
    cfg = D.cfg
    T, E = cfg.T, cfg.E
    Gt = T if G == 0 else G
    pr = "rank" if priority else "token"
    e_dev = t["expert"].cpu().numpy().astype(np.int64).reshape(T, k)
    dout = workloads.bf16_bits_to_f32(dout_bits).astype(np.float64)
    say(f"backward_ex {label}: oracle")
    L = so.layer_forward_grouped(D.inp.x, D.inp.w_r, D.inp.b_r, D.inp.w1, D.inp.w2, cfg.c, cfg.alpha, k=k, G=Gt,
                                 priority=pr, expert_override=e_dev, Cg=Cg)
    shp = lambda a: a.cpu().numpy().reshape(T, k)
    keep = shp(t["keep"]).astype(bool)
    np.testing.assert_array_equal(keep, L.slots.keep)
    slot_dev = shp(t["slot"]) if "slot" in t else shp(t["position"])
    np.testing.assert_array_equal(np.where(keep, slot_dev, -1), L.slots.slot)
    # the ReLU derivative: the device's decision within rounding of zero (as in
    # the Switch-layer backward test), the oracle's [a > 0] elsewhere
    h_dev = dev_bits(t["h"]) if Cg > 0 else None
    n_near = [0]

    def relu_active(e, a):
        dev = (h_dev[e, :a.shape[0]] & 0x7FFF) != 0
        rms = np.sqrt(np.mean(a ** 2)) if a.size else 0.0
        near = np.abs(a) <= 1e-4 * rms
        np.testing.assert_array_equal(dev[~near], (a > 0)[~near], err_msg=f"{label} ReLU mask of expert {e}")
        n_near[0] += int(near.sum())
        return np.where(near, dev, a > 0)

    ref = so.layer_backward_grouped(D.inp.x, D.inp.w_r, D.inp.b_r, D.inp.w1, D.inp.w2, cfg.c, cfg.alpha, dout, k=k,
                                    G=Gt, priority=pr, beta=z_beta, Cg=Cg, forward=L, relu_active=relu_active)
    say(f"backward_ex {label}: {n_near[0]} pre-activations within rounding of zero")
    # dgate_ti = <dout_t, y[e_ti, s_ti]>: |error| <= 2^-7 |dout_t| |y[e_ti, s_ti]|
    y_ch = np.zeros(keep.shape + (cfg.d,))
    ti, ci = np.nonzero(keep)
    y_ch[ti, ci] = L.y[e_dev[ti, ci], L.slots.slot[ti, ci]]
    bound = 2.0 ** -7 * np.linalg.norm(dout, axis=1)[:, None] * np.linalg.norm(y_ch, axis=2)
    dg = g["dgate"].cpu().numpy().astype(np.float64).reshape(T, k)
    assert np.all(dg[~keep] == 0), "dropped choices carry no gate gradient"
    err = np.abs(dg - ref.dgate)
    assert np.all(err <= bound + 1e-6 * np.abs(ref.dgate) + 1e-30), f"{label} dgate: worst {np.max(err - bound):.3e}"
    dz = g["dz"].cpu().numpy().astype(np.float64)
    zb = np.zeros((T, E))
    for i in range(k):
        onehot = np.zeros((T, E))
        onehot[np.arange(T), e_dev[:, i]] = 1.0
        zb += (2.0 * bound[:, i] * L.routing.gate[:, i])[:, None] * np.abs(onehot - L.routing.p)
    zerr = np.abs(dz - ref.dz)
    rms = np.sqrt(np.mean(ref.dz ** 2)) if ref.dz.size else 0.0
    bad = zerr > zb + 1e-2 * np.abs(ref.dz) + 1e-3 * rms + 1e-30
    assert not bad.any(), f"{label} dz: {int(bad.sum())} elements off"
    assert rel_fro(dz, ref.dz) <= 5e-3, f"{label} dz: relative Frobenius {rel_fro(dz, ref.dz):.3e}"
    assert_grad_close(g["db_r"].cpu().numpy(), ref.db_r, f"{label} db_r")
    assert_grad_close(g["dw_r"].cpu().numpy(), ref.dw_r, f"{label} dW_r")
    dw1 = g["dw1"].cpu().numpy()
    dw2 = g["dw2"].cpu().numpy()
    empty = L.slots.accepted_total == 0
    assert np.all(dw1[empty] == 0) and np.all(dw2[empty] == 0), "experts without rows get zero gradients"
    if (~empty).any():
        assert_grad_close(dw1, ref.dw1, f"{label} dW1")
        assert_grad_close(dw2, ref.dw2, f"{label} dW2")
    assert_residual_close(dev_bits(g["dx"]), dout, ref.dx - dout, f"{label} dx")
    # the branch of dx alone, at the gradient tolerance (two bf16 roundings: dy and dA)
    rf = assert_grad_close(workloads.bf16_bits_to_f32(dev_bits(g["dx_branch"])), ref.dx - dout, f"{label} dx branch")
    say(f"backward_ex {label}: ok, kept {int(keep.sum())}/{T * k} choices, dx branch rel fro {rf:.2e}")
    return ref


SMALL_CASES = [
    # (T, d, d_ff, E, c, k, tokens per group (0: one), priority, bias on expert 0)
    (512, 64, 128, 4, 1.25, 2, 128, 0, 2.0),     # hot expert, many dropped choices; transposed weight gradients
    (1024, 128, 192, 6, 1.0, 2, 256, 1, 0.0),    # rank order, K-major weight gradients, ragged d_ff tiles
    (768, 64, 128, 8, 1.0, 3, 0, 0, 0.0),        # one group, k = 3
    (640, 128, 128, 32, 1.0, 4, 64, 1, 1.0),     # k = 4, ten 64-row groups, the MFMA dx kernel
    (1024, 128, 256, 32, 1.25, 2, 0, 1, 0.0),    # one group, rank order, MFMA dx with two choices
    (1024, 128, 128, 32, 1.0, 1, 64, 0, 0.0),    # k = 1 in 64-row groups: C_g = 2
    (1000, 64, 128, 5, 0.5, 2, 0, 0, 0.0),       # ragged T (one group), half capacity
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "T{}_E{}_k{}_G{}_p{}".format(c[0], c[3], c[5], c[6], c[7]))
def test_backward_ex_small(case):
    T, d, F, E, c, k, G, priority, bias0 = case
    D = Small(T, d, F, E, c, seed=hash(case) % 997, bias0=bias0)
    Gt = T if G == 0 else G
    Cg = so.group_capacity(Gt, E, c, k)
    say(f"backward_ex {case}: C_g = {Cg}")
    t, g, dout_bits, _ = run_fwd_bwd(D, k, G, Cg, priority, seed=3)
    check_bwd_ex(D, t, g, dout_bits, k, G, Cg, priority, label=str(case))


def test_backward_ex_z_loss_and_one_group_k1_matches_plain():
    """z-loss with groups; and k = 1 with one group through the extended
    fields gives the Switch-layer backward bit for bit."""
    D = Small(512, 64, 128, 8, 1.0, seed=7)
    Cg = so.group_capacity(128, 8, 1.0, 2)
    t, g, dout_bits, _ = run_fwd_bwd(D, 2, 128, Cg, 0, seed=4, z_beta=0.02)
    check_bwd_ex(D, t, g, dout_bits, 2, 128, Cg, 0, z_beta=0.02, label="z-loss, k = 2, G = 128")
    C = so.capacity(512, 8, 1.0)
    t1, g1, _, dout1 = run_fwd_bwd(D, 1, 0, C, 0, seed=5)
    g0 = sw.layer_bwd_tensors(512, 64, 128, 8, C, inspect=True)
    ws0 = g0.pop("ws")
    b0 = sw.make_layer_bwd_args(t1, D.x, D.w_r, D.w1, D.w2, dout1, g0, 512, 64, 128, 8, C, D.cfg.alpha)
    b0.k, b0.group = 0, 0
    sw.switch_layer_bwd(b0, ws0)
    torch.cuda.synchronize()
    for name in ("dx", "dw_r", "db_r", "dw1", "dw2", "dz", "dgate"):
        assert torch.equal(g1[name], g0[name]), name


@pytest.mark.parametrize("ci,k,G,priority", [(2, 2, 2048, 0), (1, 2, 64, 1)])
def test_backward_ex_layer_configs(ci, k, G, priority):
    """Top-2 with routing groups at the layer shapes: full comparison."""
    D = DeviceInputs(workloads.CONFIGS[ci])
    cfg = D.cfg
    Cg = so.group_capacity(G, cfg.E, cfg.c, k)
    say(f"backward_ex cfg{ci} k={k} G={G} C_g={Cg}: run")
    t, g, dout_bits, _ = run_fwd_bwd(D, k, G, Cg, priority, seed=20 + ci)
    check_bwd_ex(D, t, g, dout_bits, k, G, Cg, priority, label=f"cfg{ci}")
    del D, t, g
    torch.cuda.empty_cache()
