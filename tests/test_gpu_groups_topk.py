"""GPU parity of routing groups and top-k choices (the extended entry points)
against the fp64 oracle, through the C ABI.

Integer and copy results (choices, in-group positions, keep masks, buffer
rows, per-group counts, slot tables, the dispatch buffer) must be bit-exact;
floating-point results meet the tolerances in tests/gpu_helpers.py.  With
one group and k = 1 the extended layer must equal the Switch layer bit for
bit.
"""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_order_amd as sw
import workloads
from oracle import switch_oracle as so
from tests.gpu_helpers import (AUX_REL, GRAD_REL, MARGIN, DeviceInputs, assert_branch_close, assert_residual_close,
                               bits_to_dev, dev_bits, dev_to_f32, f32_dev, i32_dev, rel_fro, sample_kept_tokens, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def ws_tensor(nbytes):
    return torch.empty(max(256, nbytes), dtype=torch.uint8, device=DEV)


def poison(t):
    for v in t.values():
        if isinstance(v, torch.Tensor):
            v.view(torch.uint8).fill_(0xFF)


def ngroups(T, G):
    return 1 if G in (0, T) else T // G


def topk_near(z: np.ndarray, k: int) -> np.ndarray:
    """Tokens whose choice list depends on a logit gap <= MARGIN (any gap
    between consecutive values among the k + 1 largest)."""
    s = -np.sort(-z, axis=1)[:, :min(k + 1, z.shape[1])]
    if s.shape[1] < 2:
        return np.zeros(z.shape[0], bool)
    return np.any(np.diff(-s, axis=1) <= MARGIN, axis=1)


def oracle_branch_topk(inp, tokens, expert, gate, keep):
    """sum over kept choices of gate * expert_e(x_t), one expert at a time."""
    out = np.zeros((tokens.size, inp.cfg.d))
    k = expert.shape[1]
    for i in range(k):
        sel_all = np.flatnonzero(keep[tokens, i])
        for e in np.unique(expert[tokens[sel_all], i]):
            sel = sel_all[expert[tokens[sel_all], i] == e]
            out[sel] += gate[tokens[sel], i, None] * so.expert_rows(inp.x[tokens[sel]], inp.w1(e), inp.w2(e))
    return out


# ------------------------------------------------------------ inputs
_CACHE = {}


# extra layer shapes by name: (T, d, d_ff, E, c)
CUSTOM = {"g64": (4096, 256, 512, 64, 1.0)}   # 4 groups of 1024 x 16 rows: 64 rows per expert, the fused FFN


def inputs(ci):
    """A config's inputs, generated once per session (the 2048-expert config
    without its expert weights: only its routing and dispatch are tested here)."""
    if ci not in _CACHE:
        if ci in CUSTOM:
            _CACHE[ci] = DeviceInputs(workloads.custom_config(*CUSTOM[ci], index=3000))
        else:
            _CACHE[ci] = DeviceInputs(workloads.CONFIGS[ci], with_experts=ci != 5)
    return _CACHE[ci]


def small(T, E):
    """Tie-heavy inputs are drawn only where the oracle sorts them quickly."""
    return T * E <= (1 << 25)


def z32(D):
    """The oracle's logits rounded to fp32: the values a dispatch-only run feeds."""
    if not hasattr(D, "_z32"):
        D._z32 = D.z.astype(np.float32)
    return D._z32


# ------------------------------------------------------------ routing
def run_route_ex(D, k, G, logits_in=None):
    cfg = D.cfg
    T, E = cfg.T, cfg.E
    ng = ngroups(T, G)
    t = dict(expert=torch.empty((T, k), dtype=torch.int32, device=DEV),
             gate=torch.empty((T, k), dtype=torch.float32, device=DEV),
             lse=torch.empty(T, dtype=torch.float32, device=DEV),
             prob_sum=torch.empty((ng, E), dtype=torch.float32, device=DEV))
    poison(t)
    ws = ws_tensor(sw.switch_route_workspace_bytes(T, cfg.d, E))
    sw.switch_route_ex(D.x, D.w_r, D.b_r, logits_in, T, cfg.d, E, k, G, None, t["expert"], t["gate"], t["lse"],
                       t["prob_sum"], ws)
    return t


@pytest.mark.parametrize("ci,k,G", [(1, 2, 128), (1, 4, 64), (3, 2, 2048), (4, 2, 4096), (2, 3, 0)])
def test_route_ex_given_logits(ci, k, G):
    """Given fp32 logits the choices are bit-exact, including tie-heavy rows."""
    D = inputs(ci)
    cfg = D.cfg
    say(f"route_ex given logits cfg{ci} k={k} G={G}")
    for kind in ("oracle", "ties"):
        if kind == "oracle":
            z = z32(D)
        else:
            z = (np.random.default_rng(50 + ci).integers(-3, 4, (cfg.T, cfg.E)) / 4).astype(np.float32)
        t = run_route_ex(D, k, G, logits_in=f32_dev(z))
        r = so.softmax_topk(z.astype(np.float64), k)
        np.testing.assert_array_equal(t["expert"].cpu().numpy(), r.expert)
        np.testing.assert_allclose(t["gate"].cpu().numpy(), r.gate, rtol=2e-6, atol=1e-30)
        np.testing.assert_allclose(t["lse"].cpu().numpy(), r.lse, rtol=1e-6, atol=1e-6)
        Gt = cfg.T if G == 0 else G
        ps = r.p.reshape(-1, Gt, cfg.E).sum(axis=1)
        np.testing.assert_allclose(t["prob_sum"].cpu().numpy(), ps, rtol=AUX_REL, atol=1e-7 * Gt)
        del t


@pytest.mark.parametrize("ci,k,G", [(1, 2, 128), (2, 2, 2048), (3, 2, 64), (5, 2, 4096)])
def test_route_ex_gemm(ci, k, G):
    """Router GEMM (fused for E <= 256, two-pass above) with k choices: ids
    bit-exact away from near ties, gates and per-group sums within tolerance."""
    D = inputs(ci)
    cfg = D.cfg
    say(f"route_ex gemm cfg{ci} k={k} G={G}")
    t = run_route_ex(D, k, G)
    r = so.softmax_topk(D.z, k)
    near = topk_near(D.z, k)
    e_dev = t["expert"].cpu().numpy()
    np.testing.assert_array_equal(e_dev[~near], r.expert[~near])
    e_res = np.where(near[:, None], e_dev, r.expert)
    gate_ref = np.take_along_axis(r.p, e_res, axis=1)
    np.testing.assert_allclose(t["gate"].cpu().numpy(), gate_ref, rtol=AUX_REL, atol=1e-12)
    Gt = cfg.T if G == 0 else G
    ps = r.p.reshape(-1, Gt, cfg.E).sum(axis=1)
    np.testing.assert_allclose(t["prob_sum"].cpu().numpy(), ps, rtol=AUX_REL, atol=1e-7 * Gt)
    say(f"route_ex gemm cfg{ci}: near ties {int(near.sum())}")


# ------------------------------------------------------------ dispatch
def run_dispatch_ex(D, expert_dev, k, G, C, priority):
    cfg = D.cfg
    T, E, d = cfg.T, cfg.E, cfg.d
    ng = ngroups(T, G)
    rows = ng * C if T else 0
    t = dict(position=torch.empty((T, k), dtype=torch.int32, device=DEV),
             keep=torch.empty((T, k), dtype=torch.uint8, device=DEV),
             slot=torch.empty((T, k), dtype=torch.int32, device=DEV),
             counts=torch.empty((ng, E), dtype=torch.int32, device=DEV),
             accepted=torch.empty((ng, E), dtype=torch.int32, device=DEV),
             accepted_total=torch.empty(E, dtype=torch.int32, device=DEV),
             slot_token=torch.empty((E, rows), dtype=torch.int32, device=DEV),
             buf=torch.empty((E, rows, d), dtype=torch.bfloat16, device=DEV))
    poison(t)
    ws = ws_tensor(sw.switch_dispatch_workspace_bytes_ex(T, E, k, G))
    sw.switch_dispatch_ex(D.x, expert_dev, T, d, E, k, G, C, priority, t["position"], t["keep"], t["slot"],
                          t["counts"], t["accepted"], t["accepted_total"], t["slot_token"], t["buf"], ws)
    return t


def check_dispatch_ex(t, D, expert_ref, G, C, priority):
    cfg = D.cfg
    Gt = cfg.T if G == 0 else G
    sl = so.slot_scan_grouped(expert_ref, cfg.E, Gt, C, "rank" if priority else "token")
    np.testing.assert_array_equal(t["position"].cpu().numpy(), sl.position)
    np.testing.assert_array_equal(t["keep"].cpu().numpy().astype(bool), sl.keep)
    np.testing.assert_array_equal(t["slot"].cpu().numpy(), sl.slot)
    np.testing.assert_array_equal(t["counts"].cpu().numpy(), sl.counts)
    np.testing.assert_array_equal(t["accepted"].cpu().numpy(), sl.accepted)
    np.testing.assert_array_equal(t["accepted_total"].cpu().numpy(), sl.accepted_total)
    np.testing.assert_array_equal(t["slot_token"].cpu().numpy(), sl.slot_token)
    buf_bits = dev_bits(t["buf"])
    filled = sl.slot_token >= 0
    np.testing.assert_array_equal(buf_bits[filled], D.inp.x_bits[sl.slot_token[filled]])
    assert np.all(buf_bits[~filled] == 0), "empty rows must be +0.0"
    return sl


DISPATCH_CASES = [
    # (config, k, tokens per group (0: one group), capacity factor, priority)
    (1, 1, 64, 1.25, 0),     # scan tiles of 64
    (1, 2, 64, 1.25, 1),     # tiles of 128, rank order
    (1, 2, 128, 1.0, 0),     # tiles of 256
    (1, 2, 0, 1.0, 1),       # one group, rank order
    (1, 3, 0, 0.5, 0),       # one group, k = 3, ragged last tile
    (2, 2, 2048, 1.0, 0),
    (2, 2, 2048, 1.0, 1),
    (2, 1, 64, 1.0, 0),      # p5's 64-row groups at the Switch-Base shape: C_g = 1
    (3, 2, 4096, 1.0, 1),    # congested router
    (5, 2, 4096, 1.0, 0),    # 2048 experts
]


@pytest.mark.parametrize("ci,k,G,c,priority", DISPATCH_CASES)
def test_dispatch_ex_bit_exact(ci, k, G, c, priority):
    D = inputs(ci)
    cfg = D.cfg
    Gt = cfg.T if G == 0 else G
    C = so.group_capacity(Gt, cfg.E, c, k)
    say(f"dispatch_ex cfg{ci} k={k} G={G} C={C} priority={priority}")
    for kind in ("oracle", "ties") if small(cfg.T, cfg.E) else ("oracle",):
        if kind == "oracle":
            z = z32(D).astype(np.float64)
        else:
            z = np.random.default_rng(60 + ci).integers(-3, 4, (cfg.T, cfg.E)) / 4.0
        e_ref = so.softmax_topk(z, k).expert
        t = run_dispatch_ex(D, i32_dev(e_ref), k, G, C, priority)
        check_dispatch_ex(t, D, e_ref, G, C, priority)
        del t


def test_dispatch_ex_group_of_192_tokens():
    """A group size that is a multiple of 64 but not of 128: tiles of 64 (k = 1)
    and 128 (k = 2), three of them per group."""
    cfg = workloads.custom_config(576, 64, 128, 6, 1.0, index=1201)

    class Dv:
        pass
    D = Dv()
    D.cfg, D.inp = cfg, workloads.make_layer_inputs(cfg, with_experts=False)
    D.x = bits_to_dev(D.inp.x_bits)
    z = so.router_logits(D.inp.x, D.inp.w_r, D.inp.b_r).astype(np.float32).astype(np.float64)
    for k in (1, 2):
        for pr in (0, 1):
            e_ref = so.softmax_topk(z, k).expert
            C = so.group_capacity(192, 6, 1.0, k)
            t = run_dispatch_ex(D, i32_dev(e_ref), k, 192, C, pr)
            check_dispatch_ex(t, D, e_ref, 192, C, pr)


# ------------------------------------------------------------ combine and aux
@pytest.mark.parametrize("ci,k,G", [(1, 2, 128), (2, 2, 2048)])
def test_combine_ex(ci, k, G):
    D = inputs(ci)
    cfg = D.cfg
    T, E, d = cfg.T, cfg.E, cfg.d
    C = so.group_capacity(G, E, cfg.c, k)
    r = so.softmax_topk(z32(D).astype(np.float64), k)
    sl = so.slot_scan_grouped(r.expert, E, G, C)
    rows = (T // G) * C
    y = np.random.default_rng(70 + ci).standard_normal((E, rows, d)).astype(np.float32)
    gate = r.gate.astype(np.float32)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    for residual in (None, D.x):
        out.view(torch.uint8).fill_(0xFF)
        sw.switch_combine_ex(f32_dev(y), i32_dev(r.expert), i32_dev(sl.slot),
                             torch.from_numpy(sl.keep.astype(np.uint8)).to(DEV), f32_dev(gate), residual, T, d, E, k,
                             rows, out)
        ref = so.combine_topk(y.astype(np.float64), r.expert, sl.slot, sl.keep, gate.astype(np.float64), None)
        ob = dev_bits(out)
        none = ~sl.keep.any(axis=1)
        some = np.flatnonzero(~none)
        if residual is None:
            assert np.all(ob[none] == 0)
            assert_branch_close(workloads.bf16_bits_to_f32(ob)[some], ref[some], "combine_ex branch")
        else:
            np.testing.assert_array_equal(ob[none], D.inp.x_bits[none])
            assert_residual_close(ob[some], D.inp.x[some], ref[some], "combine_ex out")
        say(f"combine_ex cfg{ci}: {int(none.sum())} tokens with every choice dropped")


@pytest.mark.parametrize("ci,k,G", [(1, 2, 64), (4, 2, 4096), (3, 1, 1024)])
def test_aux_loss_ex(ci, k, G):
    D = inputs(ci)
    cfg = D.cfg
    T, E = cfg.T, cfg.E
    z = z32(D).astype(np.float64)
    r = so.softmax_topk(z, k)
    counts = so.slot_scan_grouped(r.expert, E, G, 1 << 20).counts
    ps = r.p.reshape(-1, G, E).sum(axis=1)
    ref = so.aux_loss_grouped(counts, r.p, G, k, cfg.alpha)
    ng = T // G
    f = torch.empty((ng, E), dtype=torch.float32, device=DEV)
    P = torch.empty((ng, E), dtype=torch.float32, device=DEV)
    loss = torch.empty(1, dtype=torch.float32, device=DEV)
    g = torch.empty((T, E), dtype=torch.float32, device=DEV)
    sw.switch_aux_loss_ex(i32_dev(counts), f32_dev(ps), f32_dev(z.astype(np.float32)), f32_dev(r.lse), T, E, k, G,
                          cfg.alpha, f, P, loss, g)
    np.testing.assert_allclose(f.cpu().numpy(), ref.f, rtol=1e-7)
    np.testing.assert_allclose(P.cpu().numpy(), ref.P, rtol=AUX_REL, atol=1e-9)
    assert abs(loss.item() - ref.loss) <= AUX_REL * abs(ref.loss)
    gd = g.cpu().numpy()
    assert rel_fro(gd, ref.dlogits) <= GRAD_REL
    assert np.abs(gd - ref.dlogits).max() <= GRAD_REL * np.abs(ref.dlogits).max()


# ------------------------------------------------------------ the layer
def run_layer_ex(D, k, G, C, priority, residual, want_grad=False, inspect=True):
    cfg = D.cfg
    t = sw.layer_tensors(cfg.T, cfg.d, cfg.d_ff, cfg.E, C, dlogits=want_grad, inspect=inspect, k=k, group=G)
    ws = t.pop("ws")
    poison(t)
    a = sw.make_layer_args(D.x, D.w_r, D.b_r, D.w1, D.w2, t, cfg.T, cfg.d, cfg.d_ff, cfg.E, C, cfg.alpha,
                           residual=residual, k=k, group=G, priority=priority)
    sw.switch_layer_fwd(a, ws)
    torch.cuda.synchronize()
    return t


LAYER_CASES = [(1, 2, 128, 0), (1, 2, 64, 1), (2, 2, 2048, 0), (3, 2, 4096, 1), (4, 2, 8192, 0)]


@pytest.mark.parametrize("ci,k,G,priority", LAYER_CASES)
def test_layer_ex_end_to_end(ci, k, G, priority):
    D = inputs(ci)
    cfg = D.cfg
    T, E = cfg.T, cfg.E
    C = so.group_capacity(G, E, cfg.c, k)
    pr = "rank" if priority else "token"
    say(f"layer_ex cfg{ci} k={k} G={G} C={C} {pr}: run")
    t = run_layer_ex(D, k, G, C, priority, residual=False, want_grad=cfg.want_grad)
    r = so.softmax_topk(D.z, k)
    near = topk_near(D.z, k)
    e_dev = t["expert"].cpu().numpy().reshape(T, k)
    np.testing.assert_array_equal(e_dev[~near], r.expert[~near])
    e_res = np.where(near[:, None], e_dev, r.expert)
    gate_ref = np.take_along_axis(r.p, e_res, axis=1)
    sl = so.slot_scan_grouped(e_res, E, G, C, pr)
    shp = lambda a: a.cpu().numpy().reshape(T, k)
    np.testing.assert_array_equal(shp(t["position"]), sl.position)
    np.testing.assert_array_equal(shp(t["keep"]).astype(bool), sl.keep)
    np.testing.assert_array_equal(shp(t["slot"]), sl.slot)
    np.testing.assert_array_equal(t["counts"].cpu().numpy(), sl.counts)
    np.testing.assert_array_equal(t["accepted"].cpu().numpy(), sl.accepted)
    np.testing.assert_array_equal(t["accepted_total"].cpu().numpy(), sl.accepted_total)
    np.testing.assert_array_equal(t["slot_token"].cpu().numpy(), sl.slot_token)
    np.testing.assert_allclose(shp(t["gate"]), gate_ref, rtol=AUX_REL, atol=1e-12)
    aux = so.aux_loss_grouped(sl.counts, r.p, G, k, cfg.alpha)
    np.testing.assert_allclose(t["f"].cpu().numpy(), aux.f, rtol=1e-7)
    np.testing.assert_allclose(t["P"].cpu().numpy(), aux.P, rtol=AUX_REL, atol=1e-9)
    assert abs(t["loss"].item() - aux.loss) <= AUX_REL * abs(aux.loss)
    if cfg.want_grad:
        g = t["dlogits"].cpu().numpy()
        assert rel_fro(g, aux.dlogits) <= GRAD_REL
    kept_any = sl.keep.any(axis=1)
    ob = dev_bits(t["out"])
    assert np.all(ob[~kept_any] == 0), "tokens with every choice dropped carry a zero branch"
    toks = sample_kept_tokens(kept_any, 100000 if T <= 4096 else 512, seed=ci)
    say(f"layer_ex cfg{ci}: oracle branch on {toks.size} tokens")
    ref = oracle_branch_topk(D.inp, toks, e_res, gate_ref, sl.keep)
    rf, mr = assert_branch_close(workloads.bf16_bits_to_f32(ob)[toks], ref, f"layer_ex cfg{ci} branch")
    say(f"layer_ex cfg{ci}: rel fro {rf:.2e}, max/rms {mr:.2e}, kept choices {int(sl.keep.sum())}/{T * k}, "
        f"near ties {int(near.sum())}")
    t2 = run_layer_ex(D, k, G, C, priority, residual=True, inspect=False)
    ob2 = dev_bits(t2["out"])
    np.testing.assert_array_equal(ob2[~kept_any], D.inp.x_bits[~kept_any])
    assert_residual_close(ob2[toks], D.inp.x[toks], ref, f"layer_ex cfg{ci} residual out")


# (config, k, group, priority) of the layer with no buf, slot_token or y kept
NO_BUF_CASES = [(2, 2, 0, 0), (2, 1, 2048, 0), (3, 2, 0, 1), (4, 2, 8192, 0), ("g64", 1, 1024, 0)]


@pytest.mark.parametrize("ci,k,G,priority", NO_BUF_CASES)
def test_layer_ex_no_buf_branch(ci, k, G, priority):
    """The extended layer as a caller that keeps no intermediates runs it: the
    first expert GEMM gathers its token rows from x through the workspace slot
    table, and with k = 1 the second GEMM writes the combine.  Branch mode,
    every token with a kept choice against the oracle at the stated
    tolerance; tokens with every choice dropped carry exactly 0."""
    D = inputs(ci)
    cfg = D.cfg
    T, E = cfg.T, cfg.E
    C = so.group_capacity(G or T, E, cfg.c, k)
    pr = "rank" if priority else "token"
    say(f"layer_ex no-buf cfg{ci} k={k} G={G} C={C} {pr}: run")
    sw.switch_profile_enable(True)
    try:
        t = run_layer_ex(D, k, G, C, priority, residual=False, inspect=False)
    finally:
        names = [n for n, _ in sw.switch_profile_collect()]
        sw.switch_profile_enable(False)
    # k = 1 with at most 64 buffer rows per expert (d, d_ff multiples of 256,
    # d <= 1024): both expert products in one kernel
    rows = ngroups(T, G) * C
    fused = k == 1 and rows <= 64 and cfg.d % 256 == 0 and cfg.d <= 1024 and cfg.d_ff % 256 == 0
    assert ("expert_ffn_fused" in names) == fused, names
    r = so.softmax_topk(D.z, k)
    near = topk_near(D.z, k)
    e_dev = t["expert"].cpu().numpy().reshape(T, k)
    np.testing.assert_array_equal(e_dev[~near], r.expert[~near])
    e_res = np.where(near[:, None], e_dev, r.expert)
    gate_ref = np.take_along_axis(r.p, e_res, axis=1)
    sl = so.slot_scan_grouped(e_res, E, G or T, C, pr)
    shp = lambda a: a.cpu().numpy().reshape(T, k)
    np.testing.assert_array_equal(shp(t["position"]), sl.position)
    np.testing.assert_array_equal(shp(t["keep"]).astype(bool), sl.keep)
    if "slot" in t:
        np.testing.assert_array_equal(shp(t["slot"]), sl.slot)
    np.testing.assert_array_equal(t["counts"].cpu().numpy().reshape(sl.counts.shape), sl.counts)
    kept_any = sl.keep.any(axis=1)
    ob = dev_bits(t["out"])
    assert np.all(ob[~kept_any] == 0), "tokens with every choice dropped carry a zero branch"
    toks = np.flatnonzero(kept_any)
    say(f"layer_ex no-buf cfg{ci}: oracle branch on all {toks.size} tokens with a kept choice")
    ref = oracle_branch_topk(D.inp, toks, e_res, gate_ref, sl.keep)
    rf, mr = assert_branch_close(workloads.bf16_bits_to_f32(ob[toks]), ref, f"layer_ex no-buf cfg{ci} branch")
    say(f"layer_ex no-buf cfg{ci}: rel fro {rf:.2e}, max/rms {mr:.2e}, kept choices {int(sl.keep.sum())}/{T * k}")


@pytest.mark.parametrize("ci", [1, 2])
def test_layer_ex_one_group_top1_is_the_switch_layer(ci):
    """k = 1 with group 0 or group T: the extended layer equals the Switch layer bit for bit."""
    D = inputs(ci)
    cfg = D.cfg
    base = run_layer_ex(D, 1, 0, D.C, 0, residual=True)
    for G, pr in ((cfg.T, 0), (0, 1)):
        t = run_layer_ex(D, 1, G, D.C, pr, residual=True)
        for name in ("out", "expert", "gate", "position", "keep", "counts", "accepted", "f", "P", "loss",
                     "slot_token", "buf"):
            assert torch.equal(t[name], base[name]), name
    # and against the default arguments (k and group zero)
    t0 = sw.layer_tensors(cfg.T, cfg.d, cfg.d_ff, cfg.E, D.C, inspect=True)
    ws = t0.pop("ws")
    a = sw.make_layer_args(D.x, D.w_r, D.b_r, D.w1, D.w2, t0, cfg.T, cfg.d, cfg.d_ff, cfg.E, D.C, cfg.alpha,
                           residual=True, k=0, group=0)
    sw.switch_layer_fwd(a, ws)
    assert torch.equal(t0["out"], base["out"]) and torch.equal(t0["loss"], base["loss"])


def test_layer_ex_empty_batch_and_zero_capacity():
    cfg = workloads.custom_config(256, 64, 128, 4, 1.0, index=1202)

    class Dv:
        pass
    D = Dv()
    D.cfg, D.inp = cfg, workloads.make_layer_inputs(cfg)
    D.x, D.w_r, D.b_r = bits_to_dev(D.inp.x_bits), f32_dev(D.inp.w_r), f32_dev(D.inp.b_r)
    D.w1, D.w2 = bits_to_dev(D.inp.w1_bits), bits_to_dev(D.inp.w2_bits)
    # C = 0 per group: every choice dropped, out = x bit for bit, statistics unchanged
    t = run_layer_ex(D, 2, 64, 0, 0, residual=True)
    assert not t["keep"].any()
    np.testing.assert_array_equal(dev_bits(t["out"]), D.inp.x_bits)
    r = so.softmax_topk(so.router_logits(D.inp.x, D.inp.w_r, D.inp.b_r), 2)
    sl = so.slot_scan_grouped(r.expert, 4, 64, 0)
    np.testing.assert_array_equal(t["counts"].cpu().numpy(), sl.counts)
    # T = 0 with groups: zero groups, nothing written, loss 0
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    t0 = sw.layer_tensors(0, 64, 128, 4, 3, k=2, group=64)
    ws = t0.pop("ws")
    a = sw.make_layer_args(e, D.w_r, D.b_r, D.w1, D.w2, t0, 0, 64, 128, 4, 3, 0.01, k=2, group=64)
    sw.switch_layer_fwd(a, ws)
    assert t0["loss"].item() == 0.0
