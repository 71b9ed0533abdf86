"""Pins for the fp64 oracle: each function checks the oracle module `so`
against something other than itself (a value the pages print, a closed form,
a library routine, brute force) and raises AssertionError on a mismatch.

They take the oracle module as an argument so that tests/test_oracle_mutations.py
can run the same pins against copies of the oracle with planted mistakes.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pins.json")))


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_round(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def pin_two_expert_balance(so):
    """wq-win sec. 2: 2(0.72 + 0.02) = 1.48, balanced = 1 (alpha removed)."""
    g = GOLDEN["two_expert_balance"]
    # 9 tokens at (0.85, 0.15) and one at (0.35, 0.65): f = (0.9, 0.1), P = (0.8, 0.2)
    p = np.array([[0.85, 0.15]] * 9 + [[0.35, 0.65]])
    r = so.softmax_top1(np.log(p))
    counts = np.bincount(r.expert, minlength=2)
    aux = so.aux_loss(counts, r.p, g["alpha"])
    np.testing.assert_allclose(aux.f, g["f"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(aux.P, g["P"], rtol=1e-14)
    assert abs(aux.loss - g["expected_loss"]) < 1e-12, aux.loss
    pb = np.array([[0.75, 0.25]] * 5 + [[0.25, 0.75]] * 5)
    rb = so.softmax_top1(np.log(pb))
    auxb = so.aux_loss(np.bincount(rb.expert, minlength=2), rb.p, 1.0)
    assert abs(auxb.loss - g["balanced_loss"]) < 1e-12, auxb.loss


def pin_uniform_counterexample(so):
    """zffjzz 'minimal experiment': uniform rows all pick expert 0, loss stays 1;
    the gradient is the closed form (alpha E / T) p (f_j - sum_e f_e p_e)."""
    g = GOLDEN["uniform_rows_counterexample"]
    T, E = g["T"], g["E"]
    r = so.softmax_top1(np.zeros((T, E)))
    assert np.all(r.expert == g["expected_expert"])
    aux = so.aux_loss(np.bincount(r.expert, minlength=E), r.p, g["alpha"])
    np.testing.assert_array_equal(aux.f, g["expected_f"])
    np.testing.assert_allclose(aux.P, [0.25] * 4, rtol=1e-15)
    assert abs(aux.loss - g["expected_loss"]) < 1e-14
    a = 0.37
    aux = so.aux_loss(np.bincount(r.expert, minlength=E), r.p, a)
    c = a * E / T
    np.testing.assert_allclose(aux.dlogits[:, 0], c * 0.25 * 0.75, rtol=1e-13)
    np.testing.assert_allclose(aux.dlogits[:, 1:], -c * 0.25 * 0.25, rtol=1e-13)


def pin_uniform_capacity(so):
    """zffjzz 'minimal experiment': C = 20 at c = 1.25, 20 kept, 68.75 % overflow."""
    g = GOLDEN["uniform_rows_capacity"]
    T, E = g["T"], g["E"]
    C = so.capacity(T, E, g["c"])
    assert C == g["expected_C"], C
    r = so.softmax_top1(np.zeros((T, E)))
    s = so.slot_scan(r.expert, E, C)
    assert int(s.accepted.sum()) == g["expected_accepted_total"]
    np.testing.assert_array_equal(s.accepted, [20, 0, 0, 0])
    np.testing.assert_array_equal(s.keep, np.arange(T) < 20)
    assert abs((T - s.keep.sum()) / T - g["expected_overflow"]) < 1e-15


def pin_raw_load_capped(so):
    """zffjzz 'minimal experiment': [28,12,12,12] capped at 8 -> [8,8,8,8]; f keeps the raw load."""
    g = GOLDEN["raw_load_capped"]
    raw = g["raw"]
    expert = np.repeat(np.arange(4), raw)
    _rng(5).shuffle(expert)
    T = len(expert)
    C = so.capacity(T, 4, 0.5)
    assert C == g["C"]
    s = so.slot_scan(expert, 4, C)
    np.testing.assert_array_equal(s.accepted, g["expected_accepted"])
    np.testing.assert_array_equal(s.counts, raw)
    # the f statistic uses the raw choices, not the accepted ones
    z = np.where(np.arange(4)[None, :] == expert[:, None], 1.0, 0.0)
    r = so.softmax_top1(z)
    layer = so.layer_forward(np.zeros((T, 2)), None, None, np.zeros((4, 2, 2)), np.zeros((4, 2, 2)),
                             0.5, 1.0, logits=z)
    np.testing.assert_allclose(layer.aux.f, np.array(raw) / T, rtol=0, atol=0)
    assert np.all(r.expert == expert)


def pin_shift_invariance(so):
    """zffjzz 'minimal experiment': +100 on every score keeps p and the choice."""
    sh = GOLDEN["shift_invariance"]["shift"]
    z = _rng(1).standard_normal((257, 9))
    a, b = so.softmax_top1(z), so.softmax_top1(z + sh)
    np.testing.assert_array_equal(a.expert, b.expert)
    np.testing.assert_allclose(a.p, b.p, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b.lse - a.lse, sh, rtol=1e-13)


def pin_softmax_library(so):
    """Softmax and log-sum-exp against scipy.special on random rows, including huge logits."""
    z = _rng(2).standard_normal((300, 17)) * 30.0
    r = so.softmax_top1(z)
    np.testing.assert_allclose(r.p, scipy.special.softmax(z, axis=1), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(r.lse, scipy.special.logsumexp(z, axis=1), rtol=1e-14)
    np.testing.assert_allclose(r.p.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_array_equal(r.gate, r.p.max(axis=1))
    # lowest index among equal maxima
    zt = np.array([[1.0, 3.0, 3.0, 0.0], [2.0, 2.0, 2.0, 2.0], [0.0, 0.0, 0.0, 5.0]])
    np.testing.assert_array_equal(so.softmax_top1(zt).expert, [1, 0, 3])


def pin_gate_not_renormalised(so):
    """wq-win sec. 2: the selected probability 0.7 stays on the expert output."""
    pg = GOLDEN["gate_not_renormalised"]["p_selected"]
    rng = _rng(3)
    T, d, F = 6, 8, 12
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((2, F, d))
    w2 = rng.standard_normal((2, d, F))
    z = np.tile(np.log([pg, 1 - pg]), (T, 1))
    layer = so.layer_forward(x, None, None, w1, w2, 2.0, 0.01, logits=z)
    xt, w1t, w2t = (torch.from_numpy(a) for a in (x, w1[0], w2[0]))
    ffn = (torch.relu(xt @ w1t.T) @ w2t.T).numpy()
    np.testing.assert_allclose(layer.routing.gate, pg, rtol=1e-14)
    np.testing.assert_allclose(layer.branch, pg * ffn, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(layer.out, x + pg * ffn, rtol=1e-12, atol=1e-12)


def pin_local_overflow(so):
    """wq-win sec. 3: 100 tokens, 10 experts, c = 1: 30 tokens on one expert drop 20."""
    g = GOLDEN["local_overflow"]
    T, E = g["T"], g["E"]
    C = so.capacity(T, E, g["c"])
    assert C == g["expected_C"]
    others = np.repeat([0, 1, 2, 4, 5, 6, 7, 8, 9], [7, 8, 8, 8, 8, 8, 8, 8, 7])
    expert = np.concatenate([others, np.full(g["hot_tokens"], 3)])
    _rng(4).shuffle(expert)
    s = so.slot_scan(expert, E, C)
    assert int((~s.keep).sum()) == g["expected_dropped"]
    hot = np.flatnonzero(expert == 3)
    np.testing.assert_array_equal(s.keep[hot], np.arange(30) < 10)      # first ten in token order
    np.testing.assert_array_equal(s.position[hot], np.arange(30))
    assert s.accepted.sum() == 80 and s.counts.sum() == T


def pin_capacity_values(so):
    """C = ceil(c T / E) at the five layer shapes and at boundaries."""
    assert so.capacity(512, 4, 1.25) == 160
    assert so.capacity(16384, 128, 1.0) == 128
    assert so.capacity(16384, 64, 2.0) == 512
    assert so.capacity(32768, 128, 1.25) == 320
    assert so.capacity(65536, 2048, 1.0) == 32
    assert so.capacity(10, 3, 1.0) == 4           # 10/3 rounds up
    assert so.capacity(9, 3, 1.0) == 3            # exact stays exact
    assert so.capacity(64, 4, 0.0) == 0
    assert so.capacity(0, 4, 1.0) == 0
    assert so.capacity(30, 3, 0.1) == 2           # binary 0.1 is slightly above 1/10
    assert so.capacity(30, 3, 0.09375) == 1       # 0.09375 = 3/32 is exact


def pin_single_expert_is_dense_ffn(so):
    """E = 1: nothing dropped, p = 1, loss = alpha, G = 0, branch = the dense FFN (torch)."""
    rng = _rng(6)
    T, d, F = 40, 16, 24
    x = _bf16_round(rng.standard_normal((T, d)))
    w_r = rng.standard_normal((d, 1)).astype(np.float32)
    w1 = rng.standard_normal((1, F, d)) * 0.3
    w2 = rng.standard_normal((1, d, F)) * 0.3
    alpha = 0.01
    L = so.layer_forward(x, w_r, None, w1, w2, 1.0, alpha)
    assert L.C >= T and L.slots.keep.all()
    np.testing.assert_allclose(L.routing.p, 1.0, rtol=0, atol=0)
    assert abs(L.aux.loss - alpha) < 1e-15
    np.testing.assert_array_equal(L.aux.dlogits, 0.0)
    ref = torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(
        torch.from_numpy(np.asarray(x, np.float64)), torch.from_numpy(w1[0]))), torch.from_numpy(w2[0])).numpy()
    np.testing.assert_allclose(L.branch, ref, rtol=1e-12, atol=1e-12)


def _tiny_problem(seed, T, d, F, E):
    rng = _rng(seed)
    x = _bf16_round(rng.standard_normal((T, d)))
    w_r = (rng.standard_normal((d, E)) * 0.5).astype(np.float32)
    b_r = (rng.standard_normal(E) * 0.3).astype(np.float32)
    w1 = _bf16_round(rng.standard_normal((E, F, d)) * 0.2)
    w2 = _bf16_round(rng.standard_normal((E, d, F)) * 0.2)
    return x, w_r, b_r, w1, w2


def pin_no_drop_brute_force(so):
    """c >= E so C >= T: every token kept; branch_t = p_{t,e*} FFN_{e*}(x_t) token by token."""
    x, w_r, b_r, w1, w2 = _tiny_problem(7, 50, 12, 20, 5)
    L = so.layer_forward(x, w_r, b_r, w1, w2, 5.0, 0.01)
    assert L.C >= 50 and L.slots.keep.all()
    z = x.astype(np.float64) @ w_r.astype(np.float64) + b_r
    for t in range(50):
        e = int(np.argmax(z[t]))
        g = math.exp(z[t, e] - z[t].max()) / np.exp(z[t] - z[t].max()).sum()
        h = np.maximum(w1[e].astype(np.float64) @ x[t], 0)
        np.testing.assert_allclose(L.branch[t], g * (w2[e].astype(np.float64) @ h), rtol=1e-12, atol=1e-13)


def pin_zero_capacity(so):
    """c = 0: C = 0, every token dropped, out = x exactly, f and P as with c = 1."""
    x, w_r, b_r, w1, w2 = _tiny_problem(8, 33, 8, 16, 3)
    L0 = so.layer_forward(x, w_r, b_r, w1, w2, 0.0, 0.01)
    L1 = so.layer_forward(x, w_r, b_r, w1, w2, 1.0, 0.01)
    assert L0.C == 0 and not L0.slots.keep.any()
    np.testing.assert_array_equal(L0.out, x.astype(np.float64))
    np.testing.assert_array_equal(L0.branch, 0.0)
    np.testing.assert_array_equal(L0.aux.f, L1.aux.f)
    np.testing.assert_array_equal(L0.aux.P, L1.aux.P)
    assert L0.buf.shape[1] == 0


def pin_invariants(so):
    """sum f = 1, sum P = 1, rows of G sum to 0, uniform f gives G = 0, slots are 0..accepted-1 in token order."""
    x, w_r, b_r, w1, w2 = _tiny_problem(9, 97, 8, 16, 6)
    for c in (0.5, 1.0, 1.7):
        L = so.layer_forward(x, w_r, b_r, w1, w2, c, 0.3)
        assert abs(L.aux.f.sum() - 1) < 1e-15 and abs(L.aux.P.sum() - 1) < 1e-14
        np.testing.assert_allclose(L.aux.dlogits.sum(axis=1), 0.0, atol=1e-16)
        E, C = L.slots.slot_token.shape
        for e in range(E):
            toks = np.flatnonzero((L.routing.expert == e) & L.slots.keep)
            np.testing.assert_array_equal(L.slots.position[toks], np.arange(len(toks)))
            np.testing.assert_array_equal(L.slots.slot_token[e, :len(toks)], toks)
            assert np.all(L.slots.slot_token[e, len(toks):] == -1)
            assert np.all(toks[:-1] < toks[1:])
        assert L.slots.accepted.sum() <= min(97, E * C)
        filled = L.slots.slot_token >= 0
        np.testing.assert_array_equal(L.buf[filled], x[L.slots.slot_token[filled]])
        np.testing.assert_array_equal(L.buf[~filled], 0.0)
    # uniform f: each expert chosen twice
    z = np.full((8, 4), -1.0)
    z[np.arange(8), np.repeat(np.arange(4), 2)] = 1.0
    z += _rng(10).standard_normal((8, 4)) * 0.1
    r = so.softmax_top1(z)
    aux = so.aux_loss(np.bincount(r.expert, minlength=4), r.p, 1.0)
    np.testing.assert_allclose(aux.f, 0.25)
    np.testing.assert_allclose(aux.dlogits, 0.0, atol=1e-17)


def pin_finite_differences(so):
    """zffjzz 'troubleshooting': central finite differences of L(z) with f held fixed."""
    rng = _rng(11)
    T, E, alpha = 7, 5, 0.7
    z = rng.standard_normal((T, E))
    r = so.softmax_top1(z)
    counts = np.bincount(r.expert, minlength=E)
    G = so.aux_loss(counts, r.p, alpha).dlogits
    h = 1e-6
    num = np.zeros_like(z)
    for t in range(T):
        for j in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, j] += h
            zm[t, j] -= h
            lp = so.aux_loss(counts, so.softmax_top1(zp).p, alpha).loss
            lm = so.aux_loss(counts, so.softmax_top1(zm).p, alpha).loss
            num[t, j] = (lp - lm) / (2 * h)
    np.testing.assert_allclose(G, num, rtol=0, atol=2e-9)


def pin_independent_forms(so, T=512, d=64, F=128, E=4, c=1.25, seed=12, bias0=2.0):
    """The index form against the dense one-hot dispatch/combine form and a per-token loop."""
    x, w_r, b_r, w1, w2 = _tiny_problem(seed, T, d, F, E)
    b_r = b_r.copy()
    b_r[0] += bias0
    L = so.layer_forward(x, w_r, b_r, w1, w2, c, 0.01)
    D, expert_in, branch_dense = so.layer_dense_onehot(x, L.z, w1, w2, L.C)
    experts, positions, branch_loop = so.layer_per_token(x, L.z, w1, w2, L.C)
    np.testing.assert_array_equal(L.routing.expert, experts)
    np.testing.assert_array_equal(L.slots.position, positions)
    np.testing.assert_array_equal(L.buf, expert_in)
    np.testing.assert_allclose(L.branch, branch_dense, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L.branch, branch_loop, rtol=1e-12, atol=1e-12)
    return L


ALL_PINS = [
    pin_two_expert_balance, pin_uniform_counterexample, pin_uniform_capacity, pin_raw_load_capped,
    pin_shift_invariance, pin_softmax_library, pin_gate_not_renormalised, pin_local_overflow,
    pin_capacity_values, pin_single_expert_is_dense_ffn, pin_no_drop_brute_force, pin_zero_capacity,
    pin_invariants, pin_finite_differences,
    lambda so: pin_independent_forms(so, T=40, d=8, F=12, E=3, c=1.0, seed=13, bias0=0.5),
]


# ------------------------------------------------ NEXT f-1: router z-loss
def pin_z_loss(so):
    """zffjzz 'core idea and formulas' / 'minimal experiment': L_z = mean lse^2;
    +100 on every score moves lse by exactly 100 (L_z changes, p does not);
    uniform rows give (log E)^2; gradient by central finite differences;
    rows of the gradient sum to beta * 2 lse_t / T."""
    sh = GOLDEN["z_loss_shift"]["shift"]
    rng = _rng(21)
    z = rng.standard_normal((33, 7))
    beta = 0.37
    a, b = so.router_z_loss(z, beta), so.router_z_loss(z + sh, beta)
    lse = scipy.special.logsumexp(z, axis=1)
    assert abs(a.loss - beta * np.mean(lse ** 2)) <= 1e-13 * a.loss
    assert abs(b.loss - beta * np.mean((lse + sh) ** 2)) <= 1e-12 * b.loss
    assert b.loss > a.loss
    np.testing.assert_allclose(so.softmax_top1(z + sh).p, so.softmax_top1(z).p, rtol=1e-12, atol=1e-15)
    u = so.router_z_loss(np.zeros((10, 8)), 1.0)
    assert abs(u.loss - math.log(8) ** 2) < 1e-14
    np.testing.assert_allclose(a.dlogits.sum(axis=1), beta * 2 * lse / z.shape[0], rtol=1e-12)
    h = 1e-6
    num = np.zeros_like(z)
    for t in range(0, 33, 4):
        for j in range(7):
            zp, zm = z.copy(), z.copy()
            zp[t, j] += h
            zm[t, j] -= h
            num[t, j] = (so.router_z_loss(zp, beta).loss - so.router_z_loss(zm, beta).loss) / (2 * h)
    np.testing.assert_allclose(a.dlogits[::4], num[::4], rtol=0, atol=1e-9)
    assert so.router_z_loss(np.zeros((0, 3)), 1.0).loss == 0.0


ALL_PINS.append(pin_z_loss)


# ------------------------------------ NEXT f-3 / f-4: routing groups and top-k
def pin_groups_reduce_to_hot_path(so):
    """One group of all T tokens and k = 1 is the hot-path layer, field by field."""
    x, w_r, b_r, w1, w2 = _tiny_problem(31, 60, 8, 12, 5)
    for c in (0.5, 1.0, 1.5):
        A = so.layer_forward(x, w_r, b_r, w1, w2, c, 0.2)
        B = so.layer_forward_grouped(x, w_r, b_r, w1, w2, c, 0.2, k=1, G=None)
        assert B.Cg == A.C
        np.testing.assert_array_equal(B.routing.expert[:, 0], A.routing.expert)
        np.testing.assert_array_equal(B.slots.position[:, 0], A.slots.position)
        np.testing.assert_array_equal(B.slots.keep[:, 0], A.slots.keep)
        np.testing.assert_array_equal(B.slots.slot[:, 0], np.where(A.slots.keep, A.slots.position, -1))
        np.testing.assert_array_equal(B.slots.counts[0], A.slots.counts)
        np.testing.assert_array_equal(B.slots.accepted_total, A.slots.accepted)
        np.testing.assert_array_equal(B.slots.slot_token, A.slots.slot_token)
        np.testing.assert_array_equal(B.branch, A.branch)
        np.testing.assert_array_equal(B.aux.f[0], A.aux.f)
        np.testing.assert_array_equal(B.aux.P[0], A.aux.P)
        assert abs(B.aux.loss - A.aux.loss) <= 1e-14 * abs(A.aux.loss)
        np.testing.assert_allclose(B.aux.dlogits, A.aux.dlogits, rtol=1e-12, atol=1e-18)


def pin_groups_are_separate_batches(so):
    """zffjzz 'evaluation protocol': each group is its own batch.  The hot-path
    layer run on every group's slice with C = C_g gives the grouped result:
    positions, masks, counts, branch, f and P per group; the grouped loss is the
    mean of the per-group losses and the grouped gradient is the per-group one
    over the number of groups.  Buffer rows pack the groups in order."""
    x, w_r, b_r, w1, w2 = _tiny_problem(32, 96, 8, 12, 4)
    b_r = b_r.copy()
    b_r[1] += 1.0
    G = 24
    for c in (0.5, 1.25):
        L = so.layer_forward_grouped(x, w_r, b_r, w1, w2, c, 0.3, k=1, G=G)
        Cg = so.capacity(G, 4, c)
        assert L.Cg == Cg
        rows = np.zeros(4, np.int64)
        losses = []
        for g in range(96 // G):
            s = slice(g * G, (g + 1) * G)
            A = so.layer_forward(x[s], w_r, b_r, w1, w2, c, 0.3, C=Cg)
            np.testing.assert_array_equal(L.slots.position[s, 0], A.slots.position)
            np.testing.assert_array_equal(L.slots.keep[s, 0], A.slots.keep)
            np.testing.assert_array_equal(L.slots.counts[g], A.slots.counts)
            np.testing.assert_array_equal(L.slots.accepted[g], A.slots.accepted)
            kept = A.slots.keep
            e = A.routing.expert
            np.testing.assert_array_equal(L.slots.slot[s, 0][kept], rows[e[kept]] + A.slots.position[kept])
            rows += A.slots.accepted
            np.testing.assert_allclose(L.branch[s], A.branch, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(L.aux.f[g], A.aux.f, rtol=1e-15)
            np.testing.assert_allclose(L.aux.P[g], A.aux.P, rtol=1e-13)
            np.testing.assert_allclose(L.aux.dlogits[s], A.aux.dlogits / (96 // G), rtol=1e-12, atol=1e-17)
            losses.append(A.aux.loss)
        np.testing.assert_array_equal(L.slots.accepted_total, rows)
        assert abs(L.aux.loss - np.mean(losses)) <= 1e-14 * abs(L.aux.loss) + 1e-17


def _logits_for_choices(choices, E, rng):
    """Tie-free logits whose top choices are the given expert lists."""
    T = len(choices)
    z = rng.uniform(-1.0, 0.0, (T, E))
    for t, ch in enumerate(choices):
        for i, e in enumerate(ch):
            z[t, e] = 3.0 - i
    return z


def pin_batch_capacity_overflow(so):
    """zffjzz: per-64-row capacity; test counts [32,2,116,106] give 24.22 %
    overflow at c = 1.25 and none at c = 4.  A split with the hot experts
    uneven across batches overflows more under groups than under one group
    of all rows (local vs merged balance)."""
    g = GOLDEN["batch_capacity_overflow"]
    G, E = g["G"], g["E"]
    rng = _rng(33)

    def run(split, c, group):
        choices = []
        for b in range(4):
            blk = [e for e in range(E) for _ in range(split[e][b])]
            rng.shuffle(blk)
            choices += [[e] for e in blk]
        z = _logits_for_choices(choices, E, rng)
        r = so.softmax_topk(z, 1)
        T = len(choices)
        Gs = group if group else T
        sl = so.slot_scan_grouped(r.expert, E, Gs, so.group_capacity(Gs, E, c, 1))
        assert sl.counts.sum(axis=0).tolist() == g["test_counts"]
        return 1.0 - sl.keep.mean(), so.group_capacity(Gs, E, c, 1)

    even = [[8] * 4, [1, 1, 0, 0], [29] * 4, [26, 26, 27, 27]]
    ov, Cg = run(even, g["c_low"], G)
    assert Cg == g["expected_Cg_low"]
    assert round(100 * ov, 2) == g["expected_overflow_low_pct"] and ov == 62 / 256
    assert run(even, g["c_high"], G)[0] == g["expected_overflow_high"]
    assert run(even, g["c_low"], None)[0] == 62 / 256          # one group of 256 rows, C = 80
    uneven = [[8] * 4, [1, 1, 0, 0], [44, 44, 14, 14], [11, 11, 42, 42]]
    assert run(uneven, g["c_low"], G)[0] == 92 / 256
    assert run(uneven, g["c_low"], None)[0] == 62 / 256


def pin_topk_capacity(so):
    """lapla.si 'full means turned back': 32 per batch, 16 experts, 2 choices, c = 1 -> 4."""
    g = GOLDEN["topk_batch_capacity"]
    assert so.group_capacity(g["G"], g["E"], g["c"], g["k"]) == g["expected_C"]
    assert so.group_capacity(32, 16, 1.25, 2) == 5 and so.group_capacity(32, 16, 2.0, 2) == 8
    assert so.group_capacity(64, 4, 1.25, 1) == 20


def pin_priority_hand_example(so):
    """A hand-worked case where the two assignment orders differ: E = 3, k = 2,
    one group of 3 tokens, C_g = ceil(0.5 * 2 * 3 / 3) = 1; choices
    t0 -> (1, 0), t1 -> (0, 2), t2 -> (0, 1).
    Token order: t0's second choice takes expert 0's slot, t1's first choice drops.
    Rank order: t1's first choice takes it and t0's second choice drops."""
    z = np.array([[1.0, 2.0, 0.0], [2.0, 0.0, 1.0], [2.0, 1.0, 0.0]])
    r = so.softmax_topk(z, 2)
    np.testing.assert_array_equal(r.expert, [[1, 0], [0, 2], [0, 1]])
    Cg = so.group_capacity(3, 3, 0.5, 2)
    assert Cg == 1
    a = so.slot_scan_grouped(r.expert, 3, 3, Cg, "token")
    np.testing.assert_array_equal(a.position, [[0, 0], [1, 0], [2, 1]])
    np.testing.assert_array_equal(a.keep, [[1, 1], [0, 1], [0, 0]])
    np.testing.assert_array_equal(a.slot_token, [[0], [0], [1]])
    b = so.slot_scan_grouped(r.expert, 3, 3, Cg, "rank")
    np.testing.assert_array_equal(b.position, [[0, 2], [0, 0], [1, 1]])
    np.testing.assert_array_equal(b.keep, [[1, 0], [1, 1], [0, 0]])
    np.testing.assert_array_equal(b.slot_token, [[1], [0], [1]])
    np.testing.assert_array_equal(a.counts, [[3, 2, 1]])
    np.testing.assert_array_equal(b.counts, [[3, 2, 1]])


def pin_topk_brute_force(so):
    """Top-k with groups against a per-token brute force (repeated strict-greater
    scans, counting earlier assignments), both orders, with and without ties."""
    x, w_r, b_r, w1, w2 = _tiny_problem(34, 48, 8, 12, 5)
    z_rand = x.astype(np.float64) @ w_r.astype(np.float64) + b_r
    z_ties = _rng(35).integers(-2, 3, (48, 5)).astype(np.float64) / 4
    for z in (z_rand, z_ties):
        for k in (1, 2, 3):
            for G in (48, 12):
                for pr in ("token", "rank"):
                    for c in (0.5, 1.0):
                        L = so.layer_forward_grouped(x, w_r, b_r, w1, w2, c, 0.1, k=k, G=G, priority=pr, logits=z)
                        ch, pos, br = so.layer_per_token_topk(x, z, w1, w2, k, G, L.Cg, pr)
                        np.testing.assert_array_equal(L.routing.expert, ch)
                        np.testing.assert_array_equal(L.slots.position, pos)
                        np.testing.assert_array_equal(L.slots.keep, pos < L.Cg)
                        np.testing.assert_allclose(L.branch, br, rtol=1e-12, atol=1e-13)


def pin_topk_all_experts_is_soft_mixture(so):
    """k = E and c = 1: C_g = G, nothing dropped, and the branch is the dense
    probability-weighted sum of every expert's FFN (torch einsum)."""
    x, w_r, b_r, w1, w2 = _tiny_problem(36, 20, 8, 12, 3)
    L = so.layer_forward_grouped(x, w_r, b_r, w1, w2, 1.0, 0.1, k=3, G=10)
    assert L.Cg == 10 and L.slots.keep.all()
    X = torch.from_numpy(x.astype(np.float64))
    H = torch.relu(torch.einsum("td,efd->tef", X, torch.from_numpy(w1.astype(np.float64))))
    Y = torch.einsum("tef,edf->ted", H, torch.from_numpy(w2.astype(np.float64)))
    p = torch.softmax(torch.from_numpy(L.z), dim=1)
    ref = torch.einsum("te,ted->td", p, Y).numpy()
    np.testing.assert_allclose(L.branch, ref, rtol=1e-12, atol=1e-13)


def pin_grouped_aux(so):
    """Grouped / top-k balance loss: uniform rows give 1 for k = 1 and 2
    (f sums to 1 over the assignments); f of each group sums to 1; gradient
    rows sum to 0; central finite differences of the grouped loss."""
    for k in (1, 2):
        r = so.softmax_topk(np.zeros((64, 4)), k)
        sl = so.slot_scan_grouped(r.expert, 4, 16, 100)
        a = so.aux_loss_grouped(sl.counts, r.p, 16, k, 1.0)
        assert abs(a.loss - 1.0) < 1e-14
        np.testing.assert_allclose(a.f.sum(axis=1), 1.0, rtol=1e-15)
    rng = _rng(37)
    T, E, G, k, alpha = 12, 4, 4, 2, 0.7
    z = rng.standard_normal((T, E))
    r = so.softmax_topk(z, k)
    counts = so.slot_scan_grouped(r.expert, E, G, 100).counts
    A = so.aux_loss_grouped(counts, r.p, G, k, alpha)
    np.testing.assert_allclose(A.dlogits.sum(axis=1), 0.0, atol=1e-16)
    h = 1e-6
    num = np.zeros_like(z)
    for t in range(T):
        for j in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, j] += h
            zm[t, j] -= h
            num[t, j] = (so.aux_loss_grouped(counts, so.softmax_top1(zp).p, G, k, alpha).loss -
                         so.aux_loss_grouped(counts, so.softmax_top1(zm).p, G, k, alpha).loss) / (2 * h)
    np.testing.assert_allclose(A.dlogits, num, rtol=0, atol=2e-9)


GROUP_TOPK_PINS = [
    pin_groups_reduce_to_hot_path, pin_groups_are_separate_batches, pin_batch_capacity_overflow,
    pin_topk_capacity, pin_priority_hand_example, pin_topk_brute_force, pin_topk_all_experts_is_soft_mixture,
    pin_grouped_aux,
]
ALL_PINS.extend(GROUP_TOPK_PINS)


# ------------------------------------------------ NEXT f-2: layer backward
def _fd_problem(seed, T=24, d=8, F=12, E=3):
    """A tiny layer whose kept tokens have every pre-activation away from the
    ReLU kink and every top-2 logit margin away from a tie, so that a 1e-6
    step changes neither the choices nor the ReLU pattern."""
    for s in range(seed, seed + 50):
        x, w_r, b_r, w1, w2 = _tiny_problem(s, T, d, F, E)
        x = x.astype(np.float64)
        z = x @ w_r.astype(np.float64) + b_r
        srt = np.sort(z, axis=1)
        if np.min(srt[:, -1] - srt[:, -2]) < 1e-3:
            continue
        a = np.einsum("td,efd->tef", x, w1.astype(np.float64))
        if np.min(np.abs(a)) < 1e-4:
            continue
        return x, w_r.astype(np.float64), b_r.astype(np.float64), w1.astype(np.float64), w2.astype(np.float64)
    raise AssertionError("no suitable tiny problem")


def pin_backward_finite_differences(so):
    """zffjzz 'troubleshooting': central finite differences of
    J = sum <dout, out> + L_aux (+ L_z) over every entry of x, W_r, b_r, W1
    and W2, with the choices and masks held fixed; some tokens are dropped."""
    x, w_r, b_r, w1, w2 = _fd_problem(41)
    T, d = x.shape
    E = w_r.shape[1]
    c, alpha = 1.0, 0.3
    dout = _rng(42).standard_normal((T, d))
    for beta in (0.0, 0.05):
        L = so.layer_forward(x, w_r, b_r, w1, w2, c, alpha)
        assert (~L.slots.keep).any() and L.slots.keep.any()
        g = so.layer_backward(x, w_r, b_r, w1, w2, c, alpha, dout, beta=beta)
        e_fix, C = L.routing.expert, L.C
        h = 1e-6

        def J(**kw):
            a = dict(x=x, w_r=w_r, b_r=b_r, w1=w1, w2=w2)
            a.update(kw)
            return so.layer_objective(a["x"], a["w_r"], a["b_r"], a["w1"], a["w2"], c, alpha, dout, beta, e_fix, C)

        for name, arr, grad in (("x", x, g.dx), ("w_r", w_r, g.dw_r), ("b_r", b_r, g.db_r),
                                ("w1", w1, g.dw1), ("w2", w2, g.dw2)):
            num = np.zeros_like(arr)
            for idx in np.ndindex(arr.shape):
                p, m = arr.copy(), arr.copy()
                p[idx] += h
                m[idx] -= h
                num[idx] = (J(**{name: p}) - J(**{name: m})) / (2 * h)
            np.testing.assert_allclose(grad, num, rtol=1e-6, atol=2e-8, err_msg=f"d{name} (beta={beta})")


def pin_backward_single_expert_is_dense_mlp(so):
    """E = 1: p = 1, nothing dropped at c = 1, so the layer is x + relu(x W1^T) W2^T
    and its gradients are torch autograd's for that MLP; the router gets no
    gradient (the softmax of one logit is constant and the aux loss is alpha)."""
    rng = _rng(43)
    T, d, F = 20, 8, 12
    x = rng.standard_normal((T, d))
    w_r = rng.standard_normal((d, 1))
    w1 = rng.standard_normal((1, F, d)) * 0.3
    w2 = rng.standard_normal((1, d, F)) * 0.3
    dout = rng.standard_normal((T, d))
    g = so.layer_backward(x, w_r, None, w1, w2, 1.0, 0.01, dout)
    X = torch.tensor(x, requires_grad=True)
    W1 = torch.tensor(w1[0], requires_grad=True)
    W2 = torch.tensor(w2[0], requires_grad=True)
    out = X + torch.nn.functional.linear(torch.relu(torch.nn.functional.linear(X, W1)), W2)
    out.backward(torch.tensor(dout))
    np.testing.assert_allclose(g.dx, X.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g.dw1[0], W1.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g.dw2[0], W2.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(g.dw_r, 0.0)
    np.testing.assert_array_equal(g.db_r, 0.0)


def pin_backward_everything_dropped(so):
    """c = 0: every token rides the residual, so the experts get no gradient,
    the gate gets none, and the input gradient is dout plus the aux loss's
    path through the router (dz = dL_aux/dz)."""
    x, w_r, b_r, w1, w2 = _fd_problem(44)
    dout = _rng(45).standard_normal(x.shape)
    g = so.layer_backward(x, w_r, b_r, w1, w2, 0.0, 0.2, dout)
    np.testing.assert_array_equal(g.dw1, 0.0)
    np.testing.assert_array_equal(g.dw2, 0.0)
    np.testing.assert_array_equal(g.dgate, 0.0)
    L = so.layer_forward(x, w_r, b_r, w1, w2, 0.0, 0.2)
    np.testing.assert_allclose(g.dz, L.aux.dlogits, rtol=1e-15, atol=0)
    np.testing.assert_allclose(g.dx, dout + L.aux.dlogits @ w_r.T, rtol=1e-13, atol=1e-15)


BACKWARD_PINS = [pin_backward_finite_differences, pin_backward_single_expert_is_dense_mlp,
                 pin_backward_everything_dropped]
ALL_PINS.extend(BACKWARD_PINS)


# ------------------------- layer backward with routing groups and top-k choices
def pin_backward_grouped_reduces_to_hot_path(so):
    """One group of all T tokens and k = 1 is the hot-path layer: the grouped
    backward equals layer_backward (its own finite-difference pins) field by
    field, with and without z-loss, with some tokens dropped."""
    x, w_r, b_r, w1, w2 = _fd_problem(51)
    dout = _rng(52).standard_normal(x.shape)
    for beta in (0.0, 0.07):
        g1 = so.layer_backward(x, w_r, b_r, w1, w2, 1.0, 0.3, dout, beta=beta)
        gk = so.layer_backward_grouped(x, w_r, b_r, w1, w2, 1.0, 0.3, dout, k=1, beta=beta)
        assert (g1.dgate == 0).any() and (g1.dgate != 0).any()
        for name in ("dx", "dw_r", "db_r", "dw1", "dw2", "dz"):
            np.testing.assert_allclose(getattr(gk, name), getattr(g1, name), rtol=1e-12, atol=1e-14, err_msg=name)
        np.testing.assert_allclose(gk.dgate[:, 0], g1.dgate, rtol=1e-12, atol=1e-14)


def pin_backward_grouped_finite_differences(so):
    """zffjzz 'troubleshooting' for the grouped top-2 layer: central finite
    differences of J = sum <dout, out> + L_aux + L_z over every entry of x,
    W_r, b_r, W1 and W2, with the choices, slots and masks held fixed; three
    groups of 8 tokens, rank priority, some choices dropped."""
    x, w_r, b_r, w1, w2 = _fd_problem(53, E=4)
    T, d = x.shape
    k, G, pr, c, alpha, beta = 2, 8, "rank", 0.75, 0.3, 0.05
    dout = _rng(54).standard_normal((T, d))
    L = so.layer_forward_grouped(x, w_r, b_r, w1, w2, c, alpha, k=k, G=G, priority=pr)
    assert (~L.slots.keep).any() and L.slots.keep.any()
    g = so.layer_backward_grouped(x, w_r, b_r, w1, w2, c, alpha, dout, k=k, G=G, priority=pr, beta=beta)
    e_fix, Cg = L.routing.expert, L.Cg
    h = 1e-6

    def J(**kw):
        a = dict(x=x, w_r=w_r, b_r=b_r, w1=w1, w2=w2)
        a.update(kw)
        return so.layer_objective_grouped(a["x"], a["w_r"], a["b_r"], a["w1"], a["w2"], c, alpha, dout, beta,
                                          k, G, pr, e_fix, Cg)

    for name, arr, grad in (("x", x, g.dx), ("w_r", w_r, g.dw_r), ("b_r", b_r, g.db_r),
                            ("w1", w1, g.dw1), ("w2", w2, g.dw2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            num[idx] = (J(**{name: p}) - J(**{name: m})) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=2e-8, err_msg=f"d{name}")


def pin_backward_soft_mixture_autograd(so):
    """k = E with nothing dropped (c = 1, two groups): the layer is
    x + sum_e p_te FFN_e(x_t) and the balance loss is the constant alpha
    (f = 1/E in every group), so the gradients, z-loss included, are torch
    autograd's of that dense formula."""
    x, w_r, b_r, w1, w2 = _fd_problem(55, T=20, E=3)
    beta, alpha = 0.04, 0.2
    dout = _rng(56).standard_normal(x.shape)
    g = so.layer_backward_grouped(x, w_r, b_r, w1, w2, 1.0, alpha, dout, k=3, G=10, beta=beta)
    X, WR, BR, W1, W2 = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, w_r, b_r, w1, w2))
    z = X @ WR + BR
    H = torch.relu(torch.einsum("td,efd->tef", X, W1))
    Y = torch.einsum("tef,edf->ted", H, W2)
    out = X + torch.einsum("te,ted->td", torch.softmax(z, dim=1), Y)
    J = (out * torch.tensor(dout)).sum() + beta * (torch.logsumexp(z, dim=1) ** 2).mean()
    J.backward()
    for name, t in (("dx", X), ("dw_r", WR), ("db_r", BR), ("dw1", W1), ("dw2", W2)):
        np.testing.assert_allclose(getattr(g, name), t.grad.numpy(), rtol=1e-11, atol=1e-13, err_msg=name)


GROUP_BACKWARD_PINS = [pin_backward_grouped_reduces_to_hot_path, pin_backward_grouped_finite_differences,
                       pin_backward_soft_mixture_autograd]
ALL_PINS.extend(GROUP_BACKWARD_PINS)
