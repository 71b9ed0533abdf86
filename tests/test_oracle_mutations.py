"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pins catch every one of them.  This is evidence that the pins fix
each part of the oracle rather than restating it."""
import inspect
import math
import types

import numpy as np
import pytest

import oracle.switch_oracle as so_real
from tests import oracle_pins as pins

SRC = inspect.getsource(so_real)


def fresh_oracle():
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(SRC, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def m_argmax_last(m):
    orig = m.softmax_top1
    def f(z):
        r = orig(z)
        z = np.asarray(z, np.float64)
        e = (z.shape[1] - 1 - np.argmax(z[:, ::-1], axis=1)).astype(np.int64)
        return m.Routing(r.p, r.lse, e, r.p[np.arange(len(e)), e])
    m.softmax_top1 = f


def m_capacity_floor(m):
    m.capacity = lambda T, E, c: int(math.floor(c * T / E))


def m_capacity_float(m):
    m.capacity = lambda T, E, c: int(math.ceil(float(c) * T / E - 1e-9))


def m_aux_no_E(m):
    orig = m.aux_loss
    def f(counts, p, alpha):
        a = orig(counts, p, alpha)
        E = np.asarray(p).shape[1]
        return m.Aux(a.f, a.P, a.loss / E, a.dlogits / E)
    m.aux_loss = f


def m_aux_grad_sign(m):
    orig = m.aux_loss
    m.aux_loss = lambda counts, p, alpha: orig(counts, p, alpha)._replace(dlogits=-orig(counts, p, alpha).dlogits)


def m_aux_grad_no_p(m):
    orig = m.aux_loss
    def f(counts, p, alpha):
        a = orig(counts, p, alpha)
        p = np.asarray(p, np.float64)
        T, E = p.shape
        return a._replace(dlogits=(alpha * E / T) * (a.f[None, :] - (p @ a.f)[:, None]))
    m.aux_loss = f


def m_f_after_capacity(m):
    orig_layer = m.layer_forward
    def f(x, w_r, b_r, w1, w2, c, alpha, logits=None, expert_override=None, C=None):
        L = orig_layer(x, w_r, b_r, w1, w2, c, alpha, logits, expert_override, C)
        return L._replace(aux=m.aux_loss(L.slots.accepted, L.routing.p, alpha))
    m.layer_forward = f


def m_gate_renormalised(m):
    orig = m.combine
    m.combine = lambda y, e, pos, keep, gate, residual=None: orig(y, e, pos, keep, np.ones_like(gate), residual)


def m_scan_reverse(m):
    orig = m.slot_scan
    def f(expert, E, C):
        expert = np.asarray(expert)
        s = orig(expert[::-1], E, C)
        T = len(expert)
        st = np.where(s.slot_token >= 0, T - 1 - s.slot_token, -1)
        return m.Slots(s.position[::-1], s.keep[::-1], s.counts, s.accepted, st)
    m.slot_scan = f


def m_no_relu(m):
    m.expert_rows = lambda rows, w1, w2: (np.asarray(rows, np.float64) @ np.asarray(w1, np.float64).T) @ np.asarray(w2, np.float64).T


def m_combine_wrong_row(m):
    def f(y, expert, position, keep, gate, residual=None):
        T = expert.shape[0]
        branch = np.zeros((T, y.shape[2]))
        k = np.flatnonzero(keep)
        branch[k] = np.asarray(gate)[k, None] * y[expert[k], np.minimum(k, y.shape[1] - 1)]
        return branch if residual is None else residual + branch
    m.combine = f


def m_lse_no_max(m):
    orig = m.softmax_top1
    def f(z):
        r = orig(z)
        z = np.asarray(z, np.float64)
        return r._replace(lse=np.log(np.exp(z - z.max(axis=1, keepdims=True)).sum(axis=1)))
    m.softmax_top1 = f


def m_P_over_kept(m):
    orig_layer = m.layer_forward
    def f(x, w_r, b_r, w1, w2, c, alpha, logits=None, expert_override=None, C=None):
        L = orig_layer(x, w_r, b_r, w1, w2, c, alpha, logits, expert_override, C)
        p = L.routing.p * L.slots.keep[:, None]
        return L._replace(aux=m.aux_loss(L.slots.counts, p, alpha))
    m.layer_forward = f


def m_dispatch_shift(m):
    orig = m.dispatch
    def f(x, slot_token):
        b = orig(x, slot_token)
        return np.roll(b, 1, axis=1)
    m.dispatch = f


def m_transposed_w2(m):
    m.expert_rows = lambda rows, w1, w2: np.maximum(np.asarray(rows, np.float64) @ np.asarray(w1, np.float64).T, 0) @ np.asarray(w2, np.float64).reshape(np.asarray(w2).shape[::-1])


MUTANTS = [m_argmax_last, m_capacity_floor, m_capacity_float, m_aux_no_E, m_aux_grad_sign, m_aux_grad_no_p,
           m_f_after_capacity, m_gate_renormalised, m_scan_reverse, m_no_relu, m_combine_wrong_row,
           m_lse_no_max, m_P_over_kept, m_dispatch_shift, m_transposed_w2]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__)
def test_pins_catch_mutant(mutate):
    m = fresh_oracle()
    mutate(m)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(m)
        except Exception:  # an assertion, or a shape error caused by the mistake
            failed.append(getattr(pin, "__name__", "independent_forms"))
    assert failed, f"no pin caught {mutate.__name__}"


def test_fresh_oracle_passes_all_pins():
    m = fresh_oracle()
    for pin in pins.ALL_PINS:
        pin(m)


def m_zloss_no_square(m):
    orig = m.router_z_loss
    def f(z, beta):
        r = orig(z, beta)
        lse = m.softmax_top1(z).lse if np.asarray(z).shape[0] else np.zeros(0)
        return r._replace(loss=float(beta * np.mean(np.abs(lse))) if lse.size else 0.0)
    m.router_z_loss = f


def m_zloss_grad_no_lse(m):
    orig = m.router_z_loss
    def f(z, beta):
        r = orig(z, beta)
        T = np.asarray(z).shape[0]
        return r._replace(dlogits=beta * (2.0 / max(T, 1)) * m.softmax_top1(z).p if T else r.dlogits)
    m.router_z_loss = f


@pytest.mark.parametrize("mutate", [m_zloss_no_square, m_zloss_grad_no_lse], ids=lambda f: f.__name__)
def test_z_loss_pin_catches_mutant(mutate):
    m = fresh_oracle()
    mutate(m)
    with pytest.raises(Exception):
        pins.pin_z_loss(m)


# ------------------------------------ routing groups and top-k
def m_group_capacity_no_k(m):
    cap = m.capacity
    m.group_capacity = lambda G, E, c, k=1: cap(G, E, c)


def m_priority_swapped(m):
    orig = m.assignment_order
    m.assignment_order = lambda G, k, priority: orig(G, k, "rank" if priority == "token" else "token")


def m_rows_not_packed(m):
    orig = m.slot_scan_grouped
    def f(expert, E, G, Cg, priority="token"):
        s = orig(expert, E, G, Cg, priority)
        slot = np.where(s.keep, s.position, -1)
        st = np.full_like(s.slot_token, -1)
        T, k = slot.shape
        for t in range(T):
            for i in range(k):
                if slot[t, i] >= 0:
                    st[int(np.asarray(expert).reshape(T, -1)[t, i]), slot[t, i]] = t
        return s._replace(slot=slot, slot_token=st)
    m.slot_scan_grouped = f


def m_counters_not_reset(m):
    def f(expert, E, G, Cg, priority="token"):
        expert = np.asarray(expert, np.int64).reshape(len(expert), -1)
        T, k = expert.shape
        one = m.slot_scan(expert[:, 0], E, Cg) if k == 1 else None
        if one is None:
            raise AssertionError("k > 1 path not mutated")
        ng = T // G
        counts = np.stack([np.bincount(expert[g * G:(g + 1) * G, 0], minlength=E) for g in range(ng)])
        slot = np.where(one.keep, one.position, -1)[:, None]
        st = np.full((E, ng * Cg), -1, np.int64)
        st[:, :Cg] = one.slot_token
        return m.SlotsG(one.position[:, None], one.keep[:, None], slot, counts, np.minimum(counts, Cg),
                        one.accepted, st)
    m.slot_scan_grouped = f


def m_grouped_f_over_G(m):
    orig = m.aux_loss_grouped
    m.aux_loss_grouped = lambda counts, p, G, k, alpha: orig(np.asarray(counts) * k, p, G, k, alpha)


def m_grouped_loss_sum(m):
    orig = m.aux_loss_grouped
    def f(counts, p, G, k, alpha):
        a = orig(counts, p, G, k, alpha)
        ng = np.asarray(counts).reshape(-1, np.asarray(p).shape[1]).shape[0]
        return a._replace(loss=a.loss * ng)
    m.aux_loss_grouped = f


def m_grouped_grad_global_f(m):
    orig = m.aux_loss_grouped
    def f(counts, p, G, k, alpha):
        a = orig(counts, p, G, k, alpha)
        p = np.asarray(p, np.float64)
        T, E = p.shape
        if T == 0:
            return a
        fm = a.f.mean(axis=0)
        return a._replace(dlogits=(alpha * E / T) * p * (fm[None, :] - (p @ fm)[:, None]))
    m.aux_loss_grouped = f


def m_topk_ties_high(m):
    orig = m.softmax_topk
    def f(z, k):
        r = orig(z, k)
        z = np.asarray(z, np.float64)
        E = z.shape[1]
        order = (E - 1 - np.argsort(-z[:, ::-1], axis=1, kind="stable"))[:, :k]
        return r._replace(expert=order, gate=np.take_along_axis(r.p, order, axis=1))
    m.softmax_topk = f


def m_topk_renormalised(m):
    orig = m.softmax_topk
    def f(z, k):
        r = orig(z, k)
        return r._replace(gate=r.gate / r.gate.sum(axis=1, keepdims=True))
    m.softmax_topk = f


def m_combine_first_choice_only(m):
    orig = m.combine_topk
    def f(y, expert, slot, keep, gate, residual=None):
        keep = np.asarray(keep, bool).reshape(len(expert), -1).copy()
        keep[:, 1:] = False
        return orig(y, expert, slot, keep, gate, residual)
    m.combine_topk = f


GROUP_MUTANTS = [m_group_capacity_no_k, m_priority_swapped, m_rows_not_packed, m_counters_not_reset,
                 m_grouped_f_over_G, m_grouped_loss_sum, m_grouped_grad_global_f, m_topk_ties_high,
                 m_topk_renormalised, m_combine_first_choice_only]


@pytest.mark.parametrize("mutate", GROUP_MUTANTS, ids=lambda f: f.__name__)
def test_group_topk_pins_catch_mutant(mutate):
    """Each planted mistake in the grouped / top-k oracle fails one of the pins
    written for it (not only a pin of the hot path)."""
    m = fresh_oracle()
    mutate(m)
    failed = []
    for pin in pins.GROUP_TOPK_PINS:
        try:
            pin(m)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no grouped/top-k pin caught {mutate.__name__}"


# ------------------------------------ layer backward: mistakes planted in the source text
BACKWARD_EDITS = [
    ("active = (a > 0) if relu_active", "active = 1.0 if relu_active"),            # no ReLU mask
    ("dy = g[:, None] * dout[toks]", "dy = dout[toks]"),                             # gate dropped
    ("dz = (dgate * r.gate)[:, None] * (onehot - r.p)",
     "dz = (dgate * r.gate)[:, None] * (r.p - onehot)"),                             # softmax sign
    ("dx = dx + dz @ w_r64.T", "dx = dx"),                                           # no router path
    ("dw2[j] = dy.T @ h", "dw2[j] = dy.T @ a"),                                      # pre-activation
    ("dz = dz + L.aux.dlogits", "dz = dz"),                                          # aux gradient lost
    ("dgate[toks] = np.sum(dout[toks] * y, axis=1)", "dgate[toks] = np.sum(dout[toks] * h @ W2.T * g[:, None], axis=1)"),
]


@pytest.mark.parametrize("edit", BACKWARD_EDITS, ids=lambda e: e[1][:30])
def test_backward_pins_catch_mutant(edit):
    old, new = edit
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in pins.BACKWARD_PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no backward pin caught {new}"


# ------------------- grouped / top-k backward: mistakes planted in the source text
GROUP_BACKWARD_EDITS = [
    ("gr = r.gate[toks, ranks]", "gr = r.gate[toks, 0]"),                               # first choice's gate
    ("dgate[toks, ranks] = np.sum(", "dgate[toks, 0] = np.sum("),                       # dgate on rank 0
    ("dz += (dgate[:, i] * r.gate[:, i])", "dz += (dgate[:, i] * r.gate[:, 0])"),       # wrong gate in dz
    ("on = (acts > 0) if relu_active", "on = 1.0 if relu_active"),                      # no ReLU mask
    ("np.add.at(dx, toks, dar @ W1)", "np.add.at(dx, toks, 0 * (dar @ W1))"),           # no expert path
    ("dz += L.aux.dlogits", "dz += 0 * L.aux.dlogits"),                                 # aux gradient lost
    ("dz += router_z_loss(L.z, beta).dlogits", "dz += 0 * router_z_loss(L.z, beta).dlogits"),   # z-loss lost
    ("dx += dz @ wr.T", "dx += 0 * (dz @ wr.T)"),                                       # no router path
]


@pytest.mark.parametrize("edit", GROUP_BACKWARD_EDITS, ids=lambda e: e[1][:30])
def test_group_backward_pins_catch_mutant(edit):
    old, new = edit
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in pins.GROUP_BACKWARD_PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no grouped backward pin caught {new}"
