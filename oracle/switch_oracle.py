"""fp64 CPU oracle for the Switch Transformer sparse expert FFN layer (forward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
It shares no code, tables or helpers with the HIP library and imports nothing
from it.

Every step is written out in plain NumPy float64, in the order and notation of
the pages, with no blocking or fusion.  Inputs are the same bf16 / fp32 values
the GPU receives, taken exactly into float64.

Sources (page title, then the section or formula used):
  [WQ]  "042 Switch Transformer: each token picks one expert"
        (wq-win.github.io/llm/042-switch.html): sec. 1 problem setting
        (router softmax, e* = argmax, y = p_e* f_e*, capacity C = (T/E)c,
        overflow rides the residual); sec. 2 (aux loss
        alpha*E*sum f_e P_e, f a hard count, P differentiable, worked example
        2(0.72+0.02) = 1.48, the gate 0.7 must not be renormalised); sec. 3
        (the layer as a step list: fp32 router, top-1, aux loss, capacity-
        truncated dispatch/combine, expert FFN, gate-scaled combine back to the
        original position, residual; the 100-token / 10-expert example).
  [DMX] "Switch Transformers: Scaling to Trillion Parameter Models with Simple
        and Efficient Sparsity" essay (dmxsf.com): "core structure" section
        (experts replace the FFN sublayer).
  [XZ]  paper card "Switch Transformers ..." (ai-papers.xuzou.cn): "bottleneck"
        (fixed capacity, overflow skips the expert layer) and "method
        adaptation" (fp32 router and softmax; dispatch/combine tensors over
        [cores, tokens, experts, capacity]).
  [LAP] "Mixture of experts" explainer (world.lapla.si/zh/moe/): "what is
        inside an expert" (d -> d_ff ReLU -> d FFN); "a small penalty"
        (alpha*N*sum f_i P_i, alpha = 0.01); "full means turned back"
        (capacity, dropped tokens continue on the residual).
  [ZF]  "MoE routing load collapse" reproduction note (zffjzz.top): "core idea
        and formulas" (Z = XW, p = softmax(Z_t), a_t = argmax, f, P, L_bal,
        C = ceil(cT/E), accept mask m_t, z-loss); "official code reading route"
        (aux statistics computed before capacity masks, slots by cumulative
        position along the sequence, argmax of a truncated mask sends dropped
        rows to expert 0); "minimal experiment" (uniform rows: f = (1,0,0,0),
        loss 1, C = 20, 68.75 % overflow; [28,12,12,12] -> [8,8,8,8]; +100
        shift leaves p and a unchanged); "troubleshooting" (central finite
        differences).

Readings where the pages are silent or disagree (each one also listed in the
design notes): argmax is taken over the logits, which equals the argmax of the
exact probabilities because softmax is strictly increasing; ties go to the
lowest index (NumPy's first-occurrence rule, [ZF] minimal experiment);
C = ceil(c*T/E) on the exact binary value of c ([ZF] formulas; [WQ] sec. 1
gives T/E*c without rounding); one routing group holds all T tokens; alpha sits
inside the aux loss ([WQ] sec. 2; [ZF] places it outside, pins use alpha = 1);
the gate is the raw p_e*, never renormalised ([WQ] sec. 2); experts carry no
biases; empty capacity slots hold zeros.

Pins: every function here is pinned by tests/test_oracle_pins.py against the
pages' worked values, closed forms, library routines (scipy softmax /
logsumexp, a dense torch MLP) and brute force on tiny inputs.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import NamedTuple, Optional

import numpy as np


# ------------------------------------------------------------------ O1 router
def router_logits(x: np.ndarray, w_r: np.ndarray, b_r: Optional[np.ndarray] = None) -> np.ndarray:
    """z_te = sum_i x_ti W_r[i, e] + b_r[e]  in float64.

    [ZF] "core idea and formulas": Z = XW with W in R^{d x E}; [WQ] sec. 1:
    p(x) = softmax(W_r x).  The bias is the constant-one input column of [ZF]
    "core idea and formulas" written as a separate vector.
    """
    z = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64)
    if b_r is not None:
        z = z + np.asarray(b_r, np.float64)[None, :]
    return z


# ------------------------------------------------------- O2, O3 softmax, top-1
class Routing(NamedTuple):
    p: np.ndarray        # [T, E] probabilities, rows sum to 1
    lse: np.ndarray      # [T] log sum_j exp(z_tj)
    expert: np.ndarray   # [T] int64, e*_t (lowest index among maximal logits)
    gate: np.ndarray     # [T] p_{t, e*_t}


def softmax_top1(z: np.ndarray) -> Routing:
    """p_te = exp(z_te - m_t) / sum_j exp(z_tj - m_t), m_t = max_j z_tj;
    e*_t = argmax_e z_te (first maximum); gate_t = p_{t,e*_t}.

    [WQ] sec. 1: e*(x) = argmax_e p_e(x), y = p_e*(x) f_e*(x).
    [ZF] "core idea and formulas": p_ti = softmax(Z_t)_i, a_t = argmax_i p_ti;
    "minimal experiment": ties go to the first index.
    """
    z = np.asarray(z, np.float64)
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logits are outside the layer's contract")
    m = z.max(axis=1)
    ez = np.exp(z - m[:, None])
    s = ez.sum(axis=1)
    p = ez / s[:, None]
    lse = m + np.log(s)
    expert = np.argmax(z, axis=1).astype(np.int64)
    gate = p[np.arange(z.shape[0]), expert]
    return Routing(p, lse, expert, gate)


# ------------------------------------------------------------- O4 capacity
def capacity(T: int, E: int, c: float) -> int:
    """C = ceil(c * T / E), exact on the binary value of c.

    [ZF] "core idea and formulas": C = ceil(cT/E) (rounding up is that page's
    convention); [WQ] sec. 1: C = (T/E) c; [XZ] "bottleneck": tokens per batch
    divided by the number of experts, times the capacity factor.
    """
    if T < 0 or E <= 0 or not (c >= 0) or math.isinf(c):
        raise ValueError("capacity needs T >= 0, E > 0, finite c >= 0")
    return math.ceil(Fraction(c) * T / E)


# ------------------------------------------------------------- O5 slot scan
class Slots(NamedTuple):
    position: np.ndarray    # [T] int64: rank of t among earlier tokens with the same expert
    keep: np.ndarray        # [T] bool: position < C
    counts: np.ndarray      # [E] raw (pre-capacity) choices
    accepted: np.ndarray    # [E] min(counts, C)
    slot_token: np.ndarray  # [E, C] token in each slot, -1 if empty


def slot_scan(expert: np.ndarray, E: int, C: int) -> Slots:
    """One pass in token order: pos_t = cnt[e*_t]; cnt[e*_t] += 1; keep_t = pos_t < C.

    [ZF] "official code reading route": positions are the cumulative count
    along the sequence, not an ordering by probability; [WQ] sec. 3:
    truncate the assignment by expert capacity.  Dropped tokens keep their
    true expert id ([ZF] "official code reading route": recovering the id
    from the truncated mask would send them to expert 0).
    """
    expert = np.asarray(expert, np.int64)
    T = expert.shape[0]
    cnt = [0] * E
    position = np.empty(T, np.int64)
    keep = np.empty(T, bool)
    slot_token = np.full((E, C), -1, np.int64)
    for t in range(T):
        e = int(expert[t])
        position[t] = cnt[e]
        cnt[e] += 1
        keep[t] = position[t] < C
        if keep[t]:
            slot_token[e, position[t]] = t
    counts = np.array(cnt, np.int64)
    return Slots(position, keep, counts, np.minimum(counts, C), slot_token)


# ------------------------------------------------------------- O6 dispatch
def dispatch(x: np.ndarray, slot_token: np.ndarray) -> np.ndarray:
    """buf[e, s] = x[slot_token[e, s]] for filled slots, zero rows otherwise.

    [WQ] sec. 3: build the dispatch tensor and send tokens to their expert;
    [XZ] "method adaptation": dispatch/combine over [tokens, experts, capacity].
    """
    E, C = slot_token.shape
    buf = np.zeros((E, C, x.shape[1]), np.float64)
    filled = slot_token >= 0
    buf[filled] = np.asarray(x, np.float64)[slot_token[filled]]
    return buf


# ------------------------------------------------------------- O7 experts
def expert_rows(rows: np.ndarray, w1_e: np.ndarray, w2_e: np.ndarray) -> np.ndarray:
    """One expert on a set of rows: max(0, rows W1_e^T) W2_e^T, fp64, no rounding.

    [DMX] "core structure": experts take the place of the FFN sublayer;
    [LAP] "what is inside an expert": d numbers -> d_ff with negatives set to
    zero -> back to d.  W1_e is [d_ff, d] and W2_e is [d, d_ff] (out-features
    major); no expert biases.
    """
    h = np.maximum(np.asarray(rows, np.float64) @ np.asarray(w1_e, np.float64).T, 0.0)
    return h @ np.asarray(w2_e, np.float64).T


def expert_ffn(buf: np.ndarray, accepted: np.ndarray, w1, w2) -> np.ndarray:
    """y[e, s] = expert_e(buf[e, s]) for s < accepted[e]; other rows zero.

    w1 and w2 are indexable by expert (arrays or callables returning a float
    matrix), so experts can be materialised one at a time.
    """
    E, C, d = buf.shape
    y = np.zeros((E, C, d), np.float64)
    for e in range(E):
        a = int(accepted[e])
        if a == 0:
            continue
        w1e = w1(e) if callable(w1) else w1[e]
        w2e = w2(e) if callable(w2) else w2[e]
        y[e, :a] = expert_rows(buf[e, :a], w1e, w2e)
    return y


# ------------------------------------------------------------- O8 combine
def combine(y: np.ndarray, expert: np.ndarray, position: np.ndarray, keep: np.ndarray,
            gate: np.ndarray, residual: Optional[np.ndarray] = None) -> np.ndarray:
    """branch_t = keep_t * gate_t * y[e*_t, pos_t] (0 if dropped); out_t = residual_t + branch_t.

    [WQ] sec. 1: y = p_e*(x) f_e*(x), overflow tokens skip the expert branch
    and continue on the residual; sec. 2: the selected probability (e.g. 0.7)
    multiplies the expert output and is not renormalised to 1; sec. 3: multiply
    by the routing probability, put back at the original position, add the
    residual.  [ZF] "core idea and formulas": y_t = residual + m_t p_{t,a_t} (...).
    """
    T = expert.shape[0]
    d = y.shape[2]
    branch = np.zeros((T, d), np.float64)
    k = np.flatnonzero(keep)
    branch[k] = np.asarray(gate, np.float64)[k, None] * y[expert[k], position[k]]
    if residual is None:
        return branch
    return np.asarray(residual, np.float64) + branch


# ------------------------------------------------------------- O9 aux loss
class Aux(NamedTuple):
    f: np.ndarray        # [E] fraction of raw (pre-capacity) choices
    P: np.ndarray        # [E] mean router probability
    loss: float          # alpha * E * sum_e f_e P_e
    dlogits: np.ndarray  # [T, E] dL/dz with f held constant


def aux_loss(counts: np.ndarray, p: np.ndarray, alpha: float) -> Aux:
    """f_e = counts_e / T, P_e = (1/T) sum_t p_te, L = alpha E sum_e f_e P_e,
    dL/dz_tj = (alpha E / T) p_tj (f_j - sum_e f_e p_te).

    [WQ] sec. 2: L_aux = alpha E sum_e f_e P_e, f from the hard choice and not
    differentiated, P differentiable.  [ZF] "core idea and formulas": f counts
    the choices before the capacity limit.  The gradient is the chain rule of
    L through P_e = mean_t softmax(z_t)_e with d p_te / d z_tj = p_te (delta_ej - p_tj).
    """
    p = np.asarray(p, np.float64)
    T, E = p.shape
    if T == 0:   # empty batch: no load, no probability mass, no loss
        return Aux(np.zeros(E), np.zeros(E), 0.0, np.zeros((0, E)))
    f = np.asarray(counts, np.float64) / T
    P = p.sum(axis=0) / T
    loss = float(alpha * E * np.dot(f, P))
    s = p @ f
    dlogits = (alpha * E / T) * p * (f[None, :] - s[:, None])
    return Aux(f, P, loss, dlogits)


# ------------------------------------------------------------- the layer
class LayerResult(NamedTuple):
    z: np.ndarray
    routing: Routing
    C: int
    slots: Slots
    buf: np.ndarray
    y: np.ndarray
    branch: np.ndarray
    out: np.ndarray
    aux: Aux


def layer_forward(x, w_r, b_r, w1, w2, c: float, alpha: float,
                  logits: Optional[np.ndarray] = None,
                  expert_override: Optional[np.ndarray] = None,
                  C: Optional[int] = None) -> LayerResult:
    """O1 .. O9 in the order of [WQ] sec. 3.

    The aux statistics use the raw choices, before capacity truncates them
    ([ZF] "official code reading route").  `logits` replaces O1 (dispatch-only
    runs are fed identical fp32 logits).  `expert_override` substitutes a
    given choice vector after O3 and re-runs O4..O9 from it; tests use it to
    resolve near-tie tokens the same way the device did.
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    z = router_logits(x, w_r, b_r) if logits is None else np.asarray(logits, np.float64)
    E = z.shape[1]
    r = softmax_top1(z)
    if expert_override is not None:
        e = np.asarray(expert_override, np.int64)
        r = Routing(r.p, r.lse, e, r.p[np.arange(T), e])
    if C is None:
        C = capacity(T, E, c)
    aux = aux_loss(np.bincount(r.expert, minlength=E), r.p, alpha)
    sl = slot_scan(r.expert, E, C)
    buf = dispatch(x, sl.slot_token)
    y = expert_ffn(buf, sl.accepted, w1, w2)
    branch = combine(y, r.expert, sl.position, sl.keep, r.gate, None)
    return LayerResult(z, r, C, sl, buf, y, branch, x + branch, aux)


# ------------------------------------------------ O10 independent formulations
def layer_dense_onehot(x, z, w1, w2, C: int):
    """The dispatch/combine-tensor form, written from its description in [XZ]
    "method adaptation" (dispatch and combine tensors over tokens x experts x
    capacity; a one-hot dispatch, a gate-weighted combine).

    Positions come from a cumulative sum of the one-hot choice matrix along
    the token axis (no running counter), expert inputs from a contraction of
    the dispatch tensor with x, and the output from a contraction of the
    combine tensor with the expert outputs.  For tiny inputs only.
    """
    x = np.asarray(x, np.float64)
    z = np.asarray(z, np.float64)
    T, E = z.shape
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    onehot = (np.arange(E)[None, :] == np.argmax(z, axis=1)[:, None]).astype(np.float64)
    pos_in_expert = (np.cumsum(onehot, axis=0) - 1.0) * onehot        # [T, E]
    dispatch_t = np.zeros((T, E, C))
    for s in range(C):
        dispatch_t[:, :, s] = onehot * (pos_in_expert == s)
    expert_in = np.einsum("tes,td->esd", dispatch_t, x)
    expert_out = np.zeros_like(expert_in)
    for e in range(E):
        w1e = w1(e) if callable(w1) else w1[e]
        w2e = w2(e) if callable(w2) else w2[e]
        expert_out[e] = np.maximum(expert_in[e] @ np.asarray(w1e, np.float64).T, 0.0) @ np.asarray(w2e, np.float64).T
    combine_t = dispatch_t * (p * onehot).sum(axis=1)[:, None, None]
    branch = np.einsum("tes,esd->td", combine_t, expert_out)
    return dispatch_t, expert_in, branch


def layer_per_token(x, z, w1, w2, C: int):
    """A per-token loop with no shared state: for each token, its expert by a
    strict-greater scan over the logits, its slot by counting earlier tokens
    with the same expert, and its branch by two matrix-vector products.
    For tiny inputs only.
    """
    x = np.asarray(x, np.float64)
    z = np.asarray(z, np.float64)
    T, E = z.shape
    experts = []
    for t in range(T):
        best = 0
        for e in range(1, E):
            if z[t, e] > z[t, best]:
                best = e
        experts.append(best)
    branch = np.zeros_like(x)
    positions = []
    for t in range(T):
        e = experts[t]
        pos = sum(1 for s in range(t) if experts[s] == e)
        positions.append(pos)
        if pos < C:
            g = math.exp(z[t, e]) / sum(math.exp(v) for v in z[t])
            w1e = np.asarray(w1(e) if callable(w1) else w1[e], np.float64)
            w2e = np.asarray(w2(e) if callable(w2) else w2[e], np.float64)
            h = np.maximum(w1e @ x[t], 0.0)
            branch[t] = g * (w2e @ h)
    return np.array(experts), np.array(positions), branch


# ------------------------------------------------ NEXT f-1: router z-loss
class ZLoss(NamedTuple):
    loss: float          # beta * (1/T) sum_t lse_t^2
    dlogits: np.ndarray  # [T, E] d loss / d z = beta * (2/T) lse_t p_tj


def router_z_loss(z: np.ndarray, beta: float) -> ZLoss:
    """L_z = beta * (1/T) sum_t (log sum_i exp(z_ti))^2 and its gradient.

    [ZF] "core idea and formulas": the router z-loss of ST-MoE penalises the
    log normaliser of every token's scores (it is not a balance measure);
    "minimal experiment": adding 100 to every score changes it while p and
    the choice do not.  beta is the coefficient the caller puts on it, kept
    inside like alpha (ZF trains with 0.001).  d lse_t / d z_tj = p_tj.
    For T = 0 the loss is 0.
    """
    z = np.asarray(z, np.float64)
    T = z.shape[0]
    if T == 0:
        return ZLoss(0.0, np.zeros_like(z))
    r = softmax_top1(z)
    loss = float(beta * np.mean(r.lse ** 2))
    dlogits = beta * (2.0 / T) * r.lse[:, None] * r.p
    return ZLoss(loss, dlogits)


# ------------------------------------ NEXT f-3 / f-4: routing groups and top-k
#
# Routing groups ([XZ] "method adaptation": the input is reshaped to
# cores x tokens per core x d and dispatch/combine carry a group axis;
# [ZF] "evaluation protocol": every 64 rows apply the capacity limit on their
# own and the batch metrics are averaged over those batches; "follow-up
# questions": compare per-group and merged statistics).  Group g holds the
# G consecutive tokens g*G .. g*G+G-1 (T must be a multiple of G); each group
# has its own capacity per expert and its own slot counters.
#
# Top-k ([LAP] "full means turned back": capacity = tokens per batch / experts
# x choices per token x capacity factor; [XZ] "method adaptation": Switch is
# the k = 1 case of the earlier top-2 MoE).  A token's k choices are its k
# largest logits, ties to the lower index; each choice keeps its raw softmax
# probability as its gate (no renormalisation over the k, as for Switch in
# [WQ] sec. 2).
#
# Order of the assignments inside a group, for the slot counters:
#   "token": (token, rank) in lexicographic order - every slot of an expert
#            goes to earlier tokens first, whatever the rank of the choice;
#   "rank":  (rank, token) - all first choices of the group before any second
#            choice (the priority of the earlier top-2 MoE).
# Both equal the hot path's token order when k = 1.
#
# Buffer rows: an expert's kept assignments are packed in (group, order)
# order, so row = (kept assignments of that expert in earlier groups) + the
# in-group position; the buffer has n_groups * C_g rows per expert and the
# filled rows of expert e are 0 .. accepted_total[e]-1.  With one group the row
# is the position, as in the hot path.

class RoutingK(NamedTuple):
    p: np.ndarray        # [T, E]
    lse: np.ndarray      # [T]
    expert: np.ndarray   # [T, k] int64, choices in decreasing logit order
    gate: np.ndarray     # [T, k] raw probabilities of the choices


def softmax_topk(z: np.ndarray, k: int) -> RoutingK:
    """The k largest logits of each token, ties to the lower index, with their
    raw softmax probabilities.  k = 1 is softmax_top1."""
    z = np.asarray(z, np.float64)
    T, E = z.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    r = softmax_top1(z)
    # a stable sort of -z keeps equal logits in index order
    order = np.argsort(-z, axis=1, kind="stable")[:, :k].astype(np.int64)
    gate = np.take_along_axis(r.p, order, axis=1)
    return RoutingK(r.p, r.lse, order, gate)


def group_capacity(G: int, E: int, c: float, k: int = 1) -> int:
    """Per-group, per-expert capacity ceil(c * k * G / E) ([LAP] "full means
    turned back"; the rounding up follows [ZF] "core idea and formulas")."""
    return capacity(k * G, E, c)


class SlotsG(NamedTuple):
    position: np.ndarray        # [T, k] in-group position of each assignment
    keep: np.ndarray            # [T, k] position < C_g
    slot: np.ndarray            # [T, k] buffer row within its expert, -1 if dropped
    counts: np.ndarray          # [n_groups, E] raw assignments per group
    accepted: np.ndarray        # [n_groups, E] min(counts, C_g)
    accepted_total: np.ndarray  # [E] sum over groups of accepted
    slot_token: np.ndarray      # [E, n_groups * C_g] token in each row, -1 if empty


def assignment_order(G: int, k: int, priority: str):
    """(local token, rank) pairs of one group in slot-counter order."""
    if priority == "token":
        return [(u, i) for u in range(G) for i in range(k)]
    if priority == "rank":
        return [(u, i) for i in range(k) for u in range(G)]
    raise ValueError("priority must be 'token' or 'rank'")


def slot_scan_grouped(expert: np.ndarray, E: int, G: int, Cg: int, priority: str = "token") -> SlotsG:
    """Per group: one pass over its assignments in the chosen order with a
    counter per expert; keep = position < C_g.  Rows packed per expert."""
    expert = np.asarray(expert, np.int64)
    if expert.ndim == 1:
        expert = expert[:, None]
    T, k = expert.shape
    if G <= 0 or T % G != 0:
        raise ValueError("T must be a multiple of the group size")
    ng = T // G
    position = np.empty((T, k), np.int64)
    keep = np.empty((T, k), bool)
    slot = np.full((T, k), -1, np.int64)
    counts = np.zeros((ng, E), np.int64)
    accepted = np.zeros((ng, E), np.int64)
    slot_token = np.full((E, ng * Cg), -1, np.int64)
    rows_used = [0] * E
    order = assignment_order(G, k, priority)
    for g in range(ng):
        cnt = [0] * E
        for u, i in order:
            t = g * G + u
            e = int(expert[t, i])
            position[t, i] = cnt[e]
            cnt[e] += 1
            keep[t, i] = position[t, i] < Cg
        for e in range(E):
            counts[g, e] = cnt[e]
            accepted[g, e] = min(cnt[e], Cg)
        # rows: this group's kept assignments of each expert follow the
        # earlier groups', in in-group position order
        for u, i in order:
            t = g * G + u
            if keep[t, i]:
                e = int(expert[t, i])
                slot[t, i] = rows_used[e] + position[t, i]
                slot_token[e, slot[t, i]] = t
        for e in range(E):
            rows_used[e] += int(accepted[g, e])
    return SlotsG(position, keep, slot, counts, accepted, np.array(rows_used, np.int64), slot_token)


def combine_topk(y: np.ndarray, expert: np.ndarray, slot: np.ndarray, keep: np.ndarray, gate: np.ndarray,
                 residual: Optional[np.ndarray] = None) -> np.ndarray:
    """branch_t = sum over the token's kept choices i of gate_ti * y[e_ti, slot_ti]
    ([WQ] sec. 1/3 for one choice; the k choices are added with their raw
    probabilities).  Dropped choices add nothing."""
    expert = np.asarray(expert, np.int64).reshape(len(expert), -1)
    slot = np.asarray(slot, np.int64).reshape(expert.shape)
    keep = np.asarray(keep, bool).reshape(expert.shape)
    gate = np.asarray(gate, np.float64).reshape(expert.shape)
    T, k = expert.shape
    branch = np.zeros((T, y.shape[2]), np.float64)
    for i in range(k):
        m = np.flatnonzero(keep[:, i])
        branch[m] += gate[m, i, None] * y[expert[m, i], slot[m, i]]
    if residual is None:
        return branch
    return np.asarray(residual, np.float64) + branch


class AuxG(NamedTuple):
    f: np.ndarray        # [n_groups, E] counts / (k G)
    P: np.ndarray        # [n_groups, E] mean probability over the group
    loss: float          # alpha E mean_g sum_e f_ge P_ge
    dlogits: np.ndarray  # [T, E] with f held constant


def aux_loss_grouped(counts: np.ndarray, p: np.ndarray, G: int, k: int, alpha: float) -> AuxG:
    """The balance loss of [WQ] sec. 2 per routing group, averaged over the
    groups ([ZF] "evaluation protocol": metrics per 64-row batch, then the
    mean).  With k choices f counts the assignments and is divided by k G so
    that it sums to 1 over the experts and the balanced loss stays alpha.
    dL/dz_tj = (alpha E / T) p_tj (f_{g(t) j} - sum_e f_{g(t) e} p_te)."""
    p = np.asarray(p, np.float64)
    T, E = p.shape
    counts = np.asarray(counts, np.float64).reshape(-1, E)
    ng = counts.shape[0]
    if T == 0:
        return AuxG(np.zeros((ng, E)), np.zeros((ng, E)), 0.0, np.zeros((0, E)))
    f = counts / (k * G)
    P = p.reshape(ng, G, E).sum(axis=1) / G
    loss = float(alpha * E * np.mean(np.sum(f * P, axis=1)))
    fg = np.repeat(f, G, axis=0)                      # f of each token's group
    s = np.sum(fg * p, axis=1)
    dlogits = (alpha * E / T) * p * (fg - s[:, None])
    return AuxG(f, P, loss, dlogits)


class LayerResultG(NamedTuple):
    z: np.ndarray
    routing: RoutingK
    G: int
    Cg: int
    slots: SlotsG
    buf: np.ndarray
    y: np.ndarray
    branch: np.ndarray
    out: np.ndarray
    aux: AuxG


def layer_forward_grouped(x, w_r, b_r, w1, w2, c: float, alpha: float, k: int = 1, G: Optional[int] = None,
                          priority: str = "token", logits: Optional[np.ndarray] = None,
                          expert_override: Optional[np.ndarray] = None, Cg: Optional[int] = None) -> LayerResultG:
    """The layer with routing groups of G tokens (default: one group of T) and
    top-k choices, in the step order of [WQ] sec. 3."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    z = router_logits(x, w_r, b_r) if logits is None else np.asarray(logits, np.float64)
    E = z.shape[1]
    G = T if G is None else int(G)
    r = softmax_topk(z, k)
    if expert_override is not None:
        e = np.asarray(expert_override, np.int64).reshape(T, k)
        r = RoutingK(r.p, r.lse, e, np.take_along_axis(r.p, e, axis=1))
    if Cg is None:
        Cg = group_capacity(G, E, c, k)
    G = max(G, 1)   # an empty batch is zero groups of any size
    sl = slot_scan_grouped(r.expert, E, G, Cg, priority)
    aux = aux_loss_grouped(sl.counts, r.p, G, k, alpha)
    buf = dispatch(x, sl.slot_token)
    y = expert_ffn(buf, sl.accepted_total, w1, w2)
    branch = combine_topk(y, r.expert, sl.slot, sl.keep, r.gate, None)
    return LayerResultG(z, r, G, Cg, sl, buf, y, branch, x + branch, aux)


def layer_per_token_topk(x, z, w1, w2, k: int, G: int, Cg: int, priority: str = "token"):
    """Brute force for tiny inputs, with no shared state between tokens: each
    token's choices by repeated strict-greater scans over the logits that skip
    the experts already chosen, each choice's in-group position by counting
    the group's assignments that come before it in the chosen order and pick
    the same expert, and its branch by matrix-vector products."""
    x = np.asarray(x, np.float64)
    z = np.asarray(z, np.float64)
    T, E = z.shape
    choices = []
    for t in range(T):
        taken = []
        for _ in range(k):
            best = -1
            for e in range(E):
                if e in taken:
                    continue
                if best < 0 or z[t, e] > z[t, best]:
                    best = e
            taken.append(best)
        choices.append(taken)

    def before(a, b):  # does assignment a = (t, i) precede b in its group's order?
        (ta, ia), (tb, ib) = a, b
        return (ta, ia) < (tb, ib) if priority == "token" else (ia, ta) < (ib, tb)

    positions = np.zeros((T, k), np.int64)
    branch = np.zeros_like(x)
    for t in range(T):
        g0 = (t // G) * G
        denom = sum(math.exp(v) for v in z[t])
        for i in range(k):
            e = choices[t][i]
            pos = sum(1 for s in range(g0, g0 + G) for j in range(k)
                      if choices[s][j] == e and before((s, j), (t, i)))
            positions[t, i] = pos
            if pos < Cg:
                gte = math.exp(z[t, e]) / denom
                w1e = np.asarray(w1(e) if callable(w1) else w1[e], np.float64)
                w2e = np.asarray(w2(e) if callable(w2) else w2[e], np.float64)
                branch[t] += gte * (w2e @ np.maximum(w1e @ x[t], 0.0))
    return np.array(choices, np.int64), positions, branch


# ------------------------------------------------ NEXT f-2: layer backward
#
# The objective whose gradient is taken:  J = sum_t <dout_t, out_t> + L_aux
# (+ L_z when beta > 0), i.e. dout is the gradient flowing into the layer's
# output and the aux (and z) losses are added to the training loss with the
# weights they carry inside ([WQ] sec. 2: the total loss adds the balance
# term; the router stays differentiable through the selected gate).  The
# choices, positions and masks are held fixed: argmax has no gradient ([WQ]
# sec. 2; [ZF] "troubleshooting": finite differences that leave the discrete
# choices and capacity masks unchanged).
#
# Chain rule for a kept token t with expert e = e*_t, slot s = pos_t:
#   out_t = x_t + g_t y_t,  y_t = W2_e relu(a_t),  a_t = W1_e x_t,  g_t = p_{t,e}
#   dy_t = g_t dout_t                       dg_t = <dout_t, y_t>
#   dW2_e += dy_t relu(a_t)^T               dh_t = W2_e^T dy_t
#   da_t = dh_t * [a_t > 0]                 dW1_e += da_t x_t^T
#   dx_t = dout_t + W1_e^T da_t   (dropped tokens: dx_t = dout_t)
# Router, with p_tj = softmax(z_t)_j and d p_te / d z_tj = p_te (delta_ej - p_tj):
#   dz_tj = dg_t g_t (delta_{j e} - p_tj) + dL_aux/dz_tj (+ dL_z/dz_tj)
#   dW_r = x^T dz,  db_r = sum_t dz_t,  dx_t += W_r dz_t.

class LayerGrads(NamedTuple):
    dx: np.ndarray      # [T, d]
    dw_r: np.ndarray    # [d, E]
    db_r: np.ndarray    # [E]
    dw1: np.ndarray     # [E, d_ff, d]
    dw2: np.ndarray     # [E, d, d_ff]
    dz: np.ndarray      # [T, E] total gradient at the logits
    dgate: np.ndarray   # [T] <dout_t, y_t> for kept tokens, 0 for dropped ones


def layer_backward(x, w_r, b_r, w1, w2, c: float, alpha: float, dout, beta: float = 0.0,
                   C: Optional[int] = None, expert_override: Optional[np.ndarray] = None,
                   forward: Optional[LayerResult] = None, relu_active=None,
                   dw_experts: Optional[np.ndarray] = None) -> LayerGrads:
    """Gradients of J = sum_t <dout_t, out_t> + L_aux (+ L_z) for the Switch
    layer (one routing group, k = 1; layer_backward_grouped below covers
    routing groups and top-k), in float64, expert by expert.

    relu_active(e, a) may replace the ReLU derivative [a > 0] of expert e's
    kept rows (a: their pre-activations, tokens in order); tests use it to
    take the device's decision on pre-activations within rounding of zero,
    as `expert_override` does for near-tie choices.

    dw_experts, if given, lists the experts whose weight gradients are
    returned: dw1 and dw2 then hold only those experts, in that order (every
    other output is unchanged; this only bounds the memory of the result
    when E * d * d_ff is large)."""
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    L = forward if forward is not None else layer_forward(x, w_r, b_r, w1, w2, c, alpha, C=C,
                                                          expert_override=expert_override)
    T, d = x.shape
    E = L.z.shape[1]
    r, sl = L.routing, L.slots
    w1e = (lambda e: np.asarray(w1(e) if callable(w1) else w1[e], np.float64))
    w2e = (lambda e: np.asarray(w2(e) if callable(w2) else w2[e], np.float64))
    F = w1e(0).shape[0]
    dx = dout.copy()
    row_of = {e: e for e in range(E)} if dw_experts is None else {int(e): i for i, e in enumerate(dw_experts)}
    dw1 = np.zeros((len(row_of), F, d))
    dw2 = np.zeros((len(row_of), d, F))
    dgate = np.zeros(T)
    for e in range(E):
        toks = np.flatnonzero((r.expert == e) & sl.keep)
        if toks.size == 0:
            continue
        W1, W2 = w1e(e), w2e(e)
        xe = x[toks]
        a = xe @ W1.T                       # pre-activations [n, F]
        h = np.maximum(a, 0.0)
        y = h @ W2.T                        # [n, d]
        g = r.gate[toks]
        dgate[toks] = np.sum(dout[toks] * y, axis=1)
        dy = g[:, None] * dout[toks]
        j = row_of.get(e)
        if j is not None:
            dw2[j] = dy.T @ h
        active = (a > 0) if relu_active is None else relu_active(e, a)
        da = (dy @ W2) * active
        if j is not None:
            dw1[j] = da.T @ xe
        dx[toks] += da @ W1
    onehot = np.zeros((T, E))
    onehot[np.arange(T), r.expert] = 1.0
    dz = (dgate * r.gate)[:, None] * (onehot - r.p)
    dz = dz + L.aux.dlogits
    if beta:
        dz = dz + router_z_loss(L.z, beta).dlogits
    w_r64 = np.asarray(w_r, np.float64)
    dw_r = x.T @ dz
    db_r = dz.sum(axis=0)
    dx = dx + dz @ w_r64.T
    return LayerGrads(dx, dw_r, db_r, dw1, dw2, dz, dgate)


def layer_objective(x, w_r, b_r, w1, w2, c, alpha, dout, beta, expert, C):
    """J = sum <dout, out> + L_aux(f fixed from `expert`) + L_z at fixed
    choices `expert` and capacity C; used by the finite-difference pins."""
    L = layer_forward(x, w_r, b_r, w1, w2, c, alpha, C=C, expert_override=expert)
    J = float(np.sum(np.asarray(dout, np.float64) * L.out)) + L.aux.loss
    if beta:
        J += router_z_loss(L.z, beta).loss
    return J


# ------------------------------- layer backward with routing groups and top-k
#
# The same objective J = sum_t <dout_t, out_t> + L_aux (+ L_z), now for the
# layer of layer_forward_grouped: out_t = x_t + sum_i keep_ti g_ti y[e_ti, s_ti]
# with g_ti = p_{t, e_ti} (raw, not renormalised), and L_aux the mean over the
# groups of the per-group balance loss (f per group held fixed).  Every kept
# assignment (t, i) is one buffer row s = slot_ti of expert e = e_ti and gets
# the single-choice chain rule of layer_backward with its own gate; the
# token's input gradient adds the contributions of all its kept choices:
#   dgate_ti = <dout_t, y[e, s]>,  dy_s = g_ti dout_t,  da_s = (dy_s W2_e) * [a_s > 0]
#   dW2_e = sum_s dy_s relu(a_s)^T,  dW1_e = sum_s da_s x_t^T,  dx_t = dout_t + sum_i da_s W1_e
# and, since every gate is a softmax entry of the same row,
#   dz_tj = sum_i dgate_ti g_ti (delta_{j e_ti} - p_tj) + dL_aux/dz_tj (+ dL_z/dz_tj).
# Dropped choices contribute nothing (dgate_ti = 0).

class LayerGradsG(NamedTuple):
    dx: np.ndarray      # [T, d]
    dw_r: np.ndarray    # [d, E]
    db_r: np.ndarray    # [E]
    dw1: np.ndarray     # [E, d_ff, d]
    dw2: np.ndarray     # [E, d, d_ff]
    dz: np.ndarray      # [T, E]
    dgate: np.ndarray   # [T, k] <dout_t, y[e_ti, s_ti]> for kept choices, 0 for dropped ones


def layer_backward_grouped(x, w_r, b_r, w1, w2, c: float, alpha: float, dout, k: int = 1,
                           G: Optional[int] = None, priority: str = "token", beta: float = 0.0,
                           Cg: Optional[int] = None, expert_override: Optional[np.ndarray] = None,
                           forward: Optional[LayerResultG] = None, relu_active=None) -> LayerGradsG:
    """Gradients of J for the layer with routing groups of G tokens and k
    choices per token, in float64, expert by expert over its buffer rows
    (rows 0 .. accepted_total[e]-1, token slot_token[e, row]).  relu_active(e,
    a) may replace [a > 0] for expert e's filled rows, as in layer_backward."""
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    L = forward if forward is not None else layer_forward_grouped(
        x, w_r, b_r, w1, w2, c, alpha, k=k, G=G, priority=priority, expert_override=expert_override, Cg=Cg)
    T, d = x.shape
    E = L.z.shape[1]
    r, sl = L.routing, L.slots
    kk = r.expert.shape[1]
    w1e = (lambda e: np.asarray(w1(e) if callable(w1) else w1[e], np.float64))
    w2e = (lambda e: np.asarray(w2(e) if callable(w2) else w2[e], np.float64))
    F = w1e(0).shape[0]
    dx = dout.copy()
    dw1 = np.zeros((E, F, d))
    dw2 = np.zeros((E, d, F))
    dgate = np.zeros((T, kk))
    # the assignment that owns each buffer row
    owner = {}
    for t in range(T):
        for i in range(kk):
            if sl.keep[t, i]:
                owner[(int(r.expert[t, i]), int(sl.slot[t, i]))] = (t, i)
    for e in range(E):
        n = int(sl.accepted_total[e])
        if n == 0:
            continue
        rows = [owner[(e, s)] for s in range(n)]
        toks = np.array([t for t, _ in rows], np.int64)
        ranks = np.array([i for _, i in rows], np.int64)
        W1, W2 = w1e(e), w2e(e)
        xe = x[toks]
        acts = xe @ W1.T                    # pre-activations of the filled rows
        hid = np.maximum(acts, 0.0)
        yr = hid @ W2.T
        gr = r.gate[toks, ranks]
        dgate[toks, ranks] = np.sum(dout[toks] * yr, axis=1)
        dyr = gr[:, None] * dout[toks]
        dw2[e] = dyr.T @ hid
        on = (acts > 0) if relu_active is None else relu_active(e, acts)
        dar = (dyr @ W2) * on
        dw1[e] = dar.T @ xe
        np.add.at(dx, toks, dar @ W1)
    dz = np.zeros((T, E))
    for i in range(kk):
        onehot = np.zeros((T, E))
        onehot[np.arange(T), r.expert[:, i]] = 1.0
        dz += (dgate[:, i] * r.gate[:, i])[:, None] * (onehot - r.p)
    dz += L.aux.dlogits
    if beta:
        dz += router_z_loss(L.z, beta).dlogits
    wr = np.asarray(w_r, np.float64)
    dx += dz @ wr.T
    return LayerGradsG(dx, x.T @ dz, dz.sum(axis=0), dw1, dw2, dz, dgate)


def layer_objective_grouped(x, w_r, b_r, w1, w2, c, alpha, dout, beta, k, G, priority, expert, Cg):
    """J = sum <dout, out> + L_aux (f fixed from `expert`) + L_z for the grouped
    top-k layer at fixed choices and capacity; for the finite-difference pins."""
    L = layer_forward_grouped(x, w_r, b_r, w1, w2, c, alpha, k=k, G=G, priority=priority,
                              expert_override=expert, Cg=Cg)
    J = float(np.sum(np.asarray(dout, np.float64) * L.out)) + L.aux.loss
    if beta:
        J += router_z_loss(L.z, beta).loss
    return J
