"""Planted mistakes: each plausible error in the oracle must make at least one pin fail.

The mistakes are planted in the oracle (on the CPU, through monkeypatch), never in
any GPU code.  A mutation "survives" if every listed pin still passes.
"""
import math

import numpy as np
import pytest

import oracle.moe_oracle as O
import oracle_pins as P

_orig = {n: getattr(O, n) for n in dir(O) if callable(getattr(O, n))}


def _cap_no_k(T, E, k, cf):
    return _orig["capacity"](T, E, 1, cf)


def _cap_floor(T, E, k, cf):
    from fractions import Fraction
    return int(math.floor(Fraction(k * T) * Fraction(cf) / E))


def _logits_no_bias(x, w_r, bias=None):
    return _orig["router_logits"](x, w_r, None)


def _logits_bias_in_f64(x, w_r, bias=None):
    h = O.as_f64(x) @ O.as_f64(w_r).T
    if bias is not None:
        h = h + np.asarray(bias, np.float64) * (1 + 2.0 ** -30)
    return h.astype(np.float32)


def _softmax_unnormalised(h):
    h = np.asarray(h, np.float64)
    return np.exp(h - h.max(axis=-1, keepdims=True))


def _topk_high_index_ties(h, k):
    h = np.asarray(h)
    E = h.shape[1]
    rev = _orig["topk"](h[:, ::-1], k)
    return (E - 1 - rev).astype(np.int32)


def _topk_smallest(h, k):
    return _orig["topk"](-np.asarray(h), k)


def _route_topk_renorm(x, w_r, bias, k):
    idx, gate, h = _orig["route_topk"](x, w_r, bias, k)
    g = gate.astype(np.float64)
    return idx, (g / g.sum(axis=1, keepdims=True)).astype(np.float32), h


def _dispatch_token_major(expert_idx, E, C):
    T, k = expert_idx.shape
    slot = np.full((T, k), -1, np.int32)
    count = np.zeros(E, np.int64)
    st = np.full((E, C), -1, np.int32)
    for t in range(T):
        for c in range(k):
            e = int(expert_idx[t, c])
            if 0 <= e < E and count[e] < C:
                slot[t, c] = count[e]
                st[e, count[e]] = t
                count[e] += 1
    return slot, count.astype(np.int32), st


def _dispatch_overfill(expert_idx, E, C):
    # off by one: lets each expert take C+1 assignments
    s, c, st = _orig["dispatch"](expert_idx, E, C + 1)
    return s, c, st[:, :C]


def _combine_no_gate(y_e, expert_idx, slot, gate, d_model):
    return _orig["combine"](y_e, expert_idx, slot, np.ones_like(gate), d_model)


def _combine_first_gate(y_e, expert_idx, slot, gate, d_model):
    g = np.repeat(gate[:, :1], gate.shape[1], axis=1)
    return _orig["combine"](y_e, expert_idx, slot, g, d_model)


def _act_tanh_gelu(z, act):
    if act == "gelu":
        return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    return _orig["act_fn"](z, act)


def _expert_apply_w2_untransposed(xrows, w1_e, w2_e, act, glu=False):
    hdn = O.expert_hidden(xrows, w1_e, act, glu)
    w2 = O.as_f64(w2_e)
    return hdn @ w2.reshape(w2.shape[1], w2.shape[0])


def _glu_hidden_variant(mode):
    def hidden(xrows, w1_e, act, glu=False):
        if not glu:
            return _orig["expert_hidden"](xrows, w1_e, act, glu)
        z = xrows @ O.as_f64(w1_e).T
        f = z.shape[1] // 2
        za, zb = z[:, :f], z[:, f:]
        if mode == "act_on_linear_branch":
            return za * O.act_fn(zb, act)
        if mode == "act_on_product":
            return O.act_fn(za * zb, act)
        if mode == "mispaired":
            return O.act_fn(za, act) * zb[:, ::-1]
        raise ValueError(mode)
    return hidden


def _backward_glu_variant(mode):
    """The oracle backward, with a planted mistake in the GLU part of dZ (test code only)."""
    def bwd(wl, inputs, fwd, dy, weights=None):
        if not getattr(wl, "glu", False):
            return _orig["backward"](wl, inputs, fwd, dy, weights)
        w1, w2 = inputs["w1"], inputs["w2"]
        dy = np.asarray(dy, np.float64)
        T, d, f, E, k = wl.T, wl.d_model, wl.d_ff, wl.E, wl.k
        x = O.as_f64(inputs["x"])
        dx, dw1, dw2, dgate = np.zeros((T, d)), np.zeros((E, 2 * f, d)), np.zeros((E, d, f)), np.zeros((T, k))
        topk_route = wl.route == "topk"
        p = O.softmax(fwd["logits"]) if topk_route else None
        for e in range(E):
            n = int(fwd["expert_count"][e])
            if n == 0:
                continue
            w1_e, w2_e = O.as_f64(w1[e]), O.as_f64(w2[e])
            owners = [O.served_choice(fwd, e, s) for s in range(n)]
            xe = x[[t for t, _ in owners]]
            z = xe @ w1_e.T
            za, zb = z[:, :f], z[:, f:]
            hdn = O.act_fn(za, wl.act) * zb
            ye = hdn @ w2_e.T
            g = np.array([p[t, e] if topk_route else 1.0 for t, _ in owners])
            dye = g[:, None] * dy[[t for t, _ in owners]]
            for s, (t, c) in enumerate(owners):
                dgate[t, c] = float(dy[t] @ ye[s])
            dw2[e] = dye.T @ hdn
            dh = dye @ w2_e
            if mode == "gate_half_uses_act_grad":
                dz = np.concatenate([dh * zb * O.act_grad(za, wl.act), dh * O.act_grad(za, wl.act)], axis=1)
            elif mode == "act_half_without_gate":
                dz = np.concatenate([dh * O.act_grad(za, wl.act), dh * O.act_fn(za, wl.act)], axis=1)
            else:
                raise ValueError(mode)
            dw1[e] = dz.T @ xe
            dxe = dz @ w1_e
            for s, (t, _) in enumerate(owners):
                dx[t] += dxe[s]
        dw_r = dbias = None
        if topk_route:
            dp = np.zeros((T, E))
            for t in range(T):
                for c in range(k):
                    if int(fwd["slot"][t, c]) >= 0:
                        dp[t, int(fwd["expert_idx"][t, c])] += dgate[t, c]
            dh_r = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            dx += dh_r @ O.as_f64(inputs["w_r"])
            dw_r = dh_r.T @ x
            dbias = dh_r.sum(axis=0) if inputs.get("bias") is not None else None
        return dict(dx=dx, dw1=dw1, dw2=dw2, dw_r=dw_r, dbias=dbias, dgate=dgate)
    return bwd


def _forward_rows_variant(mode):
    """forward_rows with one planted mistake: the second choice skipped, or the
    first choice's gate used for every choice (test code only)."""
    def rows_fn(wl, inputs, rows, weights, routing=None):
        if routing is None:
            routing = O.route_and_dispatch(wl, inputs)
        out = np.zeros((len(rows), wl.d_model))
        for i, t in enumerate(rows):
            for c in range(wl.k):
                s = int(routing["slot"][t, c])
                if s < 0 or (mode == "first_choice_only" and c >= 1):
                    continue
                e = int(routing["expert_idx"][t, c])
                w1_e, w2_e = weights(e)
                ye = O.expert_apply(O.as_f64(inputs["x"][t:t + 1]), w1_e, w2_e, wl.act, O.is_glu(wl))[0]
                g = routing["gate"][t, 0] if mode == "first_gate_for_all" else routing["gate"][t, c]
                out[i] += float(g) * ye
        return out
    return rows_fn


def _route_and_dispatch_no_capacity(wl, inputs):
    r = _orig["route_and_dispatch"](wl, inputs)
    idx = r["expert_idx"]
    slot, count, st = O.dispatch(idx, wl.E, wl.T * wl.k)
    return dict(r, slot=slot, expert_count=count, slot_token=st[:, :r["capacity"]])


def _splitmix_bad_shift(seed, n):
    out, state, M = [], seed, (1 << 64) - 1
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & M
        z = state
        z = ((z ^ (z >> 31)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        out.append(z ^ (z >> 31))
    return out


def _rre_shifted(group_id, E, n_groups, seed):
    T = len(group_id)
    r = O.splitmix64(seed, T + 1)[1:]
    size = E // n_groups
    idx = np.array([[int(g) * size + v % size] for g, v in zip(group_id, r)], np.int32)
    return idx, np.ones((T, 1), np.float32)


def _gelu_grad_no_density(z, act):
    if act == "gelu":
        return 0.5 * (1.0 + np.vectorize(math.erf)(z / math.sqrt(2.0)))
    return _orig["act_grad"](z, act)


def _backward_variant(mode):
    """The oracle backward with one planted mistake (test code only)."""
    def bwd(wl, inputs, fwd, dy, weights=None):
        if weights is None:
            w1, w2 = inputs["w1"], inputs["w2"]
            weights = lambda e: (w1[e], w2[e])  # noqa: E731
        dy = np.asarray(dy, np.float64)
        T, d, f, E, k = wl.T, wl.d_model, wl.d_ff, wl.E, wl.k
        x = O.as_f64(inputs["x"])
        dx, dw1, dw2, dgate = np.zeros((T, d)), np.zeros((E, f, d)), np.zeros((E, d, f)), np.zeros((T, k))
        topk_route = wl.route == "topk"
        p = O.softmax(fwd["logits"]) if topk_route else None
        for e in range(E):
            n = int(fwd["expert_count"][e])
            if n == 0:
                continue
            w1_e, w2_e = (O.as_f64(w) for w in weights(e))
            owners = [O.served_choice(fwd, e, s) for s in range(n)]
            xe = x[[t for t, _ in owners]]
            z = xe @ w1_e.T
            hdn = O.act_fn(z, wl.act)
            ye = hdn @ w2_e.T
            g = np.array([p[t, e] if topk_route else 1.0 for t, _ in owners])
            dye = dy[[t for t, _ in owners]] if mode == "no_gate" else g[:, None] * dy[[t for t, _ in owners]]
            for s, (t, c) in enumerate(owners):
                dgate[t, c] = float(dy[t] @ ye[s])
            dw2[e] = dye.T @ hdn
            dz = (dye @ w2_e) * O.act_grad(z, wl.act)
            dw1[e] = (xe.T @ dz).T if mode != "dw1_from_hidden" else dz.T @ np.tile(xe, (1, 1))[:, :d] * 0.5
            for s, (t, _) in enumerate(owners):
                dx[t] += (dz @ w1_e)[s]
        dw_r = dbias = None
        if topk_route:
            dp = np.zeros((T, E))
            for t in range(T):
                for c in range(k):
                    if int(fwd["slot"][t, c]) >= 0:
                        dp[t, int(fwd["expert_idx"][t, c])] += dgate[t, c]
            if mode == "jacobian_sign":
                dh = p * (np.sum(p * dp, axis=1, keepdims=True) - dp)
            elif mode == "jacobian_diag_only":
                dh = p * dp
            else:
                dh = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
            w_r = O.as_f64(inputs["w_r"])
            dx += dh @ w_r
            dw_r = dh.T @ x
            dbias = dh.sum(axis=0) if inputs.get("bias") is not None else None
        return dict(dx=dx, dw1=dw1, dw2=dw2, dw_r=dw_r, dbias=dbias, dgate=dgate)
    return bwd


def _sparse_clip_kappa_not_squared(grads, E, max_norm):
    dense = [g for g in (grads.get("dw_r"), grads.get("dbias")) if g is not None]
    sq_d = sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in dense)
    sq_m = sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in (grads["dw1"], grads["dw2"]))
    norm = math.sqrt(sq_d + sq_m / math.sqrt(E))
    coef = min(1.0, max_norm / (norm + 1e-6))
    return {k: (None if v is None else np.asarray(v, np.float64) * coef) for k, v in grads.items()}, norm, coef


ALL_PINS = [
    lambda rng: P.check_worked_fixture("switch_top1_worked.json"),
    lambda rng: P.check_worked_fixture("top2_priority_worked.json"),
    lambda rng: P.check_capacity_values(),
    P.check_capacity_bruteforce, P.check_logits_exact, P.check_logits_bias, P.check_softmax,
    P.check_topk_rank, P.check_gate_raw, lambda rng: P.check_splitmix_reference(), P.check_rre,
    P.check_dispatch_invariants, P.check_dispatch_no_drop, P.check_choice_priority,
    lambda rng: P.check_gelu_values(), P.check_dense_equals_sparse, P.check_single_expert_is_mlp,
    P.check_forward_rows, P.check_route_and_dispatch,
    P.check_glu_coordinate_gate, P.check_glu_linear_in_v,
    P.check_k_equals_E_is_softmax_mixture, P.check_expert_permutation, P.check_aux_loss,
    P.check_backward_autograd, P.check_backward_finite_differences,
    P.check_backward_single_expert_is_mlp, P.check_backward_rre_no_router_grad, P.check_sparse_clip,
]

MUTATIONS = {
    "capacity_without_k": ("capacity", _cap_no_k),
    "capacity_floor": ("capacity", _cap_floor),
    "logits_drop_bias": ("router_logits", _logits_no_bias),
    "logits_bias_rounded_wrong": ("router_logits", _logits_bias_in_f64),
    "softmax_unnormalised": ("softmax", _softmax_unnormalised),
    "topk_ties_to_high_index": ("topk", _topk_high_index_ties),
    "topk_smallest": ("topk", _topk_smallest),
    "gates_renormalised": ("route_topk", _route_topk_renorm),
    "dispatch_token_major": ("dispatch", _dispatch_token_major),
    "dispatch_overfill": ("dispatch", _dispatch_overfill),
    "combine_without_gate": ("combine", _combine_no_gate),
    "combine_wrong_choice_gate": ("combine", _combine_first_gate),
    "gelu_tanh_approximation": ("act_fn", _act_tanh_gelu),
    "w2_not_transposed": ("expert_apply", _expert_apply_w2_untransposed),
    "glu_act_on_linear_branch": ("expert_hidden", _glu_hidden_variant("act_on_linear_branch")),
    "glu_act_on_product": ("expert_hidden", _glu_hidden_variant("act_on_product")),
    "glu_units_mispaired": ("expert_hidden", _glu_hidden_variant("mispaired")),
    "backward_glu_gate_half_uses_act_grad": ("backward", _backward_glu_variant("gate_half_uses_act_grad")),
    "backward_glu_act_half_without_gate": ("backward", _backward_glu_variant("act_half_without_gate")),
    "forward_rows_first_choice_only": ("forward_rows", _forward_rows_variant("first_choice_only")),
    "forward_rows_first_gate_for_all": ("forward_rows", _forward_rows_variant("first_gate_for_all")),
    "route_and_dispatch_without_capacity": ("route_and_dispatch", _route_and_dispatch_no_capacity),
    "splitmix_wrong_shift": ("splitmix64", _splitmix_bad_shift),
    "rre_off_by_one_token": ("route_rre", _rre_shifted),
    "gelu_grad_without_density_term": ("act_grad", _gelu_grad_no_density),
    "backward_without_gate": ("backward", _backward_variant("no_gate")),
    "backward_softmax_jacobian_sign": ("backward", _backward_variant("jacobian_sign")),
    "backward_softmax_jacobian_diagonal": ("backward", _backward_variant("jacobian_diag_only")),
    "backward_dw1_wrong": ("backward", _backward_variant("dw1_from_hidden")),
    "sparse_clip_kappa_not_squared": ("sparse_clip", _sparse_clip_kappa_not_squared),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = 0
    for pin in ALL_PINS:
        try:
            pin(np.random.default_rng(7))
        except Exception:  # an assertion or a shape error both expose the mistake
            caught += 1
    assert caught > 0, f"planted mistake {name} survived every pin"
