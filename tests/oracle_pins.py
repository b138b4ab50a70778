"""Pin checks for the CPU oracle.

Each ``check_*`` function compares the oracle against something other than
itself: a hand-worked fixture, a closed form, a brute-force characterisation,
a second formulation of the same step, or a published generator output.  The
checks read the oracle through the module object ``O`` at call time, so the
mutation tests can plant a mistake in the oracle and confirm a pin fails.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


class _WL:
    """Minimal workload record for the oracle's ``forward``."""

    def __init__(self, **kw):
        self.route = "topk"
        self.n_groups = 1
        self.rre_seed = 0
        self.__dict__.update(kw)


# ---------------------------------------------------------------------------
# worked fixtures
# ---------------------------------------------------------------------------

def check_worked_fixture(name):
    g = load_golden(name)
    wl = _WL(T=g["T"], d_model=g["d_model"], d_ff=g["d_ff"], E=g["E"], k=g["k"],
             capacity_factor=g["capacity_factor"], act=g["act"])
    inputs = {"x": np.array(g["x"], np.float32), "w_r": np.array(g["w_r"], np.float32),
              "bias": None, "group_id": None,
              "w1": np.array(g["w1"], np.float32), "w2": np.array(g["w2"], np.float32)}
    r = O.forward(wl, inputs)
    assert r["capacity"] == g["capacity"]
    np.testing.assert_array_equal(r["expert_idx"], np.array(g["expert_idx"]))
    np.testing.assert_allclose(r["gate"], np.array(g["gate"]), rtol=1e-7, atol=0)
    np.testing.assert_array_equal(r["slot"], np.array(g["slot"]))
    np.testing.assert_array_equal(r["expert_count"], np.array(g["expert_count"]))
    np.testing.assert_array_equal(r["slot_token"], np.array(g["slot_token"]))
    np.testing.assert_allclose(r["y"], np.array(g["y"]), rtol=1e-6, atol=1e-12)


# ---------------------------------------------------------------------------
# capacity
# ---------------------------------------------------------------------------

def check_capacity_values():
    # The five layer shapes: (T, E, k, cf) -> capacity, by hand from Eq. 3 with k and ceil.
    assert O.capacity(512, 8, 1, 1.25) == 80        # 512/8*1.25 = 80
    assert O.capacity(8192, 128, 1, 1.0) == 64      # 8192/128 = 64
    assert O.capacity(16384, 64, 2, 2.0) == 1024    # 2*16384/64*2 = 1024
    assert O.capacity(8192, 64, 1, 1.25) == 160     # 8192/64*1.25 = 160
    assert O.capacity(32768, 256, 2, 1.25) == 320   # 2*32768/256*1.25 = 320
    assert O.capacity(10, 4, 1, 1.0) == 3           # 2.5 rounds up
    assert O.capacity(3, 3, 2, 1.0) == 2


def check_capacity_bruteforce(rng):
    for _ in range(200):
        T = int(rng.integers(1, 5000))
        E = int(rng.integers(1, 300))
        k = int(rng.integers(1, min(E, 4) + 1))
        cf = float(rng.choice([0.5, 1.0, 1.1, 1.25, 1.5, 2.0, 3.3, 0.07]))
        need = Fraction(k * T) * Fraction(cf)
        # smallest integer C with C * E >= k*T*cf, by search
        C = 0
        while C * E < need:
            C += 1
        assert O.capacity(T, E, k, cf) == C, (T, E, k, cf)


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------

def check_logits_exact(rng):
    T, d, E = 37, 96, 11
    xi = rng.integers(-8, 9, size=(T, d))
    wi = rng.integers(-8, 9, size=(E, d))
    x = (xi / 8).astype(np.float32)
    w = (wi / 8).astype(np.float32)
    h = O.router_logits(x, w)
    assert h.dtype == np.float32 and h.shape == (T, E)
    # integer arithmetic: h[t, e] = sum_j xi[t, j] * wi[e, j] / 64
    ref = np.array([[sum(int(xi[t, j]) * int(wi[e, j]) for j in range(d)) for e in range(E)]
                    for t in range(T)]) / 64.0
    np.testing.assert_array_equal(h.astype(np.float64), ref)


def check_logits_bias(rng):
    T, d, E = 9, 16, 7
    x = (rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float32)
    w = (rng.integers(-8, 9, size=(E, d)) / 8).astype(np.float32)
    b = (-1.1 * np.log(np.arange(1, E + 1))).astype(np.float32)
    h = O.router_logits(x, w, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, j])) * Fraction(float(w[e, j])) for j in range(d))
            s = exact + Fraction(float(b[e]))   # fits in float64 exactly
            assert h[t, e] == np.float32(float(s)), (t, e)


def check_softmax(rng):
    h = rng.normal(size=(50, 9)) * 3
    p = O.softmax(h)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (p > 0).all()
    # two experts: p_0 = 1 / (1 + exp(h_1 - h_0))
    h2 = rng.normal(size=(20, 2)) * 4
    p2 = O.softmax(h2)
    np.testing.assert_allclose(p2[:, 0], 1.0 / (1.0 + np.exp(h2[:, 1] - h2[:, 0])), rtol=1e-14)
    # equal logits -> uniform; one expert -> 1
    np.testing.assert_allclose(O.softmax(np.full((3, 5), 2.5)), 0.2, rtol=1e-15)
    np.testing.assert_array_equal(O.softmax(np.array([[7.0], [-3.0]])), [[1.0], [1.0]])
    # ratio of two gates = exp of the logit difference (Eq. 1)
    np.testing.assert_allclose(p[:, 3] / p[:, 5], np.exp(h[:, 3] - h[:, 5]), rtol=1e-12)


def check_topk_rank(rng):
    # logits on a coarse grid to force many ties, plus signed zeros
    for k in (1, 2, 3):
        h = (rng.integers(-2, 3, size=(200, 6)) * 0.5).astype(np.float32)
        h[0] = [0.0, -0.0, 0.0, -0.0, -1.0, -1.0]
        h[1] = [-0.0, 0.0, -0.5, -0.5, -0.5, -0.0]
        idx = O.topk(h, k)
        for t in range(h.shape[0]):
            assert len(set(idx[t].tolist())) == k
            for c in range(k):
                i = idx[t, c]
                # number of experts that beat i under (larger logit, then lower index)
                better = sum(1 for j in range(h.shape[1])
                             if h[t, j] > h[t, i] or (h[t, j] == h[t, i] and j < i))
                assert better == c, (t, c, h[t], idx[t])
    assert O.topk(np.array([[0.0, -0.0, 0.0]], np.float32), 2).tolist() == [[0, 1]]
    assert O.topk(np.array([[-0.0, 0.0]], np.float32), 1).tolist() == [[0]]


def check_gate_raw(rng):
    T, d, E = 40, 8, 5
    x = (rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float32)
    w = (rng.integers(-8, 9, size=(E, d)) / 8).astype(np.float32)
    idx, gate, h = O.route_topk(x, w, None, 2)
    hh = h.astype(np.float64)
    for t in range(T):
        z = sum(math.exp(v) for v in hh[t])
        for c in range(2):
            assert abs(float(gate[t, c]) - math.exp(hh[t, idx[t, c]]) / z) <= 1e-7 * gate[t, c]
        assert gate[t, 0] >= gate[t, 1]


def check_splitmix_reference():
    g = load_golden("splitmix64_reference.json")
    got = O.splitmix64(g["seed"], len(g["outputs_hex"]))
    assert [int(h, 16) for h in g["outputs_hex"]] == got


def check_rre(rng):
    E, G, T = 64, 4, 20000
    gid = rng.integers(0, G, size=T).astype(np.int32)
    idx, gate = O.route_rre(gid, E, G, seed=12345)
    size = E // G
    assert idx.shape == (T, 1) and (gate == 1.0).all()
    assert ((idx[:, 0] // size) == gid).all()
    # uniform within the group: chi-square over the 16 members of each group
    for g in range(G):
        members = idx[gid == g, 0] - g * size
        counts = np.bincount(members, minlength=size)
        exp = len(members) / size
        chi2 = float(((counts - exp) ** 2 / exp).sum())
        assert chi2 < 45.0, chi2       # 15 dof, p ~ 1e-4
    # the pick for token t is the t-th SplitMix64 output (not shifted by a token)
    r = O.splitmix64(7, 5)
    idx2, _ = O.route_rre(np.zeros(5, np.int32), 8, 1, seed=7)
    assert idx2[:, 0].tolist() == [v % 8 for v in r]
    bad, gbad = O.route_rre(np.array([0, 4, -1], np.int32), 8, 4, 0)
    assert bad[1, 0] == -1 and bad[2, 0] == -1 and gbad[1, 0] == 0.0


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------

def onehot_dispatch(expert_idx, E, C):
    """Second formulation: one-hot dispatch masks with cumulative sums.

    Position of each assignment in its expert's buffer = number of earlier
    assignments to that expert, counted with a cumulative sum over tokens for
    each choice, offset by the totals of all earlier choices.  Returns the
    dense dispatch tensor D[t, e, c] (0/1) of shape [T, E, C] plus slot.
    """
    T, k = expert_idx.shape
    D = np.zeros((T, E, C), np.int64)
    slot = np.full((T, k), -1, np.int64)
    offset = np.zeros(E, np.int64)
    for c in range(k):
        valid = (expert_idx[:, c] >= 0) & (expert_idx[:, c] < E)
        m = np.zeros((T, E), np.int64)
        m[np.nonzero(valid)[0], expert_idx[valid, c]] = 1
        pos = np.cumsum(m, axis=0) - 1 + offset[None, :]
        keep = (m == 1) & (pos < C)
        tt, ee = np.nonzero(keep)
        D[tt, ee, pos[tt, ee]] = 1
        slot[tt, c] = pos[tt, ee]
        offset += m.sum(axis=0)
    return D, slot


def check_dispatch_invariants(rng):
    for trial in range(60):
        T = int(rng.integers(1, 300))
        E = int(rng.integers(1, 12))
        k = int(rng.integers(1, min(E, 3) + 1))
        C = int(rng.integers(1, 2 * T // max(E, 1) + 3))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        if trial % 5 == 0:
            idx[rng.random(T) < 0.1, 0] = -1
        slot, count, slot_token = O.dispatch(idx, E, C)
        assert (count <= C).all()
        valid = ((idx >= 0) & (idx < E)).sum()
        assert count.sum() + ((slot < 0) & (idx >= 0)).sum() == valid
        for e in range(E):
            served = [(t, c) for c in range(k) for t in range(T) if idx[t, c] == e and slot[t, c] >= 0]
            assert len(served) == count[e]
            for t, c in served:
                assert slot_token[e, slot[t, c]] == t
            assert (slot_token[e, count[e]:] == -1).all()
        D, slot2 = onehot_dispatch(idx, E, C)
        np.testing.assert_array_equal(slot, slot2)


def check_dispatch_no_drop(rng):
    # capacity factor >= E/k makes capacity >= T: every token is served
    for _ in range(20):
        T = int(rng.integers(1, 200))
        E = int(rng.integers(2, 10))
        k = int(rng.integers(1, 3))
        cf = E / k
        C = O.capacity(T, E, k, cf)
        assert C >= T
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        slot, count, _ = O.dispatch(idx, E, C)
        assert (slot >= 0).all() and count.sum() == k * T


def check_choice_priority(rng):
    # a second choice is never served by an expert that dropped a first choice
    for _ in range(30):
        T, E, C = 120, 4, int(rng.integers(10, 40))
        idx = np.stack([rng.permutation(E)[:2] for _ in range(T)]).astype(np.int32)
        slot, count, _ = O.dispatch(idx, E, C)
        for e in range(E):
            dropped_first = ((idx[:, 0] == e) & (slot[:, 0] < 0)).any()
            if dropped_first:
                assert not ((idx[:, 1] == e) & (slot[:, 1] >= 0)).any()


# ---------------------------------------------------------------------------
# FFN and combine
# ---------------------------------------------------------------------------

def check_gelu_values():
    z = np.array([0.0, 1.0, -1.0, 2.0, -3.0])
    g = O.act_fn(z, "gelu")
    # Phi(1) = 0.8413447460685429 (standard normal CDF, textbook value)
    np.testing.assert_allclose(g[:3], [0.0, 0.8413447460685429, -0.15865525393145707], rtol=1e-14)
    # GELU(z) - GELU(-z) = z  (since Phi(z) + Phi(-z) = 1)
    zz = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(O.act_fn(zz, "gelu") - O.act_fn(-zz, "gelu"), zz, atol=1e-14)
    np.testing.assert_array_equal(O.act_fn(np.array([-2.0, 0.0, 3.5]), "relu"), [0.0, 0.0, 3.5])


def _rand_layer(rng, T, d, f, E, k, cf, act, zipf=False, ties=False, glu=False):
    wl = _WL(T=T, d_model=d, d_ff=f, E=E, k=k, capacity_factor=cf, act=act, glu=glu)
    x = (rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float32)
    w_r = (rng.integers(-8, 9, size=(E, d)) / 8).astype(np.float32)
    if not ties:
        # break every tie: distinct per-expert offsets far below the 1/64 grid
        bias = (np.arange(E) * 2.0 ** -12).astype(np.float32)
    else:
        bias = None
    if zipf:
        bias = (-1.1 * np.log(np.arange(1, E + 1))).astype(np.float32)
    w1 = (rng.normal(size=(E, 2 * f if glu else f, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.normal(size=(E, d, f)) / math.sqrt(f)).astype(np.float32)
    return wl, {"x": x, "w_r": w_r, "bias": bias, "group_id": None, "w1": w1, "w2": w2}


def dense_layer(wl, inputs, r):
    """Dense brute force: every expert on every token, masked by the served choices.

    Built from the one-hot dispatch tensor D and the combine tensor gate * D,
    evaluated with einsum over [T, E, C] (the dispatch/combine tensor form of
    Switch notes 2.4).
    """
    x = O.as_f64(inputs["x"])
    D, _ = onehot_dispatch(r["expert_idx"], wl.E, r["capacity"])
    Wc = np.zeros(D.shape)
    T, k = r["expert_idx"].shape
    for t in range(T):
        for c in range(k):
            e = r["expert_idx"][t, c]
            if 0 <= e < wl.E:
                Wc[t, e] += float(r["gate"][t, c]) * D[t, e]
    xe = np.einsum("tec,td->ecd", D, x)
    w1 = O.as_f64(inputs["w1"])
    w2 = O.as_f64(inputs["w2"])
    zz = np.einsum("ecd,efd->ecf", xe, w1)
    if getattr(wl, "glu", False):
        f = wl.d_ff
        hid = O.act_fn(zz[:, :, :f], wl.act) * zz[:, :, f:]
    else:
        hid = O.act_fn(zz, wl.act)
    ye = np.einsum("ecf,edf->ecd", hid, w2)
    return np.einsum("tec,ecd->td", Wc, ye)


def check_dense_equals_sparse(rng):
    for (T, d, f, E, k, cf, act, zipf) in [(64, 16, 24, 4, 1, 1.0, "relu", False),
                                           (90, 8, 12, 6, 2, 1.0, "gelu", False),
                                           (50, 16, 8, 5, 2, 0.5, "gelu", True),
                                           (33, 8, 8, 3, 3, 1.0, "relu", False)]:
        for glu in (False, True):
            wl, inp = _rand_layer(rng, T, d, f, E, k, cf, act, zipf, glu=glu)
            r = O.forward(wl, inp)
            np.testing.assert_allclose(r["y"], dense_layer(wl, inp, r), rtol=1e-12, atol=1e-12)


def _rows_cases(rng):
    """Small layers for the sampled-token path: top-1 with drops, top-2 whose second
    choices overflow, a Zipf bias, GLU experts, and RRE with invalid group ids."""
    cases = []
    wl, inp = _rand_layer(rng, 96, 16, 24, 4, 1, 0.75, "relu")
    cases.append(("top1_drops", wl, inp))
    wl, inp = _rand_layer(rng, 80, 8, 12, 5, 2, 1.0, "gelu")
    cases.append(("top2_second_choice_drops", wl, inp))
    wl, inp = _rand_layer(rng, 64, 16, 8, 6, 2, 0.8, "gelu", zipf=True)
    cases.append(("top2_zipf", wl, inp))
    wl, inp = _rand_layer(rng, 70, 8, 12, 4, 2, 1.25, "relu", glu=True)
    cases.append(("top2_glu", wl, inp))
    T, G, E = 90, 3, 6
    wl, inp = _rand_layer(rng, T, 8, 12, E, 1, 1.0, "gelu")
    wl.route, wl.n_groups, wl.rre_seed = "rre", G, 99
    gid = rng.integers(0, G, size=T).astype(np.int32)
    gid[[3, 17, 40]] = [-1, G, 7]
    inp["group_id"], inp["w_r"], inp["bias"] = gid, None, None
    cases.append(("rre_invalid_groups", wl, inp))
    return cases


def check_forward_rows(rng):
    """forward_rows (one token at a time) against the dense one-hot formulation of the
    whole layer and against forward's y, on rows that include dropped tokens and tokens
    with both choices served (Switch notes 2.1 Eq. 2, 2.2 dropping)."""
    for name, wl, inp in _rand_cases_checked(rng):
        r = O.forward(wl, inp)
        served = (r["slot"] >= 0).sum(axis=1)
        T = wl.T
        rows = [0, T - 1]
        rows += list(np.nonzero(served == 0)[0][:4])
        rows += list(np.nonzero(served >= 2)[0][:4])
        rows += list(np.nonzero((served == 1) & (r["slot"][:, 0] < 0))[0][:4])
        rows += list(rng.choice(T, size=6, replace=False))
        rows = np.array(sorted(set(int(t) for t in rows)))
        w1, w2 = inp["w1"], inp["w2"]
        got = O.forward_rows(wl, inp, rows, lambda e: (w1[e], w2[e]))
        np.testing.assert_allclose(got, dense_layer(wl, inp, r)[rows], rtol=1e-12, atol=1e-12,
                                   err_msg=name)
        np.testing.assert_allclose(got, r["y"][rows], rtol=1e-12, atol=1e-12, err_msg=name)
        assert (got[served[rows] == 0] == 0).all(), name


def _rand_cases_checked(rng):
    """The cases of ``_rows_cases`` after checking that each exercises what it names."""
    cases = _rows_cases(rng)
    for name, wl, inp in cases:
        r = O.forward(wl, inp)
        if "drops" in name or name == "top2_zipf":
            assert (r["slot"] < 0).any(), name
        if name == "top2_second_choice_drops":
            assert ((r["slot"][:, 0] >= 0) & (r["slot"][:, 1] < 0)).any(), name
            assert ((r["slot"] >= 0).sum(axis=1) == 2).any(), name
        if name == "rre_invalid_groups":
            assert (r["expert_idx"][:, 0] < 0).sum() == 3, name
    return cases


def check_route_and_dispatch(rng):
    """route_and_dispatch (routing for the sampled-token path) against the routing that
    forward returns, the one-hot dispatch formulation and a brute-force top-k
    (Switch notes 2.1 and 2.2)."""
    for name, wl, inp in _rows_cases(rng):
        rd = O.route_and_dispatch(wl, inp)
        r = O.forward(wl, inp)
        for key in ("expert_idx", "slot", "expert_count", "slot_token"):
            np.testing.assert_array_equal(rd[key], r[key], err_msg=f"{name}: {key}")
        np.testing.assert_array_equal(rd["gate"], r["gate"], err_msg=name)
        assert rd["capacity"] == r["capacity"]
        C = math.ceil(Fraction(wl.k * wl.T) * Fraction(wl.capacity_factor) / wl.E)
        assert rd["capacity"] == C, name
        _, slot2 = onehot_dispatch(rd["expert_idx"], wl.E, C)
        np.testing.assert_array_equal(rd["slot"], slot2, err_msg=name)
        if wl.route == "topk":
            # the logits themselves are pinned by the exact-arithmetic checks above; rank
            # those by brute force (value desc, index asc) and form the softmax in float64
            h = np.asarray(rd["logits"], np.float64)
            h_exact = O.as_f64(inp["x"]) @ O.as_f64(inp["w_r"]).T
            if inp["bias"] is not None:
                h_exact = h_exact + O.as_f64(inp["bias"])
            np.testing.assert_allclose(h, h_exact, rtol=1e-6, atol=1e-6, err_msg=name)
            for t in range(wl.T):
                order = sorted(range(wl.E), key=lambda e: (-h[t, e], e))
                assert list(rd["expert_idx"][t]) == order[:wl.k], name
                p = np.exp(h[t] - h[t].max())
                p /= p.sum()
                np.testing.assert_allclose(rd["gate"][t], p[order[:wl.k]], rtol=1e-6, err_msg=name)


def check_glu_coordinate_gate(rng):
    """GLU FFN (MosaicBERT review, methodology) reduced to the plain FFN: with every V
    row a multiple a_j of the unit vector of input coordinate i, unit j's gate is
    a_j x_i, so the GLU expert equals x_i times the plain expert whose w2 columns are
    scaled by a.  Pins which branch takes the activation, the order of the stacked
    halves and the pairing of W row j with V row j."""
    T, d, f = 20, 12, 10
    x = (rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float64)
    for act in ("relu", "gelu"):
        W = rng.normal(size=(f, d)) / math.sqrt(d)
        w2 = rng.normal(size=(d, f)) / math.sqrt(f)
        a = rng.normal(size=f)
        i = int(rng.integers(0, d))
        V = np.zeros((f, d))
        V[:, i] = a
        got = O.expert_apply(x, np.concatenate([W, V]), w2, act, glu=True)
        ref = x[:, i:i + 1] * O.expert_apply(x, W, w2 * a[None, :], act)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def check_glu_linear_in_v(rng):
    """The GLU expert is linear in V (x V enters the product once, unactivated):
    y(V1 + V2) = y(V1) + y(V2) and y(c V) = c y(V); with the coordinate-gate pin this
    ties the GLU expert to the plain one for every V."""
    T, d, f = 16, 8, 12
    x = (rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float64)
    for act in ("relu", "gelu"):
        W, V1, V2 = (rng.normal(size=(f, d)) for _ in range(3))
        w2 = rng.normal(size=(d, f))

        def y(V):
            return O.expert_apply(x, np.concatenate([W, V]), w2, act, glu=True)

        np.testing.assert_allclose(y(V1 + V2), y(V1) + y(V2), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y(-2.5 * V1), -2.5 * y(V1), rtol=1e-12, atol=1e-12)


def check_single_expert_is_mlp(rng):
    import torch
    T, d, f = 30, 12, 20
    for act in ("relu", "gelu"):
        wl, inp = _rand_layer(rng, T, d, f, 1, 1, 1.0, act, ties=True)
        inp["bias"] = None
        r = O.forward(wl, inp)
        assert (r["gate"] == 1.0).all() and (r["slot"][:, 0] == np.arange(T)).all()
        xt = torch.tensor(inp["x"], dtype=torch.float64)
        l1 = torch.nn.Linear(d, f, bias=False, dtype=torch.float64)
        l2 = torch.nn.Linear(f, d, bias=False, dtype=torch.float64)
        with torch.no_grad():
            l1.weight.copy_(torch.tensor(inp["w1"][0], dtype=torch.float64))
            l2.weight.copy_(torch.tensor(inp["w2"][0], dtype=torch.float64))
            a = torch.relu if act == "relu" else (lambda z: torch.nn.functional.gelu(z, approximate="none"))
            ref = l2(a(l1(xt))).numpy()
        np.testing.assert_allclose(r["y"], ref, rtol=1e-12, atol=1e-13)


def check_k_equals_E_is_softmax_mixture(rng):
    T, d, f, E = 25, 8, 10, 4
    wl, inp = _rand_layer(rng, T, d, f, E, E, float(E), "gelu")
    r = O.forward(wl, inp)
    assert (r["slot"] >= 0).all()
    x = O.as_f64(inp["x"])
    h = x @ O.as_f64(inp["w_r"]).T + O.as_f64(inp["bias"])
    p = np.exp(h) / np.exp(h).sum(axis=1, keepdims=True)
    ref = np.zeros((T, d))
    for e in range(E):
        z = x @ O.as_f64(inp["w1"][e]).T
        g = z * 0.5 * (1 + np.vectorize(math.erf)(z / math.sqrt(2)))
        ref += p[:, e:e + 1] * (g @ O.as_f64(inp["w2"][e]).T)
    # gates are float32, so agreement is to float32 rounding
    np.testing.assert_allclose(r["y"], ref, rtol=2e-7 * 4, atol=1e-7)


def check_expert_permutation(rng):
    T, d, f, E, k = 80, 16, 12, 6, 2
    wl, inp = _rand_layer(rng, T, d, f, E, k, 1.25, "gelu", ties=True)
    # distinct offsets far below the 1/64 logit grid make every row tie-free, so
    # the lowest-index tie rule never applies and relabelling is exact
    inp["bias"] = (rng.permutation(E) * 2.0 ** -12).astype(np.float32)
    r = O.forward(wl, inp)
    assert (np.diff(np.sort(r["logits"], axis=1), axis=1) != 0).all()
    perm = rng.permutation(E)           # new expert j is old expert perm[j]
    inv = np.argsort(perm)
    inp2 = dict(inp)
    for key in ("w_r", "bias", "w1", "w2"):
        inp2[key] = inp[key][perm]
    r2 = O.forward(wl, inp2)
    np.testing.assert_array_equal(r2["expert_idx"], inv[r["expert_idx"]])
    np.testing.assert_array_equal(r2["expert_count"], r["expert_count"][perm])
    np.testing.assert_array_equal(r2["slot"], r["slot"])
    np.testing.assert_allclose(r2["y"], r["y"], rtol=1e-13, atol=1e-13)


def check_aux_loss(rng):
    # uniform routing: f_i = P_i = 1/N -> loss = alpha (Switch notes 2.2 after Eq. 6)
    N = 8
    # all-equal logits: p_i = 1/N; every argmax ties to expert 0, f = (1, 0, ..., 0),
    # so loss = alpha * N * (1 * 1/N) = alpha
    logits = np.zeros((N * 5, N), np.float32)
    assert abs(O.aux_loss(logits) - 1e-2) < 1e-15
    # balanced argmax with near-uniform probabilities
    eps = 2.0 ** -30
    lg = np.zeros((N * 4, N))
    for t in range(N * 4):
        lg[t, t % N] = eps
    assert abs(O.aux_loss(lg, alpha=1.0) - 1.0) < 1e-6
    # hand-worked: N=2, tokens with logits [0, ln 3] and [0, 0]:
    # p = (1/4, 3/4) and (1/2, 1/2); f = (1/2, 1/2) (second row ties -> expert 0);
    # P = (3/8, 5/8); loss = alpha * 2 * (1/2*3/8 + 1/2*5/8) = alpha
    lg2 = np.array([[0.0, math.log(3.0)], [0.0, 0.0]])
    assert abs(O.aux_loss(lg2, alpha=1.0) - 1.0) < 1e-12
    # all tokens to expert 1 with p_1 = 3/4: f = (0, 1), P = (1/4, 3/4) -> 2 * 3/4 = 1.5
    lg3 = np.array([[0.0, math.log(3.0)]] * 3)
    assert abs(O.aux_loss(lg3, alpha=1.0) - 1.5) < 1e-12


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------


def _torch_dense_grads(wl, inp, r, dy):
    """Gradients of <y, dy> by torch autograd (float64) on a dense formulation: every
    expert on every token, y = sum_e m[t, e] softmax(h)[t, e] FFN_e(x_t), with m the
    served-choice mask from the oracle's dispatch held constant."""
    import torch
    T, E = wl.T, wl.E
    m = np.zeros((T, E))
    for t in range(T):
        for c in range(wl.k):
            if r["slot"][t, c] >= 0:
                m[t, r["expert_idx"][t, c]] = 1.0
    x = torch.tensor(O.as_f64(inp["x"]), requires_grad=True)
    w_r = torch.tensor(O.as_f64(inp["w_r"]), requires_grad=True)
    w1 = torch.tensor(O.as_f64(inp["w1"]), requires_grad=True)
    w2 = torch.tensor(O.as_f64(inp["w2"]), requires_grad=True)
    h = x @ w_r.T
    bias = None
    if inp.get("bias") is not None:
        bias = torch.tensor(O.as_f64(inp["bias"]), requires_grad=True)
        h = h + bias
    p = torch.softmax(h, dim=1)
    act = torch.relu if wl.act == "relu" else (lambda z: torch.nn.functional.gelu(z, approximate="none"))
    y = torch.zeros(T, wl.d_model, dtype=torch.float64)
    mt = torch.tensor(m)
    f = wl.d_ff
    for e in range(E):
        if getattr(wl, "glu", False):
            fe = (act(x @ w1[e][:f].T) * (x @ w1[e][f:].T)) @ w2[e].T
        else:
            fe = act(x @ w1[e].T) @ w2[e].T
        y = y + (mt[:, e] * p[:, e])[:, None] * fe
    (y * torch.tensor(dy)).sum().backward()
    out = dict(dx=x.grad.numpy(), dw_r=w_r.grad.numpy(), dw1=w1.grad.numpy(), dw2=w2.grad.numpy())
    out["dbias"] = bias.grad.numpy() if bias is not None else None
    return out


def check_backward_autograd(rng):
    # dyadic x and w_r: the float32 logits the oracle routes on equal the float64 ones;
    # the tiny bias only breaks ties (rounded to float32 once, like the oracle's)
    for (T, d, f, E, k, cf, act, zipf, glu) in [(40, 16, 24, 4, 1, 1.0, "gelu", False, False),
                                                (60, 8, 12, 6, 2, 1.0, "gelu", False, False),
                                                (50, 16, 8, 5, 2, 0.5, "relu", True, False),
                                                (24, 8, 8, 3, 3, 2.0, "gelu", False, False),
                                                (40, 16, 12, 4, 2, 1.0, "gelu", False, True),
                                                (36, 8, 8, 3, 1, 1.0, "relu", True, True)]:
        wl, inp = _rand_layer(rng, T, d, f, E, k, cf, act, zipf, glu=glu)
        if not zipf:
            inp["bias"] = None
            inp["x"] = inp["x"] + (rng.integers(0, 64, size=inp["x"].shape) / 512).astype(np.float32)
        r = O.forward(wl, inp)
        dy = rng.normal(size=(T, d))
        g = O.backward(wl, inp, r, dy)
        ref = _torch_dense_grads(wl, inp, r, dy)
        for key in ("dx", "dw_r", "dw1", "dw2"):
            scale = max(np.abs(ref[key]).max(), 1e-300)
            np.testing.assert_allclose(g[key] / scale, ref[key] / scale, atol=1e-6 if zipf else 1e-12,
                                       err_msg=key)
        if zipf:
            scale = np.abs(ref["dbias"]).max()
            np.testing.assert_allclose(g["dbias"] / scale, ref["dbias"] / scale, atol=1e-6)


def check_backward_finite_differences(rng):
    # central differences of L = <y, dy> in the expert weights (GELU: smooth; the
    # routing does not depend on w1, w2).  The router weight is pinned by autograd
    # instead: the forward stores float32 gates, whose rounding swamps a small step.
    # GLU: both halves of the stacked w1 (the activated W rows and the linear V rows)
    T, d, f, E, k = 30, 8, 10, 3, 2
    for glu in (False, True):
        wl, inp = _rand_layer(rng, T, d, f, E, k, 1.0, "gelu", glu=glu)
        inp["bias"] = None
        for key in ("w1", "w2"):
            inp[key] = inp[key].astype(np.float64)
        r = O.forward(wl, inp)
        dy = rng.normal(size=(T, d))
        g = O.backward(wl, inp, r, dy)

        def loss(i2):
            return float((O.forward(wl, i2)["y"] * dy).sum())

        for key, grad in (("w1", g["dw1"]), ("w2", g["dw2"])):
            picks = [tuple(int(rng.integers(0, n)) for n in inp[key].shape) for _ in range(6)]
            if glu and key == "w1":  # at least three entries in each half
                picks = [(e, (j % f) + (f if q >= 3 else 0), c) for q, (e, j, c) in enumerate(picks)]
            for idx in picks:
                eps = 1e-5
                ip, im = dict(inp), dict(inp)
                ip[key] = inp[key].copy(); ip[key][idx] += eps
                im[key] = inp[key].copy(); im[key][idx] -= eps
                fd = (loss(ip) - loss(im)) / (2 * eps)
                assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (glu, key, idx, fd, grad[idx])


def check_backward_single_expert_is_mlp(rng):
    # E = 1, k = 1, no drops: gate 1 (softmax of one logit), the layer is a 2-layer MLP;
    # torch.nn.Linear autograd gives dx, dW1, dW2, and the router gets no gradient
    import torch
    T, d, f = 30, 12, 20
    for act in ("relu", "gelu"):
        wl, inp = _rand_layer(rng, T, d, f, 1, 1, 1.0, act, ties=True)
        inp["bias"] = None
        r = O.forward(wl, inp)
        dy = rng.normal(size=(T, d))
        g = O.backward(wl, inp, r, dy)
        xt = torch.tensor(inp["x"], dtype=torch.float64, requires_grad=True)
        l1 = torch.nn.Linear(d, f, bias=False, dtype=torch.float64)
        l2 = torch.nn.Linear(f, d, bias=False, dtype=torch.float64)
        with torch.no_grad():
            l1.weight.copy_(torch.tensor(inp["w1"][0], dtype=torch.float64))
            l2.weight.copy_(torch.tensor(inp["w2"][0], dtype=torch.float64))
        a = torch.relu if act == "relu" else (lambda z: torch.nn.functional.gelu(z, approximate="none"))
        (l2(a(l1(xt))) * torch.tensor(dy)).sum().backward()
        np.testing.assert_allclose(g["dx"], xt.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dw1"][0], l1.weight.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dw2"][0], l2.weight.grad.numpy(), rtol=1e-12, atol=1e-12)
        assert np.abs(g["dw_r"]).max() == 0.0


def check_backward_rre_no_router_grad(rng):
    # random routed experts: gates are the constant 1, so dx is the expert path only and
    # equals the sum of the per-expert MLP input gradients of the tokens each expert serves
    T, d, f, E, G = 48, 8, 12, 8, 2
    wl = _WL(T=T, d_model=d, d_ff=f, E=E, k=1, capacity_factor=2.0, act="gelu", route="rre",
             n_groups=G)
    x = (rng.integers(-8, 9, size=(T, d)) / 8).astype(np.float32)
    w1 = (rng.normal(size=(E, f, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.normal(size=(E, d, f)) / math.sqrt(f)).astype(np.float32)
    inp = {"x": x, "w_r": None, "bias": None, "group_id": rng.integers(0, G, size=T).astype(np.int32),
           "w1": w1, "w2": w2}
    r = O.forward(wl, inp)
    dy = rng.normal(size=(T, d))
    g = O.backward(wl, inp, r, dy)
    assert g["dw_r"] is None and g["dbias"] is None
    import torch
    dx_ref = np.zeros((T, d))
    for t in range(T):
        e, s = int(r["expert_idx"][t, 0]), int(r["slot"][t, 0])
        if s < 0:
            continue
        xt = torch.tensor(O.as_f64(x[t:t + 1]), requires_grad=True)
        z = xt @ torch.tensor(O.as_f64(w1[e])).T
        yv = torch.nn.functional.gelu(z, approximate="none") @ torch.tensor(O.as_f64(w2[e])).T
        (yv * torch.tensor(dy[t:t + 1])).sum().backward()
        dx_ref[t] = xt.grad.numpy()[0]
    np.testing.assert_allclose(g["dx"], dx_ref, rtol=1e-12, atol=1e-12)


def check_sparse_clip(rng):
    import torch
    # E = 1: kappa = 1, the norm is the plain global 2-norm; torch's clip_grad_norm_ agrees
    g = {"dw_r": rng.normal(size=(1, 5)), "dbias": rng.normal(size=1),
         "dw1": rng.normal(size=(1, 6, 5)), "dw2": rng.normal(size=(1, 5, 6))}
    for max_norm in (0.5, 1e6):
        out, norm, coef = O.sparse_clip(g, 1, max_norm)
        ts = [torch.tensor(g[k], requires_grad=True) for k in ("dw_r", "dbias", "dw1", "dw2")]
        for t, k in zip(ts, ("dw_r", "dbias", "dw1", "dw2")):
            t.grad = torch.tensor(g[k])
        tn = float(torch.nn.utils.clip_grad_norm_(ts, max_norm))
        assert abs(norm - tn) <= 1e-12 * tn
        for t, k in zip(ts, ("dw_r", "dbias", "dw1", "dw2")):
            np.testing.assert_allclose(out[k], t.grad.numpy(), rtol=1e-12, atol=0)
        assert coef == (1.0 if max_norm > norm else coef) and coef <= 1.0
    # kappa = 1/sqrt(E): scaling every expert gradient by sqrt(E) and the dense ones by 1
    # gives the norm of the unscaled gradients with E = 1
    E = 16
    g2 = {"dw_r": rng.normal(size=(E, 4)), "dbias": None,
          "dw1": rng.normal(size=(E, 3, 4)), "dw2": rng.normal(size=(E, 4, 3))}
    _, n1, _ = O.sparse_clip(g2, 1, 1.0)
    g3 = dict(g2, dw1=g2["dw1"] * math.sqrt(E), dw2=g2["dw2"] * math.sqrt(E))
    _, n2, _ = O.sparse_clip(g3, E, 1.0)
    assert abs(n1 - n2) <= 1e-12 * n1
    # hand-worked: dense (3, 4) -> 25; experts all 2, 8 values, E = 4: 8*4/4 = 8 -> norm sqrt(33)
    g4 = {"dw_r": np.array([[3.0, 4.0]]), "dbias": None, "dw1": np.full((4, 1, 1), 2.0),
          "dw2": np.full((4, 1, 1), 2.0)}
    out, norm, coef = O.sparse_clip(g4, 4, 1.0)
    assert abs(norm - math.sqrt(33.0)) < 1e-12
    assert abs(coef - 1.0 / (math.sqrt(33.0) + 1e-6)) < 1e-15
    np.testing.assert_allclose(out["dw_r"], g4["dw_r"] * coef, rtol=1e-15)
