"""CPU oracle of the sparse Mixture-of-Experts layer: forward pass, and its backward pass.

TEST INFRASTRUCTURE. This module is the slow, obviously-correct reference the
GPU library is checked against.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP library (no kernels, headers, tables or helpers).

Arithmetic: float64 NumPy/SciPy from the exact input values, with no
intermediate rounding except where the method itself fixes a precision (the
router's float32 logits, see ``router_logits``).  Every function cites the
passage of the source pages it follows:

  [Switch]   "Switch Transformers: Scaling to Trillion Parameter Models with
             Simple and Efficient Sparsity" (aipapernotes notes), sections
             2.1 (Eq. 1, Eq. 2), 2.2 (Eq. 3 - Eq. 6) and 2.4 (selective precision).
  [X-MoE]    "TorchScale: Transformers at Scale" (nubint.ai review), proposed
             method: X-MoE with top-1 and top-2 routing.
  [PanGu]    "PanGu-Sigma: Towards Trillion Parameter Language Model with Sparse
             Heterogeneous Computing" (nubint.ai review), proposed method:
             Random Routed Experts (RRE).
  [Mosaic]   "MosaicBERT: A Bidirectional Encoder Optimized for Fast
             Pretraining" (nubint.ai review), methodology: gated linear units
             in the feed-forward layer (the GLU expert variant).

Where the pages leave a step open, the reading taken is stated at the function.

Pinned by tests/test_oracle_*.py against closed forms, brute force, a second
formulation (one-hot dispatch/combine tensors), hand-worked fixtures in
tests/golden/ and the published SplitMix64 outputs.  The sampled-token path used
at full layer size (``forward_rows``, ``route_and_dispatch``) is pinned against
the dense one-hot formulation and a brute-force top-k on small layers with drops,
two served choices, a Zipf bias, GLU experts and invalid RRE groups.  Every
function here has a pin; none is "parity unpinned".

Array conventions: bf16 tensors are np.uint16 raw bit patterns, fp32 tensors
np.float32 (see ``as_f64``).
"""
from __future__ import annotations

from fractions import Fraction
import math
from typing import Callable, Optional

import numpy as np
from scipy.special import erf

# ---------------------------------------------------------------------------
# storage decoding
# ---------------------------------------------------------------------------


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored tensor (uint16 = bf16 bit patterns, else float)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# O1: capacity
# ---------------------------------------------------------------------------


def capacity(T: int, E: int, k: int, capacity_factor: float) -> int:
    """Expert capacity, [Switch] 2.2 Eq. 3: (tokens per batch / experts) x capacity factor.

    Readings: "tokens per batch" is every token of the call, flattened; the
    count is multiplied by k because each token occupies k expert slots (2.1
    notes that routing to one expert lets capacity be at least halved); the
    fractional value is rounded up.  Evaluated exactly on the rational value of
    the float ``capacity_factor``.
    """
    num = Fraction(k * T) * Fraction(capacity_factor)
    return int(math.ceil(num / E))


# ---------------------------------------------------------------------------
# O2-O4: router
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_r: np.ndarray, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits h(x) = W_r . x, [Switch] 2.1, as float32 [T, E].

    [Switch] 2.4 (selective precision) runs the router in float32.  The dot
    product is taken in float64 and rounded once to float32; on the dyadic
    input grid (products are multiples of 1/64, |h| < 2^18) it is exact, so any
    float32 summation order gives the same value.  The per-expert bias is then
    added with one float32 rounding.
    """
    h = as_f64(x) @ as_f64(w_r).T
    h32 = h.astype(np.float32)
    if bias is not None:
        h32 = (h32 + np.asarray(bias, np.float32)).astype(np.float32)
    return h32


def softmax(h: np.ndarray) -> np.ndarray:
    """Gate values p_i(x) = exp(h_i) / sum_j exp(h_j), [Switch] 2.1 Eq. 1 (float64)."""
    h = np.asarray(h, np.float64)
    z = np.exp(h - h.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def topk(h: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, [Switch] 2.1 (the set T of top-k indices).

    Order: larger logit first; equal logits go to the lower expert index (the
    pages name no tie rule; lowest index is the reading taken).  Selecting on
    the logits h rather than on p keeps ties exact (p is monotone in h).
    Returns int32 [T, k], column c = the token's (c+1)-th choice.
    """
    h = np.asarray(h)
    T, E = h.shape
    idx = np.empty((T, k), np.int32)
    experts = np.arange(E)
    for t in range(T):
        # primary key: -h (descending logit); secondary: expert index (ascending)
        order = np.lexsort((experts, -h[t].astype(np.float64)))
        idx[t] = order[:k]
    return idx


def route_topk(x, w_r, bias, k: int):
    """Learned top-k routing ([Switch] 2.1; top-1 Switch / top-2 [X-MoE]).

    Returns (expert_idx int32 [T,k], gate float32 [T,k], logits float32 [T,E]).
    The gate of a choice is the raw softmax probability p_i(x) of Eq. 1 over all
    experts, not renormalised over the chosen ones (Eq. 2 uses p_i directly).
    """
    h = router_logits(x, w_r, bias)
    p = softmax(h)
    idx = topk(h, k)
    gate = np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32)
    return idx, gate, h


# SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014; the mixing function with the constants of
# Java's SplittableRandom / Vigna's splitmix64.c).
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1


def splitmix64(seed: int, n: int) -> list:
    """The first n outputs of SplitMix64 started from state ``seed`` (Python ints).

    Output i: state_i = seed + (i+1)*gamma mod 2^64, then three xor-shift /
    multiply rounds.
    """
    out = []
    state = seed & _MASK
    for _ in range(n):
        state = (state + _GAMMA) & _MASK
        z = state
        z = ((z ^ (z >> 30)) * _M1) & _MASK
        z = ((z ^ (z >> 27)) * _M2) & _MASK
        out.append(z ^ (z >> 31))
    return out


def route_rre(group_id: np.ndarray, E: int, n_groups: int, seed: int):
    """Random Routed Experts, [PanGu] proposed method.

    Experts are split into ``n_groups`` consecutive groups of E/n_groups; a
    token of group g goes to one expert of that group, uniformly at random and
    without any learned gate.  Reading: the random pick for token t is
    SplitMix64's t-th output for ``seed`` reduced modulo the group size, and the
    gate is 1 (a weightless gate leaves the expert output unscaled).  A group
    id outside [0, n_groups) routes the token nowhere (index -1, gate 0).
    Returns (expert_idx int32 [T,1], gate float32 [T,1]).
    """
    T = len(group_id)
    size = E // n_groups
    r = splitmix64(seed, T)
    idx = np.empty((T, 1), np.int32)
    gate = np.empty((T, 1), np.float32)
    for t in range(T):
        g = int(group_id[t])
        if 0 <= g < n_groups:
            idx[t, 0] = g * size + (r[t] % size)
            gate[t, 0] = 1.0
        else:
            idx[t, 0] = -1
            gate[t, 0] = 0.0
    return idx, gate


# ---------------------------------------------------------------------------
# O5-O6: capacity-limited dispatch and gather
# ---------------------------------------------------------------------------


def dispatch(expert_idx: np.ndarray, E: int, C: int):
    """Capacity-limited slot assignment, [Switch] 2.2 (Eq. 3 and the dropping rule).

    Assignments are visited choice by choice and, within a choice, in token
    order (every first choice is placed before any second choice); each takes
    the next free slot of its expert, and an assignment that finds its expert
    full is dropped (its slot is -1: the token skips that expert and only the
    residual carries it).  Indices outside [0, E) are not routed (slot -1).

    Returns slot int32 [T,k], expert_count int32 [E] (<= C) and
    slot_token int32 [E,C] (token held by each slot, -1 where empty).
    """
    T, k = expert_idx.shape
    slot = np.full((T, k), -1, np.int32)
    count = np.zeros(E, np.int64)
    slot_token = np.full((E, C), -1, np.int32)
    for c in range(k):
        for t in range(T):
            e = int(expert_idx[t, c])
            if not (0 <= e < E):
                continue
            if count[e] < C:
                slot[t, c] = count[e]
                slot_token[e, count[e]] = t
                count[e] += 1
    return slot, count.astype(np.int32), slot_token


def gather(x: np.ndarray, slot_token: np.ndarray, expert_count: np.ndarray) -> list:
    """Expert-major batches: rows of x in slot order, one float64 array per expert.

    Row s of expert e is the token in slot s ([Switch] 2.2: each expert computes
    a static-size batch of its tokens).
    """
    xf = as_f64(x)
    return [xf[slot_token[e, :expert_count[e]]] for e in range(len(expert_count))]


# ---------------------------------------------------------------------------
# O7: expert FFN
# ---------------------------------------------------------------------------


def act_fn(z: np.ndarray, act: str) -> np.ndarray:
    """ReLU max(0, z), or GELU with the exact Gaussian CDF: z * (1 + erf(z / sqrt 2)) / 2."""
    if act == "relu":
        return np.maximum(z, 0.0)
    if act == "gelu":
        return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))
    raise ValueError(act)


def expert_hidden(xrows: np.ndarray, w1_e: np.ndarray, act: str, glu: bool = False) -> np.ndarray:
    """Hidden activations H of one expert on a batch of rows (float64).

    Plain FFN ([Switch] 2.1): H = act(x W1), W1 = w1_e^T, w1_e stored [d_ff, d_model].
    GLU FFN ([Mosaic] methodology, gated linear units in the feed-forward layer):
    H = act(x W) * (x V), the product elementwise.  Reading taken where the page is
    silent: the activation is the layer's (ReLU or exact GELU), it is applied to the
    x W branch only, and the two projections are stored stacked in one matrix
    w1_e [2 d_ff, d_model], rows 0 .. d_ff - 1 being W^T and rows d_ff .. 2 d_ff - 1
    being V^T, so both come from one product x w1_e^T.
    """
    z = xrows @ as_f64(w1_e).T
    if not glu:
        return act_fn(z, act)
    f = z.shape[1] // 2
    return act_fn(z[:, :f], act) * z[:, f:]


def expert_apply(xrows: np.ndarray, w1_e: np.ndarray, w2_e: np.ndarray, act: str,
                 glu: bool = False) -> np.ndarray:
    """One expert E_i on a batch of rows: H W2 with H from ``expert_hidden`` and
    W2 = w2_e^T, w2_e stored [d_model, d_ff] (output x input).  float64."""
    return expert_hidden(xrows, w1_e, act, glu) @ as_f64(w2_e).T


def expert_ffn(x_e: list, weights: Callable[[int], tuple], act: str, glu: bool = False) -> list:
    """Apply every expert to its batch; ``weights(e)`` returns (w1_e, w2_e)."""
    out = []
    for e, rows in enumerate(x_e):
        if len(rows) == 0:
            out.append(np.zeros((0, rows.shape[1] if rows.ndim == 2 else 0)))
            continue
        w1_e, w2_e = weights(e)
        out.append(expert_apply(rows, w1_e, w2_e, act, glu))
    return out


def is_glu(wl) -> bool:
    """Whether a workload record uses the GLU expert FFN (records without the field do not)."""
    return bool(getattr(wl, "glu", False))


# ---------------------------------------------------------------------------
# O8: combine
# ---------------------------------------------------------------------------


def combine(y_e: list, expert_idx: np.ndarray, slot: np.ndarray, gate: np.ndarray,
            d_model: int) -> np.ndarray:
    """y = sum_{i in T} p_i(x) E_i(x), [Switch] 2.1 Eq. 2, over the served choices only.

    A choice that was dropped contributes nothing; a token with every choice
    dropped gets an all-zero layer output ([Switch] 2.2: it reaches the next
    layer through the residual, which is outside this layer).  float64.
    """
    T, k = expert_idx.shape
    y = np.zeros((T, d_model))
    for t in range(T):
        for c in range(k):
            s = int(slot[t, c])
            if s >= 0:
                y[t] += float(gate[t, c]) * y_e[int(expert_idx[t, c])][s]
    return y


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------


def route(wl, inputs):
    """Router step for a workload: learned top-k or RRE."""
    if wl.route == "rre":
        idx, gate = route_rre(inputs["group_id"], wl.E, wl.n_groups, wl.rre_seed)
        return idx, gate, None
    return route_topk(inputs["x"], inputs["w_r"], inputs["bias"], wl.k)


def forward(wl, inputs, weights: Optional[Callable[[int], tuple]] = None) -> dict:
    """The full layer: router -> dispatch -> gather -> expert FFN -> combine.

    ``inputs`` holds x, w_r, bias, group_id and (unless ``weights`` is given) the
    stacked expert weights w1 [E, d_ff, d_model] ([E, 2 d_ff, d_model] for the GLU
    FFN, see ``expert_hidden``), w2 [E, d_model, d_ff].
    Returns every intermediate: expert_idx, gate, logits, slot, expert_count,
    slot_token, x_e (list), y_e (list) and y [T, d_model] (float64).
    """
    if weights is None:
        w1, w2 = inputs["w1"], inputs["w2"]
        weights = lambda e: (w1[e], w2[e])  # noqa: E731
    C = capacity(wl.T, wl.E, wl.k, wl.capacity_factor)
    idx, gate, logits = route(wl, inputs)
    slot, count, slot_token = dispatch(idx, wl.E, C)
    x_e = gather(inputs["x"], slot_token, count)
    y_e = expert_ffn(x_e, weights, wl.act, is_glu(wl))
    y = combine(y_e, idx, slot, gate, wl.d_model)
    return dict(capacity=C, expert_idx=idx, gate=gate, logits=logits, slot=slot,
                expert_count=count, slot_token=slot_token, x_e=x_e, y_e=y_e, y=y)


def forward_rows(wl, inputs, rows: np.ndarray, weights: Callable[[int], tuple],
                 routing: Optional[dict] = None) -> np.ndarray:
    """Layer output for a sample of tokens, computed one token at a time.

    Routing and dispatch are computed for the whole call (a token's slot depends
    on every earlier token); the expert FFN runs only on the sampled tokens.
    Returns float64 [len(rows), d_model].
    """
    if routing is None:
        routing = route_and_dispatch(wl, inputs)
    xf = inputs["x"]
    out = np.zeros((len(rows), wl.d_model))
    cache = {}
    for i, t in enumerate(rows):
        for c in range(wl.k):
            s = int(routing["slot"][t, c])
            if s < 0:
                continue
            e = int(routing["expert_idx"][t, c])
            if e not in cache:
                cache[e] = weights(e)
            w1_e, w2_e = cache[e]
            ye = expert_apply(as_f64(xf[t:t + 1]), w1_e, w2_e, wl.act, is_glu(wl))[0]
            out[i] += float(routing["gate"][t, c]) * ye
    return out


def route_and_dispatch(wl, inputs) -> dict:
    """Router + dispatch for the whole call (no expert work)."""
    C = capacity(wl.T, wl.E, wl.k, wl.capacity_factor)
    idx, gate, logits = route(wl, inputs)
    slot, count, slot_token = dispatch(idx, wl.E, C)
    return dict(capacity=C, expert_idx=idx, gate=gate, logits=logits, slot=slot,
                expert_count=count, slot_token=slot_token)


# ---------------------------------------------------------------------------
# NEXT: load-balancing auxiliary loss
# ---------------------------------------------------------------------------


def aux_loss(logits: np.ndarray, alpha: float = 1e-2) -> float:
    """Load-balancing loss, [Switch] 2.2 Eq. 4-6: alpha * N * sum_i f_i P_i.

    f_i: fraction of the T tokens whose argmax p(x) is expert i (Eq. 5; argmax
    ties go to the lowest index, as in ``topk``); P_i: mean router probability
    of expert i (Eq. 6).  float64.
    """
    T, N = logits.shape
    top1 = topk(logits, 1)[:, 0]
    f = np.bincount(top1, minlength=N) / T
    P = softmax(logits).mean(axis=0)
    return float(alpha * N * np.sum(f * P))


# ---------------------------------------------------------------------------
# NEXT: backward pass of the layer
# ---------------------------------------------------------------------------


def act_grad(z: np.ndarray, act: str) -> np.ndarray:
    """Derivative of ``act_fn``: ReLU 1 where z > 0 and 0 elsewhere (the value at the kink
    z = 0 is taken as 0); GELU d/dz [z Phi(z)] = Phi(z) + z phi(z) with the standard normal
    density phi(z) = exp(-z^2 / 2) / sqrt(2 pi)."""
    if act == "relu":
        return (z > 0.0).astype(np.float64)
    if act == "gelu":
        cdf = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
        pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
        return cdf + z * pdf
    raise ValueError(act)


def served_choice(fwd: dict, e: int, s: int) -> tuple:
    """(token, choice) that holds slot s of expert e."""
    t = int(fwd["slot_token"][e, s])
    for c in range(fwd["expert_idx"].shape[1]):
        if int(fwd["expert_idx"][t, c]) == e and int(fwd["slot"][t, c]) == s:
            return t, c
    raise AssertionError("slot map inconsistent")


def backward(wl, inputs, fwd: dict, dy: np.ndarray,
             weights: Optional[Callable[[int], tuple]] = None) -> dict:
    """Gradients of the layer for an upstream gradient dy = dL/dy [T, d_model] (float64).

    The layer is [Switch] 2.1 Eq. 2, y(x) = sum over the served choices c of
    p_{i_c}(x) E_{i_c}(x), with p = softmax(h) (Eq. 1), h = W_r x (+ bias) and
    E_i(x) = act(x W1_i) W2_i; the gate keeps the router differentiable (2.1).
    The chosen set and the capacity drop ([Switch] 2.2) are piecewise constant in
    the inputs, so no gradient flows through them: this is the derivative
    wherever they do not switch, and a dropped choice contributes nothing.
    Per served choice (token t, choice c, expert e, slot s):
      expert term: dE = p_e dy[t]; with Z = x W1_e, H = act(Z), E = H W2_e:
        dW2_e += dE^T H, dH = dE W2_e^T, dZ = dH * act'(Z),
        dW1_e += dZ^T x, dx[t] += dZ W1_e^T;
      GLU FFN (``expert_hidden``): Z = (Za, Zb) = (x W, x V), H = act(Za) * Zb, so
        dZ = (dH * Zb * act'(Za), dH * act(Za)) over the stacked w1 rows;
      gate term: dp_e(t) = dy[t] . E_e(x_t), and through the softmax Jacobian
        dh = p * (dp - <p, dp>), then dx[t] += dh W_r, dW_r += dh^T x, dbias += dh.
    Random routed experts have constant gates 1: no router gradient (dw_r, dbias None).
    Weights are taken at their stored values (``weights(e)`` -> (w1_e, w2_e) in the
    stored [d_ff, d_model] / [d_model, d_ff] layout), every product in float64.
    Returns dx [T, d], dw1 [E, f, d] ([E, 2f, d] for GLU), dw2 [E, d, f], dw_r [E, d] or None,
    dbias [E] or None, dgate [T, k] (dL/dp of each served choice, 0 if dropped).
    """
    if weights is None:
        w1, w2 = inputs["w1"], inputs["w2"]
        weights = lambda e: (w1[e], w2[e])  # noqa: E731
    dy = np.asarray(dy, np.float64)
    T, d, f, E, k = wl.T, wl.d_model, wl.d_ff, wl.E, wl.k
    x = as_f64(inputs["x"])
    dx = np.zeros((T, d))
    glu = is_glu(wl)
    dw1 = np.zeros((E, 2 * f if glu else f, d))
    dw2 = np.zeros((E, d, f))
    dgate = np.zeros((T, k))
    topk_route = wl.route == "topk"
    p = softmax(fwd["logits"]) if topk_route else None
    for e in range(E):
        n = int(fwd["expert_count"][e])
        if n == 0:
            continue
        w1_e, w2_e = (as_f64(w) for w in weights(e))
        owners = [served_choice(fwd, e, s) for s in range(n)]
        xe = x[[t for t, _ in owners]]
        z = xe @ w1_e.T
        if glu:
            za, zb = z[:, :f], z[:, f:]
            hdn = act_fn(za, wl.act) * zb
        else:
            hdn = act_fn(z, wl.act)
        ye = hdn @ w2_e.T
        g = np.array([p[t, e] if topk_route else 1.0 for t, _ in owners])
        dye = g[:, None] * dy[[t for t, _ in owners]]
        for s, (t, c) in enumerate(owners):
            dgate[t, c] = float(dy[t] @ ye[s])
        dw2[e] = dye.T @ hdn
        dhdn = dye @ w2_e
        if glu:
            dz = np.concatenate([dhdn * zb * act_grad(za, wl.act), dhdn * act_fn(za, wl.act)], axis=1)
        else:
            dz = dhdn * act_grad(z, wl.act)
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
        dh = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        w_r = as_f64(inputs["w_r"])
        dx += dh @ w_r
        dw_r = dh.T @ x
        dbias = dh.sum(axis=0) if inputs.get("bias") is not None else None
    return dict(dx=dx, dw1=dw1, dw2=dw2, dw_r=dw_r, dbias=dbias, dgate=dgate)


# ---------------------------------------------------------------------------
# NEXT: SparseClip gradient clipping
# ---------------------------------------------------------------------------


def sparse_clip(grads: dict, E: int, max_norm: float) -> tuple:
    """SparseClip ([X-MoE] TorchScale review, methodology): gradient clipping whose norm
    re-weights the MoE (expert) gradients by kappa = 1/sqrt(E), balancing them against the
    dense ones: norm = ||(g_dense, kappa * g_moe)||_2.

    Reading taken where the page is silent: the dense gradients of this layer are the
    router's (dw_r, dbias), the MoE gradients the experts' (dw1, dw2); the clipping
    coefficient is min(1, max_norm / (norm + 1e-6)) applied to every gradient, the usual
    clip-by-global-norm rule.  float64.  Returns (clipped gradients, norm, coefficient).
    """
    dense = [g for g in (grads.get("dw_r"), grads.get("dbias")) if g is not None]
    moe = [grads["dw1"], grads["dw2"]]
    sq_dense = sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in dense)
    sq_moe = sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in moe)
    norm = math.sqrt(sq_dense + sq_moe / E)
    coef = min(1.0, max_norm / (norm + 1e-6))
    out = {k: (None if v is None else np.asarray(v, np.float64) * coef) for k, v in grads.items()}
    return out, norm, coef
