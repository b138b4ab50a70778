"""GPU parity at the five full layer sizes, in the configuration the benchmark times.

moe_forward runs on the whole workload; the oracle recomputes routing and
dispatch for every token (bit-exact comparison of expert_idx, slot,
expert_count and slot_token, gates within tolerance), every expert's batch at
its tile-edge rows (x_e bit-exact for every row, H and y_e within tolerance),
and the layer output of a sample of tokens one by one (normwise max-abs-rel
within 2e-2 bf16 / 1e-5 fp32; dropped tokens exactly 0); the step-wise calls
give the same layer output bit for bit.
"""
import time

import numpy as np
import pytest

import moe_workloads as W
import oracle
from gpu_util import (Dev, check_backward, check_layer_output, check_router_aux, check_routing,
                      make_dy, to_host_f64)

pytestmark = pytest.mark.gpu


def _sample(ref, T, rng, n=40):
    served = (ref["slot"] >= 0).any(axis=1)
    picks = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    picks.update([0, T - 1])
    dropped = np.nonzero(~served)[0]
    picks.update(dropped[:6].tolist())
    two = np.nonzero((ref["slot"] >= 0).sum(axis=1) == 2)[0] if ref["slot"].shape[1] > 1 else []
    picks.update(list(two[:6]))
    return np.array(sorted(picks))


# gated-linear-unit forms of two layer shapes (GELU gate: the GeGLU form)
GLU_FULL = W.GLU_WORKLOADS


# rows of every expert's batch checked at full size: both sides of the 64-, 128- and
# 256-row tile edges of the grouped GEMMs, and the expert's last row
EDGE_ROWS = (0, 63, 64, 127, 128, 255, 256)


def _edge_rows(cnt):
    return sorted({r for r in EDGE_ROWS if r < cnt} | ({cnt - 1} if cnt > 0 else set()))


@pytest.mark.parametrize("name", list(W.WORKLOADS) + list(GLU_FULL))
def test_full_size_forward(name):
    """moe_forward at full size (the benchmark's launch configuration), then the
    step-wise calls on the same inputs: routing bit-exact for every token; the
    gathered rows x_e bit-exact for every expert and slot; the hidden rows H (from
    moe_forward's workspace) and the expert outputs y_e at the tile-edge rows of
    every expert within tolerance of the oracle; y on sampled tokens."""
    import torch
    import sparse_mixture_experts_13_amd as moe
    from gpu_util import max_abs_rel, out_tol, raw_bits
    wl = W.WORKLOADS.get(name) or GLU_FULL[name]
    t0 = time.time()
    print(f"[gpu] full {name}: generating inputs and the oracle's routing", flush=True)
    inputs = W.make_inputs(wl, with_weights=False)
    ref = oracle.route_and_dispatch(wl, inputs)
    counts = ref["expert_count"]
    glu = bool(getattr(wl, "glu", False))
    want_h, want_ye = {}, {}

    def on_expert(e, w1_e, w2_e):
        rr = _edge_rows(int(counts[e]))
        if rr:
            xr = oracle.as_f64(inputs["x"][ref["slot_token"][e, rr]])
            want_h[e] = oracle.expert_hidden(xr, w1_e, wl.act, glu)
            want_ye[e] = want_h[e] @ oracle.as_f64(w2_e).T

    dev = Dev(wl, inputs)
    dev.upload_weights_per_expert(on_expert)
    print(f"[gpu] full {name}: inputs ready {time.time() - t0:.1f}s; forward", flush=True)
    got = dev.run_forward()
    y = got["y"]
    check_routing(wl, got, ref, name)
    tol = out_tol(wl)
    hidden = moe.workspace_view(dev.ws, dev.cfg, "hidden")
    worst_h = 0.0
    for e, want in want_h.items():
        rr = _edge_rows(int(counts[e]))
        err = max_abs_rel(to_host_f64(hidden[e, rr]), want)
        assert err <= tol, f"{name} H expert {e} rows {rr}: {err:.3g}"
        worst_h = max(worst_h, err)
    print(f"[gpu] full {name}: H ok on {len(want_h)} experts (worst {worst_h:.3g}); step-wise calls",
          flush=True)
    steps = dev.run_steps()
    check_routing(wl, steps, ref, name + " step-wise")
    xe = raw_bits(steps["x_e"])
    x = inputs["x"]
    for e in range(wl.E):
        n = int(counts[e])
        np.testing.assert_array_equal(xe[e, :n], x[ref["slot_token"][e, :n]], err_msg=f"{name} x_e expert {e}")
    del xe
    worst_ye, n_rows = 0.0, 0
    for e, want in want_ye.items():
        rr = _edge_rows(int(counts[e]))
        err = max_abs_rel(to_host_f64(steps["y_e"][e, rr]), want)
        assert err <= tol, f"{name} y_e expert {e} rows {rr}: {err:.3g}"
        worst_ye, n_rows = max(worst_ye, err), n_rows + len(rr)
    # the same kernels on the same values (moe_forward's up-projection may read the
    # token rows through slot_token instead of x_e): identical bits
    assert torch.equal(steps["y"], y), \
        f"{name} forward and step-wise y differ by {max_abs_rel(to_host_f64(steps['y']), to_host_f64(y)):.3g}"
    del steps
    torch.cuda.empty_cache()
    rows = _sample(ref, wl.T, np.random.default_rng(1))
    print(f"[gpu] full {name}: x_e exact on {wl.E} experts, y_e on {n_rows} rows of {len(want_ye)} experts "
          f"(worst {worst_ye:.3g}); oracle on {len(rows)} sampled tokens", flush=True)
    y_ref = oracle.forward_rows(wl, inputs, rows, lambda e: W.expert_weights(wl, e), ref)
    y_got = to_host_f64(y[rows.tolist()])
    served = (ref["slot"][rows] >= 0).any(axis=1)
    err = check_layer_output(wl, y_got, y_ref, served, name)
    drops = int((ref["slot"] < 0).sum())
    print(f"[gpu] full {name}: ok, y err {err:.3g}, drops {drops}, {time.time() - t0:.1f}s", flush=True)


def test_full_size_fused_ffn_switch_base():
    """moe_expert_ffn_fused on the Switch-Base shape equals moe_expert_ffn bit for bit."""
    import torch
    import sparse_mixture_experts_13_amd as moe
    from gpu_util import raw_bits
    wl = W.WORKLOADS["switch_base_bf16"]
    print("[gpu] full fused ffn switch_base_bf16", flush=True)
    inputs = W.make_inputs(wl, with_weights=False)
    dev = Dev(wl, inputs)
    dev.upload_weights_per_expert()
    steps = dev.run_steps()
    y_e = torch.zeros_like(steps["y_e"])
    moe.expert_ffn_fused(dev.cfg, steps["x_e"], steps["expert_count"], dev.w1, dev.w2, y_e)
    torch.cuda.synchronize()
    counts = steps["expert_count"].cpu().numpy()
    a, b = raw_bits(steps["y_e"]), raw_bits(y_e)
    for e in range(wl.E):
        n = int(counts[e])
        np.testing.assert_array_equal(b[e, :n], a[e, :n], err_msg=f"fused y_e expert {e}")


@pytest.mark.parametrize("name", ["switch_base_bf16", "large_zipf_top2_bf16"])
def test_full_size_router_aux(name):
    """moe_router_aux at full size: Eq. 4-6 against the oracle on the same logits."""
    wl = W.WORKLOADS[name]
    print(f"[gpu] full router aux {name}", flush=True)
    inputs = W.make_inputs(wl, with_weights=False)
    dev = Dev(wl, inputs)
    idx, gate, aux = dev.run_router_aux(alpha=1e-2)
    err = check_router_aux(wl, inputs, idx, gate, aux, 1e-2, name)
    print(f"[gpu] full router aux {name}: loss {aux[0]:.6g}, rel err {err:.3g}", flush=True)


@pytest.mark.parametrize("name", ["switch_base_bf16", "switch_base_geglu_bf16"])
def test_full_size_backward_switch_base(name):
    """moe_backward on the Switch-Base layer (plain and GeGLU experts) against the
    oracle's float64 backward (all gradients, every token and expert)."""
    wl = W.WORKLOADS.get(name) or GLU_FULL[name]
    t0 = time.time()
    print(f"[gpu] full backward {name}: inputs", flush=True)
    inputs = W.make_inputs(wl)
    dev = Dev(wl, inputs)
    dy = make_dy(wl)
    got = dev.run_backward(dy)
    print(f"[gpu] full backward {name}: oracle ({time.time() - t0:.1f}s)", flush=True)
    fwd = oracle.forward(wl, inputs)
    ref = oracle.backward(wl, inputs, fwd, oracle.as_f64(dy))
    errs = check_backward(wl, got, ref, name)
    print(f"[gpu] full backward {name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items())
          + f" ({time.time() - t0:.1f}s)", flush=True)
