"""GPU parity on seeded random layer shapes (a sweep over the configuration space).

Each case draws a layer — dtype, E, k, routing (learned top-k with or without
the log-Zipf bias, or random routed experts), T, d_model, d_ff, capacity
factor, activation, plain or GLU experts — and checks ``moe_forward`` and the
step-wise calls against the oracle on the same seeded inputs: routing, slots,
counts and gathered rows bit for bit, expert outputs and the layer output within
the output tolerance, and the two paths bit-identical to each other.  Router
weights are dyadic, so the logits are exact in any summation order and the
routing has a unique correct answer.  The shapes are small enough for the
oracle (float64, CPU) to finish each case in about a second; they still cross
every router block width, several GEMM tile sizes and ragged tails.  A second
set draws bf16 layers at capacity <= 64 with a wide FFN, the shapes whose
forward gathers the token rows in the up-projection and pairs the
down-projection's column tiles.
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from gpu_util import Dev, check_layer_output, check_routing, max_abs_rel, out_tol, raw_bits, to_host_f64

pytestmark = pytest.mark.gpu

E_CHOICES = (1, 2, 3, 7, 16, 33, 64, 100, 128, 129, 200, 256, 300)


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    E = int(rng.choice(E_CHOICES))
    divisors = [g for g in range(2, E + 1) if E % g == 0]
    route = "rre" if (divisors and rng.random() < 0.15) else "topk"
    k = 1 if route == "rre" else int(rng.integers(1, min(4, E) + 1))
    return W.Workload(
        f"sweep{seed}", T=int(rng.integers(1, 1201)), d_model=64 * int(rng.integers(1, 7)),
        d_ff=64 * int(rng.integers(1, 9)), E=E, k=k, capacity_factor=float(rng.uniform(0.3, 4.0)),
        act=str(rng.choice(["relu", "gelu"])), dtype=dtype, route=route,
        n_groups=int(rng.choice(divisors)) if route == "rre" else 1,
        zipf_s=1.1 if (route == "topk" and rng.random() < 0.3) else 0.0,
        seed=seed, rre_seed=seed + 7, glu=bool(rng.random() < 0.25))


def draw_capacity64(seed):
    """bf16 layers with capacity <= 64, d_model 384 or 768 and d_ff above 768: the forward's
    up-projection gathers the token rows itself (resident activations) and the
    down-projection runs on the paired 64 x 192 ring."""
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.choice((16, 40, 64)))
    k = 1 if seed < 3 else 2                             # top-1 and top-2, plain and GLU,
    T = int(rng.integers(16 * E, 48 * E + 1))            # both widths, with and without the
    cap = int(rng.integers(8, 65))                       # Zipf bias
    cf = float(cap * E / (k * T)) * float(rng.uniform(0.9, 1.0))
    return W.Workload(
        f"sweep64_{seed}", T=T, d_model=768 if seed % 2 == 0 else 384,
        d_ff=int(rng.choice((832, 1024, 1536))), E=E, k=k, capacity_factor=cf,
        act="gelu" if seed % 2 else "relu", dtype="bf16", route="topk",
        zipf_s=1.1 if seed in (2, 5) else 0.0, seed=100 + seed, glu=seed in (1, 4))


def _check_layer(wl, label):
    inputs = W.make_inputs(wl)
    ref = oracle.forward(wl, inputs)
    served = (ref["slot"] >= 0).any(axis=1)
    dev = Dev(wl, inputs)
    fw = dev.run_forward()
    check_routing(wl, fw, ref, f"{label} forward")
    check_layer_output(wl, to_host_f64(fw["y"]), ref["y"], served, f"{label} forward")
    steps = dev.run_steps()
    check_routing(wl, steps, ref, f"{label} steps")
    xe = raw_bits(steps["x_e"])
    ye = to_host_f64(steps["y_e"])
    for e in range(wl.E):
        n = int(ref["expert_count"][e])
        np.testing.assert_array_equal(xe[e, :n], inputs["x"][ref["slot_token"][e, :n]],
                                      err_msg=f"{label} x_e expert {e}")
        if n:
            err = max_abs_rel(ye[e, :n], ref["y_e"][e])
            assert err <= out_tol(wl), f"{label} y_e expert {e}: {err:.3g}"
    assert torch.equal(fw["y"], steps["y"]), f"{label}: forward and step-wise results differ"


@pytest.mark.parametrize("seed", range(32))
def test_random_layer_matches_oracle(seed):
    wl = draw(seed)
    print(f"[gpu] sweep {seed}: {wl}", flush=True)
    _check_layer(wl, f"sweep {seed}")


@pytest.mark.parametrize("seed", range(6))
def test_random_capacity64_layer_matches_oracle(seed):
    wl = draw_capacity64(seed)
    print(f"[gpu] sweep64 {seed}: {wl}", flush=True)
    _check_layer(wl, f"sweep64 {seed}")
