"""The seeded input generators: shapes, value grids, determinism, bf16 rounding."""
import numpy as np
import torch

import moe_workloads as W
from oracle import capacity


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    a = (rng.standard_normal(100000) * 10 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]   # ties to even
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(a), ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_small_inputs_deterministic_and_on_grid():
    for name, wl in W.TEST_WORKLOADS.items():
        a = W.make_inputs(wl)
        b = W.make_inputs(wl)
        for key in a:
            if a[key] is None:
                assert b[key] is None
            else:
                np.testing.assert_array_equal(a[key], b[key])
        x = a["x"]
        assert x.shape == (wl.T, wl.d_model)
        x32 = W.bf16_bits_to_f32(x) if wl.dtype == "bf16" else x
        assert set(np.unique(x32 * 8).tolist()) <= set(range(-8, 9))
        if wl.route == "topk":
            assert a["w_r"].shape == (wl.E, wl.d_model) and a["w_r"].dtype == np.float32
            assert set(np.unique(a["w_r"] * 8).tolist()) <= set(range(-8, 9))
        else:
            assert a["group_id"].min() >= 0 and a["group_id"].max() < wl.n_groups
        assert a["w1"].shape == (wl.E, W.w1_rows(wl), wl.d_model)
        assert a["w2"].shape == (wl.E, wl.d_model, wl.d_ff)
        # one expert regenerated alone equals its slice of the stack
        w1e, w2e = W.expert_weights(wl, wl.E - 1)
        np.testing.assert_array_equal(w1e, a["w1"][-1])
        np.testing.assert_array_equal(w2e, a["w2"][-1])


def test_weight_scale():
    wl = W.TEST_WORKLOADS["xmoe_small_bf16"]
    w1, w2 = W.expert_weights(wl, 0)
    s1 = W.bf16_bits_to_f32(w1).std() * np.sqrt(wl.d_model)
    s2 = W.bf16_bits_to_f32(w2).std() * np.sqrt(wl.d_ff)
    assert abs(s1 - 1) < 0.02 and abs(s2 - 1) < 0.02


def test_full_configs():
    assert [(w.T, w.d_model, w.d_ff, w.E, w.k) for w in W.WORKLOADS.values()] == [
        (512, 64, 256, 8, 1), (8192, 768, 3072, 128, 1), (16384, 1024, 4096, 64, 2),
        (8192, 2560, 10240, 64, 1), (32768, 2048, 8192, 256, 2)]
    wl = W.WORKLOADS["large_zipf_top2_bf16"]
    b = W.make_inputs(wl, with_weights=False)["bias"]
    np.testing.assert_allclose(b, -1.1 * np.log(np.arange(1, 257)), rtol=1e-7)


def test_long_contraction_cases_keep_their_shape():
    # a 2048-long contraction in the down- (first, capacity 161..384) and the GLU
    # up-projection (second, capacity above 384), with more than one 256-row block
    # per expert
    for name, k_len, lo, hi in (("longk_top2_bf16", "d_ff", 161, 384),
                                ("geglu_longk_bf16", "d_model", 385, 10 ** 9)):
        wl = W.TEST_WORKLOADS[name]
        c = capacity(wl.T, wl.E, wl.k, wl.capacity_factor)
        assert lo <= c <= hi and getattr(wl, k_len) >= 2048
        assert min(c, wl.T * wl.k / wl.E) > 256


def test_wide_long_contraction_cases_keep_their_shape():
    # N >= 2048 and K >= 2048 in the named GEMMs at a capacity in 161..384 with a
    # ragged last 128-row block
    for name in ("wide_longk_bf16", "geglu_wide_longk_bf16"):
        wl = W.TEST_WORKLOADS[name]
        c = capacity(wl.T, wl.E, wl.k, wl.capacity_factor)
        assert 161 <= c <= 384 and c % 128 != 0 and wl.T * wl.k / wl.E > c
        assert wl.d_model >= 2048 and W.w1_rows(wl) >= 2048
