"""Seeded synthetic workloads for the sparse MoE layer forward.

This module is shared by the tests, the benchmark and the oracle's tests. It
holds no arithmetic of the MoE method itself (no routing, softmax, dispatch,
FFN or combine): it only names the workloads and draws their input arrays.

Array conventions (NumPy, host memory):
  * bf16 tensors are ``np.uint16`` arrays of raw bfloat16 bit patterns;
    fp32 tensors are ``np.float32``.
  * ``x``        [T, d_model]        layer input, config dtype
  * ``w_r``      [E, d_model] f32    router weight (learned routing only)
  * ``bias``     [E] f32 or None     per-expert router logit bias (Zipf skew)
  * ``group_id`` [T] int32 or None   expert group of each token (RRE only)
  * ``w1[e]``    [d_ff, d_model]     expert up-projection, stored out x in
                 ([2 d_ff, d_model] for the GLU FFN: the activated projection's
                 rows, then the linear gate projection's rows)
  * ``w2[e]``    [d_model, d_ff]     expert down-projection, stored out x in

Value distributions follow the workload descriptions of the Switch/X-MoE/
PanGu-Sigma layer shapes: router inputs and router weights are integers in
[-8, 8] divided by 8 (so every product is a multiple of 1/64 and fp32 logits
are exact in any summation order); expert weights are normal with standard
deviation 1/sqrt(fan_in), drawn in fp32 and rounded to nearest-even bf16 for
the bf16 workloads.  Every tensor has its own child stream of
``np.random.SeedSequence(seed)``; each expert's weights have their own grand-
child stream, so any expert can be regenerated alone.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Callable, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "GLU_WORKLOADS", "TEST_WORKLOADS", "get", "make_inputs",
    "expert_weights", "w1_rows", "f32_to_bf16_bits", "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    d_ff: int
    E: int
    k: int
    capacity_factor: float
    act: str                 # "relu" | "gelu"
    dtype: str               # "f32" | "bf16"
    route: str = "topk"      # "topk" | "rre"
    n_groups: int = 1
    zipf_s: float = 0.0      # > 0: add log-Zipf(s) per-expert bias to the logits
    seed: int = 0
    rre_seed: int = 0
    # "dyadic" (integers/8) or "gauss" (N(0, 1/d_model) rounded to fp32) router weight
    w_r_dist: str = "dyadic"
    glu: bool = False        # gated-linear-unit expert FFN (w1 holds 2 * d_ff rows)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five layer shapes (name -> sizes).  Descriptions:
#  tiny_switch_f32      Tiny Switch layer, fp32, top-1, ReLU
#  switch_base_bf16     Switch-Base-shaped layer (8 sequences x 1024 tokens), top-1, ReLU
#  xmoe_top2_bf16       X-MoE-shaped top-2 layer, raw softmax gates, GELU
#  rre_4x16_bf16        random-routed-experts layer, 4 groups x 16 experts, GELU
#  large_zipf_top2_bf16 large top-2 layer with log-Zipf(1.1) logit skew, GELU
WORKLOADS = {
    "tiny_switch_f32": Workload("tiny_switch_f32", T=512, d_model=64, d_ff=256, E=8, k=1,
                                capacity_factor=1.25, act="relu", dtype="f32"),
    "switch_base_bf16": Workload("switch_base_bf16", T=8192, d_model=768, d_ff=3072, E=128,
                                 k=1, capacity_factor=1.0, act="relu", dtype="bf16"),
    "xmoe_top2_bf16": Workload("xmoe_top2_bf16", T=16384, d_model=1024, d_ff=4096, E=64, k=2,
                               capacity_factor=2.0, act="gelu", dtype="bf16"),
    "rre_4x16_bf16": Workload("rre_4x16_bf16", T=8192, d_model=2560, d_ff=10240, E=64, k=1,
                              capacity_factor=1.25, act="gelu", dtype="bf16", route="rre",
                              n_groups=4),
    "large_zipf_top2_bf16": Workload("large_zipf_top2_bf16", T=32768, d_model=2048, d_ff=8192,
                                     E=256, k=2, capacity_factor=1.25, act="gelu",
                                     dtype="bf16", zipf_s=1.1),
}

# Gated-linear-unit (GeGLU) forms of two layer shapes: w1 holds 2 * d_ff rows.
GLU_WORKLOADS = {
    "switch_base_geglu_bf16": WORKLOADS["switch_base_bf16"].replace(name="switch_base_geglu_bf16",
                                                                    act="gelu", glu=True),
    "xmoe_top2_geglu_bf16": WORKLOADS["xmoe_top2_bf16"].replace(name="xmoe_top2_geglu_bf16", glu=True),
}

# Reduced shapes of the same five kinds: small enough for the full oracle in
# seconds, large enough to span several router blocks, several GEMM tiles and
# ragged tails (T, counts and d_ff not multiples of the tile sizes).
TEST_WORKLOADS = {
    "tiny_switch_f32": WORKLOADS["tiny_switch_f32"],
    "switch_small_bf16": Workload("switch_small_bf16", T=1000, d_model=256, d_ff=576, E=16, k=1,
                                  capacity_factor=1.0, act="relu", dtype="bf16"),
    "xmoe_small_bf16": Workload("xmoe_small_bf16", T=1237, d_model=320, d_ff=704, E=12, k=2,
                                capacity_factor=2.0, act="gelu", dtype="bf16"),
    "rre_small_bf16": Workload("rre_small_bf16", T=777, d_model=384, d_ff=512, E=16, k=1,
                               capacity_factor=1.25, act="gelu", dtype="bf16", route="rre",
                               n_groups=4),
    "zipf_small_bf16": Workload("zipf_small_bf16", T=2048, d_model=256, d_ff=512, E=40, k=2,
                                capacity_factor=1.25, act="gelu", dtype="bf16", zipf_s=1.1),
    # d_model a multiple of 384 with capacity <= 64 (the single-pass expert FFN),
    # top-1 with two 384-column groups per expert, and top-2 with one
    "wide_top1_bf16": Workload("wide_top1_bf16", T=1500, d_model=768, d_ff=384, E=24, k=1,
                               capacity_factor=1.0, act="gelu", dtype="bf16"),
    "wide_top2_bf16": Workload("wide_top2_bf16", T=1200, d_model=384, d_ff=256, E=40, k=2,
                               capacity_factor=1.0, act="relu", dtype="bf16"),
    # gated-linear-unit experts, one per grouped-GEMM capacity range: C = 63 (384-row
    # weight tiles), 100, 150, 230 and 500 (256 x 256 tiles), and float32
    "geglu_wide_top1_bf16": Workload("geglu_wide_top1_bf16", T=1500, d_model=768, d_ff=384, E=24,
                                     k=1, capacity_factor=1.0, act="gelu", dtype="bf16", glu=True),
    "reglu_c100_bf16": Workload("reglu_c100_bf16", T=1000, d_model=256, d_ff=320, E=10, k=1,
                                capacity_factor=1.0, act="relu", dtype="bf16", glu=True),
    "geglu_c150_bf16": Workload("geglu_c150_bf16", T=1500, d_model=256, d_ff=192, E=10, k=1,
                                capacity_factor=1.0, act="gelu", dtype="bf16", glu=True),
    "geglu_top2_bf16": Workload("geglu_top2_bf16", T=1100, d_model=320, d_ff=448, E=12, k=2,
                                capacity_factor=1.25, act="gelu", dtype="bf16", glu=True),
    "reglu_c500_bf16": Workload("reglu_c500_bf16", T=3000, d_model=256, d_ff=256, E=6, k=1,
                                capacity_factor=1.0, act="relu", dtype="bf16", glu=True),
    "reglu_small_f32": Workload("reglu_small_f32", T=600, d_model=128, d_ff=192, E=8, k=1,
                                capacity_factor=1.25, act="relu", dtype="f32", glu=True),
    # capacities above 160 with a contraction of 2048: the down-projection (K = d_ff)
    # of a top-2 GELU layer at capacity 315 (every expert full, two 256-row blocks)
    # with 128 output columns (half a 256-row weight tile), and the GeGLU
    # up-projection (K = d_model) at capacity 480
    "longk_top2_bf16": Workload("longk_top2_bf16", T=900, d_model=128, d_ff=2048, E=4, k=2,
                                capacity_factor=0.7, act="gelu", dtype="bf16"),
    "geglu_longk_bf16": Workload("geglu_longk_bf16", T=900, d_model=2048, d_ff=192, E=3, k=1,
                                 capacity_factor=1.6, act="gelu", dtype="bf16", glu=True),
    # 2048 x 2048 projections at capacity 315 (three 128-row blocks, the last one
    # ragged): both GEMMs of the plain layer and the GLU up-projection of the second
    # (2 x 1024 w1 rows) have at least four 512-row column blocks
    "wide_longk_bf16": Workload("wide_longk_bf16", T=700, d_model=2048, d_ff=2048, E=2, k=1,
                                capacity_factor=0.9, act="gelu", dtype="bf16"),
    "geglu_wide_longk_bf16": Workload("geglu_wide_longk_bf16", T=700, d_model=2048, d_ff=1024, E=2,
                                      k=1, capacity_factor=0.9, act="gelu", dtype="bf16", glu=True),
    # capacity 100 with d_model 1024 and d_ff 2048: the backward's dZ product (K = 1024,
    # N = 2048) on the ping-pong GEMM at a capacity below 161
    "mid_wide_bf16": Workload("mid_wide_bf16", T=600, d_model=1024, d_ff=2048, E=6, k=1,
                              capacity_factor=1.0, act="gelu", dtype="bf16"),
    # d_ff = 2112: the last 512-row column tile of the up-projection and of the backward's
    # dZ holds 64 rows, and the down-projection's contraction is 66 stages of 32
    "wide_ragged_bf16": Workload("wide_ragged_bf16", T=700, d_model=2048, d_ff=2112, E=2, k=1,
                                 capacity_factor=0.9, act="gelu", dtype="bf16"),
}


def get(name: str) -> Workload:
    for table in (WORKLOADS, GLU_WORKLOADS):
        if name in table:
            return table[name]
    return TEST_WORKLOADS[name]


# ---------------------------------------------------------------------------
# bf16 bit helpers (storage format only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); return the raw 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

_STREAMS = ("x", "w_r", "group_id", "w1", "w2")


def _children(wl: Workload) -> dict:
    kids = np.random.SeedSequence(wl.seed).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, kids))


def _dyadic(rng: np.random.Generator, shape) -> np.ndarray:
    """Integers uniform on {-8, ..., 8} divided by 8, as fp32 (exact)."""
    return (rng.integers(-8, 9, size=shape, dtype=np.int8).astype(np.float32) / np.float32(8.0))


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def w1_rows(wl: Workload) -> int:
    """Rows of one expert's w1: d_ff, or 2 * d_ff for the GLU FFN."""
    return 2 * wl.d_ff if wl.glu else wl.d_ff


def expert_weights(wl: Workload, e: int):
    """(w1[e] [w1_rows, d_model], w2[e] [d_model, d_ff]) in the workload dtype."""
    kids = _children(wl)
    s1 = kids["w1"].spawn(wl.E)[e]
    s2 = kids["w2"].spawn(wl.E)[e]
    r1 = np.random.Generator(np.random.PCG64(s1))
    r2 = np.random.Generator(np.random.PCG64(s2))
    w1 = r1.standard_normal((w1_rows(wl), wl.d_model), dtype=np.float32)
    w1 *= np.float32(1.0 / math.sqrt(wl.d_model))
    w2 = r2.standard_normal((wl.d_model, wl.d_ff), dtype=np.float32)
    w2 *= np.float32(1.0 / math.sqrt(wl.d_ff))
    return _store(w1, wl.dtype), _store(w2, wl.dtype)


def for_each_expert(wl: Workload, fn: Callable[[int, np.ndarray, np.ndarray], None],
                    threads: Optional[int] = None) -> None:
    """Generate every expert's weights in a thread pool and hand each to ``fn(e, w1, w2)``.

    ``fn`` is called from the pool threads; the caller makes it thread-safe.
    """
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=threads) as pool:
        futs = [pool.submit(lambda e=e: fn(e, *expert_weights(wl, e))) for e in range(wl.E)]
        for f in futs:
            f.result()


def stacked_weights(wl: Workload):
    """All experts stacked: w1 [E, w1_rows, d_model], w2 [E, d_model, d_ff] (host memory)."""
    dt = np.uint16 if wl.dtype == "bf16" else np.float32
    w1 = np.empty((wl.E, w1_rows(wl), wl.d_model), dt)
    w2 = np.empty((wl.E, wl.d_model, wl.d_ff), dt)

    def put(e, a, b):
        w1[e] = a
        w2[e] = b

    for_each_expert(wl, put)
    return w1, w2


def make_inputs(wl: Workload, with_weights: bool = True) -> dict:
    """Router-side inputs (and, optionally, all expert weights) of a workload."""
    kids = _children(wl)
    rx = np.random.Generator(np.random.PCG64(kids["x"]))
    x32 = _dyadic(rx, (wl.T, wl.d_model))
    out = {"x": _store(x32, wl.dtype), "w_r": None, "bias": None, "group_id": None}
    if wl.route == "topk":
        rw = np.random.Generator(np.random.PCG64(kids["w_r"]))
        if wl.w_r_dist == "dyadic":
            out["w_r"] = _dyadic(rw, (wl.E, wl.d_model))
        else:
            out["w_r"] = (rw.standard_normal((wl.E, wl.d_model)) / math.sqrt(wl.d_model)).astype(np.float32)
        if wl.zipf_s > 0:
            # log of Zipf(s) weights (e+1)^-s; the normaliser is a uniform shift and is omitted
            out["bias"] = (-wl.zipf_s * np.log(np.arange(1, wl.E + 1, dtype=np.float64))).astype(np.float32)
    else:
        rg = np.random.Generator(np.random.PCG64(kids["group_id"]))
        out["group_id"] = rg.integers(0, wl.n_groups, size=wl.T, dtype=np.int32)
    if with_weights:
        out["w1"], out["w2"] = stacked_weights(wl)
    return out
