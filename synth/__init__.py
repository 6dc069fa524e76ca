"""Seeded synthetic inputs for one MoE layer.

This module only draws random numbers and lays them out in memory.  It
holds none of the layer's arithmetic: both the CPU oracle and the HIP path
consume exactly the arrays it returns (bf16 values travel as identical
uint16 bit patterns), and neither side is imported here.

The workloads mirror the one concrete experiment on the pages (Ultralytics
glossary "Expert Parallelism", section "How tokens move between GPUs": unit
normal hidden states, a randomly initialised linear router, top-k over raw
router scores) at the shapes of five MoE layers:

  tiny_fp32         T=4096  H=512  I=256    E=8   k=2 all local, fp32, router bias
  mixtral_like      T=8192  H=4096 I=14336  E=8   k=2 all local, bf16
  gptoss_ep8_share  T=16384 H=2880 I=2880   E=128 k=4 experts 0-15 local, bf16
  decode_small      T=64    H=2048 I=768    E=128 k=8 all local, bf16
  skewed_capacity   T=32768 H=2048 I=1408   E=64  k=6 all local, bf16, Zipf-shaped
                    router bias, capacity factor 1.25

Draw recipe: numpy PCG64 streams spawned from SeedSequence(seed), one child
per array in this order (bf16 rounding and float32 scaling are per element,
so the values do not depend on how the work is split over threads):
  1. x        [T, H]  ~ N(0, 1)
  2. w_router [E, H]  ~ N(0, 1/H)               (nn.Linear layout: out x in)
  3. b_router [E]     fp32; tiny: U(-1/sqrt(H), 1/sqrt(H)) (nn.Linear's default
                      bias init); skewed: -s*ln(rank_e) with rank a random
                      permutation of 1..E and s = 1.2 (the log of a Zipf pmf);
                      otherwise none
  4. per local expert, ascending id:
       w_gate [I, H] ~ N(0, 1/H), w_up [I, H] ~ N(0, 1/H), w_down [H, I] ~ N(0, 1/I)
Large arrays are split into row chunks of at most 2^20 elements, chunk c
drawing from child c of its array's stream.  Normals are drawn as float32
(numpy's float32 ziggurat) and scaled in float32; bf16 layers round those float32 values to bf16 (nearest, ties to
even).  Every expert matrix is drawn as nn.Linear stores its weight,
[out_features, in_features] (the math form of the layer is x @ W.T); a spec
with weight_layout "in_out" then stores each expert matrix transposed
(w_gate, w_up [L, H, I], w_down [L, I, H]), the same values in the other
layout.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "LayerSpec",
    "WORKLOADS",
    "spec",
    "make_layer",
    "f32_to_bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    I: int                 # expert FFN width
    E: int                 # experts (global)
    k: int                 # experts per token
    local_begin: int       # local experts are [local_begin, local_begin + L)
    L: int                 # local expert count
    dtype: str             # "f32" or "bf16"
    bias: str = "none"     # "none" | "linear_default" | "zipf"
    zipf_s: float = 1.2
    capacity_factor: float = 0.0   # <= 0: no capacity limit
    seed: int = 0
    weight_layout: str = "out_in"  # "out_in": w_gate [L,I,H] ...; "in_out": w_gate [L,H,I] ...

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)

    @property
    def pairs(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny_fp32": LayerSpec("tiny_fp32", T=4096, H=512, I=256, E=8, k=2,
                           local_begin=0, L=8, dtype="f32", bias="linear_default"),
    "mixtral_like": LayerSpec("mixtral_like", T=8192, H=4096, I=14336, E=8, k=2,
                              local_begin=0, L=8, dtype="bf16"),
    "gptoss_ep8_share": LayerSpec("gptoss_ep8_share", T=16384, H=2880, I=2880, E=128,
                                  k=4, local_begin=0, L=16, dtype="bf16"),
    "decode_small": LayerSpec("decode_small", T=64, H=2048, I=768, E=128, k=8,
                              local_begin=0, L=128, dtype="bf16"),
    "skewed_capacity": LayerSpec("skewed_capacity", T=32768, H=2048, I=1408, E=64, k=6,
                                 local_begin=0, L=64, dtype="bf16", bias="zipf",
                                 capacity_factor=1.25),
}


def spec(name: str, **overrides) -> LayerSpec:
    return WORKLOADS[name].replace(**overrides)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    # NaN is not produced by the generator; the rounding below is for finite values.
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


_CHUNK = 1 << 20
_POOL = ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1))


def _normal_into(dst: np.ndarray, seq: np.random.SeedSequence, std: float, dtype: str) -> None:
    """Fill dst (2-D, rows x cols) with N(0, std^2) values stored as `dtype`."""
    rows, cols = dst.shape
    rows_per = max(1, _CHUNK // max(cols, 1))
    starts = list(range(0, rows, rows_per))
    kids = seq.spawn(len(starts))

    def one(c):
        r0 = starts[c]
        r1 = min(rows, r0 + rows_per)
        a = np.random.Generator(np.random.PCG64(kids[c])).standard_normal((r1 - r0, cols), dtype=np.float32)
        a *= np.float32(std)
        dst[r0:r1] = f32_to_bf16_bits(a) if dtype == "bf16" else a

    list(_POOL.map(one, range(len(starts))))


def _normal(seq, shape, std: float, dtype: str) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    _normal_into(out, seq, std, dtype)
    return out


def make_layer(s: LayerSpec, with_experts: bool = True) -> dict:
    """Draw one layer's inputs.

    Returns a dict with
      x [T,H], w_router [E,H], w_gate [L,I,H], w_up [L,I,H], w_down [L,H,I]
        (weight_layout "in_out": w_gate, w_up [L,H,I], w_down [L,I,H], the same values)
        -- float32 arrays for dtype "f32", uint16 bf16 bit patterns for "bf16";
      b_router [E] float32 or None; and "spec".
    """
    root = np.random.SeedSequence(s.seed)
    seq_x, seq_wr, seq_b, seq_exp = root.spawn(4)
    out = {"spec": s}
    out["x"] = _normal(seq_x, (s.T, s.H), 1.0, s.dtype)
    out["w_router"] = _normal(seq_wr, (s.E, s.H), 1.0 / math.sqrt(s.H), s.dtype)
    rng_b = np.random.Generator(np.random.PCG64(seq_b))
    if s.bias == "linear_default":
        bound = 1.0 / math.sqrt(s.H)
        out["b_router"] = rng_b.uniform(-bound, bound, s.E).astype(np.float32)
    elif s.bias == "zipf":
        rank = rng_b.permutation(s.E) + 1
        out["b_router"] = (-s.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    elif s.bias == "none":
        out["b_router"] = None
    else:
        raise ValueError(f"unknown bias kind {s.bias!r}")
    if with_experts:
        st = np.uint16 if s.dtype == "bf16" else np.float32
        wg = np.empty((s.L, s.I, s.H), dtype=st)
        wu = np.empty((s.L, s.I, s.H), dtype=st)
        wd = np.empty((s.L, s.H, s.I), dtype=st)
        kids = seq_exp.spawn(3 * s.L)
        for e in range(s.L):
            _normal_into(wg[e], kids[3 * e + 0], 1.0 / math.sqrt(s.H), s.dtype)
            _normal_into(wu[e], kids[3 * e + 1], 1.0 / math.sqrt(s.H), s.dtype)
            _normal_into(wd[e], kids[3 * e + 2], 1.0 / math.sqrt(s.I), s.dtype)
        if s.weight_layout == "in_out":
            wg, wu, wd = (np.ascontiguousarray(w.transpose(0, 2, 1)) for w in (wg, wu, wd))
        elif s.weight_layout != "out_in":
            raise ValueError(f"unknown weight layout {s.weight_layout!r}")
        out["w_gate"], out["w_up"], out["w_down"] = wg, wu, wd
    return out


def make_upstream_grad(s: LayerSpec) -> np.ndarray:
    """Seeded upstream gradient dy [T,H] of the layer output, N(0,1), in the layer's storage type.

    Drawn from its own child of the layer seed (spawn key 4), so the other
    draws of `make_layer` are unchanged.
    """
    seq = np.random.SeedSequence(s.seed, spawn_key=(4,))
    return _normal(seq, (s.T, s.H), 1.0, s.dtype)
