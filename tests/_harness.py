"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
on seeded inputs, and compare with the oracle by the agreed measures."""

from __future__ import annotations

import sys

import numpy as np

import oracle

# tolerances (see the design notes): float32 layers by the row's max norm,
# bf16 layers by the row's L2 norm; top-k flips only inside this logit gap
TOL_F32 = 1e-5
TOL_BF16 = 2e-2
FLIP_GAP = 1e-5


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def np_of(t) -> np.ndarray:
    """Device tensor -> float64/int numpy (bf16 widened exactly)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def desc_of(s):
    import expert_token_dispatch_amd as etd
    return etd.make_desc(s.T, s.H, s.I, s.E, s.k, s.local_begin, s.L, s.capacity_factor, s.dtype, s.weight_layout)


def layer_of(inp):
    from expert_token_dispatch_amd.layer import MoELayer, to_device
    s = inp["spec"]
    layer = MoELayer.from_host(desc_of(s), inp)
    x = to_device(inp["x"], s.dtype)
    return layer, x


def row_error(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """max over rows of max |got - ref| / norm(ref row); zero reference rows must match exactly."""
    d = np.abs(got - ref).max(axis=1)
    if dtype == "f32":
        n = np.abs(ref).max(axis=1)
    else:
        n = np.sqrt((ref * ref).sum(axis=1))
    zero = n == 0
    if np.any(d[zero] != 0):
        return float("inf")
    if np.all(zero):
        return 0.0
    return float((d[~zero] / n[~zero]).max())


def tol(dtype: str) -> float:
    return TOL_F32 if dtype == "f32" else TOL_BF16


def topk_gap(logits64: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit per token (inf if k == E)."""
    if k >= logits64.shape[1]:
        return np.full(logits64.shape[0], np.inf)
    srt = -np.sort(-logits64, axis=1)
    return srt[:, k - 1] - srt[:, k]


def flips(gpu_ids: np.ndarray, ref_ids: np.ndarray, logits64: np.ndarray, k: int):
    """Tokens whose chosen set differs; each must sit within FLIP_GAP of the boundary."""
    g = np.sort(gpu_ids, axis=1)
    r = np.sort(ref_ids, axis=1)
    bad = np.flatnonzero(np.any(g != r, axis=1))
    gap = topk_gap(logits64, k)
    return bad, gap[bad]
