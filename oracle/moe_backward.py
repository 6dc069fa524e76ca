"""CPU oracle for the backward pass of one MoE layer on one GPU's share of experts.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product
path never routes through it; it shares no code, tables or helpers with the
HIP library and imports nothing from it.

Sources (cited by page title and section):
  [HF]  Hugging Face Transformers docs, "Expert parallelism", "Token dispatch":
        every rank trains on its own share of the batch through the route /
        dispatch / local experts / combine path; an expert's weight gradient is
        the sum over all the batches whose pairs reached it, and an expert that
        received no tokens still takes part in that reduction (its zero-padding
        row adds nothing).
  [UL]  Ultralytics glossary, "Expert Parallelism", "How tokens move between
        GPUs": the forward this differentiates (route, dispatch, compute,
        combine weighted by the router scores).

What is computed: for the layer output y (no residual, as in the forward
oracle) and an upstream gradient dy = dLoss/dy, the gradients of the loss with
respect to x, the router weight and bias, and the three expert matrices, by the
chain rule through the forward definition

    y[t] = sum_{j kept local} w[t,j] * FFN_{e[t,j]}(x[t]),
    w[t,:] = softmax over the k chosen logits,  logits = x Wr^T + b,
    FFN_e(v) = (silu(v Wg_e^T) * (v Wu_e^T)) Wd_e^T.

Readings where the pages are silent (listed in the design notes):
  * which experts a token uses (top-k, selection bias, group limit, capacity
    drops) is a discrete choice and carries no gradient; the selection bias
    gets none.  The gradient reaches the router only through the softmax
    weights of the chosen slots, all k of them (a slot whose pair is not
    local or was dropped contributes no output, so its weight's gradient is
    0, but it still takes part in the softmax);
  * an expert with an empty segment gets an exactly zero weight gradient;
  * a token whose pairs were all dropped gets dx = 0 (its output was 0).

All arithmetic is float64.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from . import moe_oracle as fwd

__all__ = [
    "combine_backward",
    "softmax_over_k_backward",
    "expert_ffn_backward",
    "grouped_ffn_backward",
    "route_backward",
    "dispatch_backward",
    "layer_backward",
]


def combine_backward(dy: np.ndarray, y_sorted: np.ndarray, pair_row: np.ndarray, topk_w: np.ndarray) -> dict:
    """Backward of the combine step ([UL] step 4).

    y[t] = sum_j w[t,j] y_sorted[q(t,j)] over the slots with a kept local row q,
    so each such row receives dy_sorted[q] = w[t,j] dy[t] and the slot's weight
    receives d_topk_w[t,j] = <dy[t], y_sorted[q]>; slots without a row get 0.
    """
    T, k = topk_w.shape
    H = dy.shape[1]
    dy_sorted = np.zeros((y_sorted.shape[0], H))
    d_topk_w = np.zeros((T, k))
    for j in range(k):
        rows = pair_row[np.arange(T) * k + j]
        has = rows >= 0
        t = np.flatnonzero(has)
        q = rows[has]
        dy_sorted[q] = topk_w[t, j][:, None] * dy[t]
        d_topk_w[t, j] = np.einsum("th,th->t", dy[t], y_sorted[q])
    return {"dy_sorted": dy_sorted, "d_topk_w": d_topk_w}


def softmax_over_k_backward(topk_w: np.ndarray, d_topk_w: np.ndarray) -> np.ndarray:
    """Gradient with respect to the k chosen logits of w = softmax(chosen).

    dw_i/dl_j = w_i (delta_ij - w_j), hence dl_j = w_j (d_topk_w_j - sum_i w_i d_topk_w_i).
    """
    inner = (topk_w * d_topk_w).sum(axis=1, keepdims=True)
    return topk_w * (d_topk_w - inner)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def expert_ffn_backward(v: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, dout: np.ndarray) -> dict:
    """Backward of one SwiGLU expert on rows v [n,H] with output gradient dout [n,H].

    Forward: g = v Wg^T, u = v Wu^T, a = silu(g) = g s(g), h = a u, out = h Wd^T.
    Chain rule: dWd = dout^T h; dh = dout Wd; du = dh a; da = dh u;
    dg = da s(g) (1 + g (1 - s(g)))  (the derivative of g s(g));
    dWg = dg^T v; dWu = du^T v; dv = dg Wg + du Wu.
    Shapes follow nn.Linear storage: wg, wu [I,H]; wd [H,I].
    """
    g = v @ wg.T
    u = v @ wu.T
    s = _sigmoid(g)
    a = g * s
    h = a * u
    dh = dout @ wd
    du = dh * a
    dg = dh * u * s * (1.0 + g * (1.0 - s))
    return {"dv": dg @ wg + du @ wu, "dwg": dg.T @ v, "dwu": du.T @ v, "dwd": dout.T @ h,
            "g": g, "u": u, "h": h, "dg": dg, "du": du}


def grouped_ffn_backward(x_sorted: np.ndarray, offsets: np.ndarray, w_gate, w_up, w_down,
                         dy_sorted: np.ndarray) -> dict:
    """Backward of the local experts ([UL] step 3) over their segments.

    Expert i's weight gradients sum over its rows [offsets[i], offsets[i+1])
    ([HF] "Token dispatch": an expert's gradient is the sum over what reached
    it); an empty segment gives zeros.  Returns dx_sorted [P,H] and the stacked
    dw_gate, dw_up [L,I,H], dw_down [L,H,I].
    """
    L = len(offsets) - 1
    I, H = w_gate.shape[1], w_gate.shape[2]
    P = x_sorted.shape[0]
    dx_sorted = np.zeros((P, H))
    dwg = np.zeros((L, I, H))
    dwu = np.zeros((L, I, H))
    dwd = np.zeros((L, H, I))
    for i in range(L):
        a, b = int(offsets[i]), int(offsets[i + 1])
        if a == b:
            continue
        r = expert_ffn_backward(x_sorted[a:b], w_gate[i], w_up[i], w_down[i], dy_sorted[a:b])
        dx_sorted[a:b] = r["dv"]
        dwg[i], dwu[i], dwd[i] = r["dwg"], r["dwu"], r["dwd"]
    return {"dx_sorted": dx_sorted, "dw_gate": dwg, "dw_up": dwu, "dw_down": dwd}


def route_backward(x: np.ndarray, topk_ids: np.ndarray, dl: np.ndarray, num_experts: int) -> dict:
    """Router parameter gradients ([UL] step 1: logits = x Wr^T + b).

    The chosen slots' logit gradients dl [T,k] scatter into dlogits [T,E]
    (zero for experts a token did not choose); then dWr = dlogits^T x and
    db = sum over tokens of dlogits.
    """
    T, k = topk_ids.shape
    dlogits = np.zeros((T, num_experts))
    for j in range(k):
        dlogits[np.arange(T), topk_ids[:, j]] += dl[:, j]
    return {"dlogits": dlogits, "dw_router": dlogits.T @ x, "db_router": dlogits.sum(axis=0)}


def dispatch_backward(dx_sorted: np.ndarray, pair_row: np.ndarray, topk_ids: np.ndarray, dl: np.ndarray,
                      w_router: np.ndarray) -> np.ndarray:
    """Gradient with respect to the layer input x.

    The gather copied x[t] to every kept local row of its pairs, so those rows'
    gradients add back: sum_j dx_sorted[q(t,j)].  The router adds
    dlogits[t] Wr = sum_j dl[t,j] Wr[e[t,j]].
    """
    T, k = topk_ids.shape
    dx = np.zeros((T, dx_sorted.shape[1]))
    for j in range(k):
        rows = pair_row[np.arange(T) * k + j]
        has = rows >= 0
        dx[has] += dx_sorted[rows[has]]
    for j in range(k):
        dx += dl[:, j][:, None] * w_router[topk_ids[:, j]]
    return dx


def layer_backward(inp: dict, dy: np.ndarray, *, logits: Optional[np.ndarray] = None,
                   route_opts: Optional[dict] = None, fwd_out: Optional[dict] = None) -> dict:
    """The whole backward on one layer's inputs (the dict the input generator returns).

    dy: [T,H] upstream gradient of the layer output.  `logits` and
    `route_opts` are passed to the forward oracle (routing on given scores,
    bias-based balancing, group-limited routing); `fwd_out` reuses a forward
    already run with the same arguments.
    """
    s = inp["spec"]
    dt = s.dtype
    f = fwd_out if fwd_out is not None else fwd.layer_forward(inp, logits=logits, route_opts=route_opts)
    x = fwd.decode(inp["x"], dt)
    wr = fwd.decode(inp["w_router"], dt)
    dy = np.asarray(dy, dtype=np.float64)
    cb = combine_backward(dy, f["y_sorted"], f["pair_row"], f["topk_w"])
    dl = softmax_over_k_backward(f["topk_w"], cb["d_topk_w"])
    wg, wu, wd = fwd.expert_views(inp)
    fb = grouped_ffn_backward(f["x_sorted"], f["offsets"], wg, wu, wd, cb["dy_sorted"])
    if getattr(s, "weight_layout", "out_in") == "in_out":
        # the weight gradients take the layout of the weights
        for k in ("dw_gate", "dw_up", "dw_down"):
            fb[k] = np.ascontiguousarray(fb[k].transpose(0, 2, 1))
    rb = route_backward(x, f["topk_ids"], dl, s.E)
    dx = dispatch_backward(fb["dx_sorted"], f["pair_row"], f["topk_ids"], dl, wr)
    out = {"forward": f, "dy_sorted": cb["dy_sorted"], "d_topk_w": cb["d_topk_w"], "dl": dl, "dx": dx, **fb,
           "dw_router": rb["dw_router"], "dlogits": rb["dlogits"]}
    out["db_router"] = rb["db_router"] if inp.get("b_router") is not None else None
    return out
