"""CPU oracle for the forward pass of one MoE layer on one GPU's share of experts.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module.  The product
path never routes through it; it shares no code, tables or helpers with the
HIP library and imports nothing from it.

Sources (cited by page title and section):
  [HF]  Hugging Face Transformers docs, "Expert parallelism"
        - "Token dispatch": a rank routes its tokens, sends every (token,
          expert) pair to the expert's owner, runs its local experts on what it
          receives, and combines the returned results with the routing weights;
          the router must yield global expert ids.
        - "How the sizes combine": ep_size splits the expert list into ep_size
          contiguous blocks held by consecutive ranks.
  [UL]  Ultralytics glossary, "Expert Parallelism"
        - "How tokens move between GPUs": the four steps route (score every
          token against every expert, keep the k best), dispatch, compute,
          combine (results weighted by router scores and summed); the routing
          snippet (nn.Linear router, topk over raw scores, bincount loads,
          owner = expert // (E / num_gpus)).
        - "Load balancing and capacity": each expert takes at most a fixed
          number of tokens per batch (e.g. 1.25x the even share); overflow
          tokens skip that expert and pass through the residual unchanged.
          Bias-based balancing: a per-expert bias is added to the router
          scores for choosing experts only, and after every step it goes down
          for overloaded experts and up for idle ones.  The same section:
          each token's experts lie on at most a few of the nodes that hold
          them (node-limited routing).

Readings where the pages are silent (each is listed in the design notes):
  * top-k ties go to the lower expert id; slot j holds the j-th best score;
  * the routing weights are a softmax over the k chosen raw scores;
  * the expert FFN is SwiGLU without biases:
        FFN_e(v) = (silu(v Wg_e^T) * (v Wu_e^T)) Wd_e^T,  silu(z) = z / (1 + e^-z),
    with weights stored as nn.Linear stores them, [out_features, in_features];
  * capacity C = floor(cf * T * k / E) per local expert; an overflowing expert
    keeps its C pairs with the largest raw router score, ties to the lower
    token index; dropped pairs contribute nothing and the other weights are
    not renormalised;
  * within an expert's segment, pairs appear in ascending pair index
    p = t*k + j (a token picks an expert at most once, so this is ascending
    token order);
  * the layer output excludes the residual branch;
  * routing with a selection bias: experts are chosen by logit + bias, added
    in float32 (the precision the kernel decides in); the order, the weights
    (softmax over the k chosen) and the capacity ranking use the router
    logits without the bias;
  * the bias step: b_e -= gamma for experts with more than the mean load
    (c_e * E > sum c), b_e += gamma for those with less, unchanged at the
    mean; float32 state, one rounding per step;
  * group-limited routing: the E experts form G contiguous groups of E/G
    (the nodes); a group scores its best expert's selection score; each
    token keeps the M best groups (equal scores to the lower group) and
    takes its k experts from those groups only.

All floating-point work is float64 on the exact input values.  A top-k or
capacity decision made on given float32 logits compares those float32 values
(float64 holds them exactly), so it is the decision a float32 kernel makes.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "decode",
    "router_logits",
    "topk_select",
    "softmax_over_k",
    "expert_counts",
    "capacity_limit",
    "capacity_keep",
    "segment_offsets",
    "counting_sort",
    "gather_rows",
    "expert_ffn",
    "grouped_ffn",
    "combine",
    "route",
    "selection_scores",
    "group_allowed",
    "route_with_options",
    "selection_bias_update",
    "dispatch",
    "layer_forward",
    "ep_local_range",
]


# --------------------------------------------------------------------------- #
# value decoding
# --------------------------------------------------------------------------- #
def decode(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact float64 value of a stored array.

    dtype "bf16": `a` holds uint16 bfloat16 bit patterns (sign, 8-bit
    exponent, 7-bit mantissa: the top half of an IEEE float32).
    dtype "f32": `a` holds float32 values.
    dtype "f64": `a` holds float64 values, taken as they are (small exact
    layers for finite-difference checks of the backward).
    """
    if a is None:
        return None
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------- #
# step 1: routing  ([UL] "How tokens move between GPUs", step 1 and snippet)
# --------------------------------------------------------------------------- #
def router_logits(x: np.ndarray, w_router: np.ndarray, b_router: Optional[np.ndarray]) -> np.ndarray:
    """Score every token against every expert: logits = x Wr^T + b  ([T,E]).

    The router is a linear layer (nn.Linear(H, E) in the snippet), weight
    stored [E, H], bias optional.
    """
    logits = x @ w_router.T
    if b_router is not None:
        logits = logits + b_router[None, :]
    return logits


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """The k best experts per token, best first; equal scores go to the lower id.

    A stable ascending sort of the negated scores keeps equal scores in
    ascending expert order.  -0.0 and +0.0 compare equal (a tie).
    Returns int64 [T, k] global expert ids.
    """
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def softmax_over_k(chosen: np.ndarray) -> np.ndarray:
    """Routing weights: softmax over the k chosen raw scores of each token."""
    m = chosen.max(axis=1, keepdims=True)
    z = np.exp(chosen - m)
    return z / z.sum(axis=1, keepdims=True)


def route(x, w_router, b_router, k: int, logits: Optional[np.ndarray] = None) -> dict:
    """Step 1 end to end.  If `logits` is given, routing runs on it instead."""
    if logits is None:
        logits = router_logits(x, w_router, b_router)
    ids = topk_select(logits, k)
    chosen = np.take_along_axis(logits, ids, axis=1)
    return {"logits": logits, "topk_ids": ids, "topk_logit": chosen, "topk_w": softmax_over_k(chosen)}


# --------------------------------------------------------------------------- #
# step 1 variants  ([UL] "Load balancing and capacity": bias-based balancing,
#                   node-limited routing)
# --------------------------------------------------------------------------- #
def selection_scores(logits: np.ndarray, selection_bias: Optional[np.ndarray]) -> np.ndarray:
    """Scores the experts are chosen by: logit + per-expert bias, in float32.

    The bias only steers the choice.  The sum is formed in float32 because a
    float32 kernel takes the same integer decisions from the same sums; the
    float64 result holds those float32 values exactly.
    """
    if selection_bias is None:
        return logits
    s32 = logits.astype(np.float32) + selection_bias.astype(np.float32)[None, :]
    return s32.astype(np.float64)


def group_allowed(scores: np.ndarray, num_groups: int, max_groups: int) -> np.ndarray:
    """[T, E] bool: experts in the max_groups best of num_groups contiguous groups.

    A group's score is the largest score among its experts; groups are
    ranked by it, equal scores to the lower group index.
    """
    T, E = scores.shape
    if num_groups <= 1 or max_groups >= num_groups:
        return np.ones((T, E), dtype=bool)
    if E % num_groups != 0:
        raise ValueError("the experts must split evenly into the groups")
    gsize = E // num_groups
    gscore = scores.reshape(T, num_groups, gsize).max(axis=2)
    best = np.argsort(-gscore, axis=1, kind="stable")[:, :max_groups]
    keep = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(keep, best, True, axis=1)
    return np.repeat(keep, gsize, axis=1)


def route_with_options(logits: np.ndarray, k: int, selection_bias: Optional[np.ndarray] = None,
                       num_groups: int = 0, max_groups: int = 0) -> dict:
    """Top-k by the selection scores among the allowed experts; weights from the logits.

    Allowed experts come first; among them the larger selection score, then
    the lower expert id.  topk_logit and the softmax use the chosen experts'
    logits without the bias.
    """
    T, E = logits.shape
    scores = selection_scores(logits, selection_bias)
    allowed = group_allowed(scores, num_groups, max_groups)
    if np.any(allowed.sum(axis=1) < k):
        raise ValueError("fewer allowed experts than k")
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        # lexsort: last key first -> allowed before not, then higher score, then (stable) lower id
        order = np.lexsort((-scores[t], ~allowed[t]))
        ids[t] = order[:k]
    chosen = np.take_along_axis(logits, ids, axis=1)
    return {"logits": logits, "topk_ids": ids, "topk_logit": chosen, "topk_w": softmax_over_k(chosen)}


def selection_bias_update(bias: np.ndarray, counts: np.ndarray, gamma: float) -> np.ndarray:
    """One balancing step on the float32 bias from the expert loads of a batch.

    Overloaded experts (load above the mean, tested as c_e * E > sum c on
    integers) lose gamma, idle ones (below the mean) gain gamma, one float32
    rounding each.
    """
    c = np.asarray(counts, dtype=np.int64)
    E = c.shape[0]
    total = int(c.sum())
    b = np.asarray(bias, dtype=np.float32).copy()
    g = np.float32(gamma)
    over = c * E > total
    under = c * E < total
    b[over] = b[over] - g
    b[under] = b[under] + g
    return b


# --------------------------------------------------------------------------- #
# step 2: dispatch  ([HF] "Token dispatch"; [UL] snippet's bincount;
#                    [UL] "Load balancing and capacity")
# --------------------------------------------------------------------------- #
def expert_counts(topk_ids: np.ndarray, num_experts: int) -> np.ndarray:
    """Assignments received by each of the E experts (the snippet's bincount)."""
    return np.bincount(topk_ids.ravel(), minlength=num_experts).astype(np.int64)


def capacity_limit(capacity_factor: float, T: int, k: int, E: int) -> Optional[int]:
    """Per-expert limit: capacity_factor times the even share T*k/E, rounded down.

    None when capacity_factor <= 0 (no limit).  The product is formed in
    float64 as (cf * T * k) / E.
    """
    if capacity_factor <= 0:
        return None
    return int(math.floor(float(capacity_factor) * T * k / E))


def capacity_keep(topk_ids: np.ndarray, topk_logit: np.ndarray, local_begin: int, L: int,
                  C: Optional[int]) -> tuple[np.ndarray, int]:
    """Which local pairs survive the capacity limit.

    Returns (keep [T*k] bool, num_dropped).  keep is False for pairs whose
    expert is not local.  An expert with more than C pairs keeps the C with
    the largest router score, ties to the lower token index.
    """
    T, k = topk_ids.shape
    ids = topk_ids.ravel()
    score = topk_logit.ravel()
    local = (ids >= local_begin) & (ids < local_begin + L)
    keep = local.copy()
    dropped = 0
    if C is None:
        return keep, 0
    token = np.arange(T * k) // k
    for e in range(local_begin, local_begin + L):
        members = np.flatnonzero(ids == e)
        if members.size <= C:
            continue
        # primary key: score descending; secondary: token ascending
        order = np.lexsort((token[members], -score[members]))
        keep[members[order[C:]]] = False
        dropped += members.size - C
    return keep, dropped


def segment_offsets(kept_per_expert: np.ndarray) -> np.ndarray:
    """Exclusive prefix sum over local experts in id order: offsets [L+1]."""
    off = np.zeros(len(kept_per_expert) + 1, dtype=np.int64)
    off[1:] = np.cumsum(kept_per_expert)
    return off


def counting_sort(topk_ids: np.ndarray, keep: np.ndarray, local_begin: int, L: int,
                  offsets: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Place every kept local pair into its expert's segment, in pair order.

    Walks p = 0 .. T*k-1 once; pair p of expert e goes to
    offsets[e - begin] + (kept pairs of e already placed).
    Returns sorted_pairs [P] (pair ids) and pair_row [T*k] (position, -1 when
    the pair is not local or was dropped).
    """
    ids = topk_ids.ravel()
    n = ids.size
    fill = [0] * L
    sorted_pairs = np.full(int(offsets[-1]), -1, dtype=np.int64)
    pair_row = np.full(n, -1, dtype=np.int64)
    off = [int(v) for v in offsets]
    ids_l = ids.tolist()
    keep_l = keep.tolist()
    for p in range(n):
        if not keep_l[p]:
            continue
        e = ids_l[p] - local_begin
        pos = off[e] + fill[e]
        fill[e] += 1
        sorted_pairs[pos] = p
        pair_row[p] = pos
    return sorted_pairs, pair_row


def gather_rows(x: np.ndarray, sorted_pairs: np.ndarray, k: int) -> np.ndarray:
    """x_sorted[q] = x[token of pair sorted_pairs[q]]."""
    return x[sorted_pairs // k]


def dispatch(topk_ids, topk_logit, num_experts: int, local_begin: int, L: int,
             capacity_factor: float = 0.0, x: Optional[np.ndarray] = None) -> dict:
    """Step 2: counts, capacity, offsets, stable permutation (and gather if x)."""
    T, k = topk_ids.shape
    counts = expert_counts(topk_ids, num_experts)
    C = capacity_limit(capacity_factor, T, k, num_experts)
    keep, dropped = capacity_keep(topk_ids, topk_logit, local_begin, L, C)
    kept_ids = topk_ids.ravel()[keep]
    kept_per_expert = np.bincount(kept_ids - local_begin, minlength=L).astype(np.int64)
    offsets = segment_offsets(kept_per_expert)
    sorted_pairs, pair_row = counting_sort(topk_ids, keep, local_begin, L, offsets)
    out = {"counts": counts, "capacity": C, "keep": keep, "num_dropped": dropped,
           "offsets": offsets, "sorted_pairs": sorted_pairs, "pair_row": pair_row}
    if x is not None:
        out["x_sorted"] = gather_rows(x, sorted_pairs, k)
    return out


# --------------------------------------------------------------------------- #
# step 3: local experts  ([UL] "How tokens move between GPUs", step 3)
# --------------------------------------------------------------------------- #
def _silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(v: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert on rows v [n,H]: (silu(v Wg^T) * (v Wu^T)) Wd^T -> [n,H].

    wg, wu: [I, H]; wd: [H, I] (nn.Linear layout).
    """
    return (_silu(v @ wg.T) * (v @ wu.T)) @ wd.T


def grouped_ffn(x_sorted: np.ndarray, offsets: np.ndarray, w_gate, w_up, w_down,
                rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Run local expert i on its segment [offsets[i], offsets[i+1]).

    If `rows` (a boolean mask over sorted positions) is given, only those rows
    are computed; the others are left as NaN.
    """
    y = np.full((x_sorted.shape[0], w_down.shape[1]), np.nan)
    for i in range(len(offsets) - 1):
        a, b = int(offsets[i]), int(offsets[i + 1])
        if a == b:
            continue
        sel = np.arange(a, b)
        if rows is not None:
            sel = sel[rows[a:b]]
            if sel.size == 0:
                continue
        y[sel] = expert_ffn(x_sorted[sel], w_gate[i], w_up[i], w_down[i])
    return y


# --------------------------------------------------------------------------- #
# step 4: combine  ([UL] step 4; [HF] "Token dispatch")
# --------------------------------------------------------------------------- #
def combine(y_sorted: np.ndarray, pair_row: np.ndarray, topk_w: np.ndarray,
            tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """y[t] = sum over j = 0..k-1 with pair_row[t*k+j] >= 0 of w[t,j] * y_sorted[pair_row[t*k+j]].

    Summed in slot order.  A token with no kept local pair gets exactly 0.
    If `tokens` is given, only those rows are formed (returned in that order).
    """
    T, k = topk_w.shape
    if tokens is None:
        tokens = np.arange(T)
    H = y_sorted.shape[1]
    y = np.zeros((len(tokens), H))
    for j in range(k):
        rows = pair_row[tokens * k + j]
        has = rows >= 0
        y[has] += topk_w[tokens[has], j][:, None] * y_sorted[rows[has]]
    return y


# --------------------------------------------------------------------------- #
# the whole layer
# --------------------------------------------------------------------------- #
def layer_forward(inp: dict, *, logits: Optional[np.ndarray] = None,
                  tokens: Optional[np.ndarray] = None, route_opts: Optional[dict] = None) -> dict:
    """All four steps on one layer's inputs (the dict the input generator returns).

    logits: optional [T,E] float32/float64 scores to route on instead of
            computing them (used to compare decisions on identical scores).
    tokens: optional token subset; routing and dispatch cover every token, the
            expert FFN and combine only the pairs of these tokens.
    route_opts: optional {"selection_bias", "num_groups", "max_groups"} for
            route_with_options (bias-based balancing, group-limited routing).
    """
    s = inp["spec"]
    dt = s.dtype
    x = decode(inp["x"], dt)
    wr = decode(inp["w_router"], dt)
    br = inp.get("b_router")
    if br is not None:
        br = np.asarray(br, dtype=np.float64) if dt == "f64" else np.asarray(br, dtype=np.float32).astype(np.float64)
    r = route(x, wr, br, s.k, logits=None if logits is None else np.asarray(logits, dtype=np.float64))
    if route_opts is not None:
        r = route_with_options(r["logits"], s.k, route_opts.get("selection_bias"), route_opts.get("num_groups", 0),
                               route_opts.get("max_groups", 0))
    d = dispatch(r["topk_ids"], r["topk_logit"], s.E, s.local_begin, s.L, s.capacity_factor, x=x)
    out = {**r, **d}
    rows = None
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        want = np.zeros(s.T, dtype=bool)
        want[tokens] = True
        rows = want[d["sorted_pairs"] // s.k] if d["sorted_pairs"].size else np.zeros(0, dtype=bool)
    wg, wu, wd = expert_views(inp)
    y_sorted = grouped_ffn(d["x_sorted"], d["offsets"], wg, wu, wd, rows=rows)
    out["y_sorted"] = y_sorted
    out["y"] = combine(y_sorted, d["pair_row"], r["topk_w"], tokens=tokens)
    out["tokens"] = tokens
    return out


class _ExpertView:
    """Decodes one expert's matrix at a time, so float64 copies stay small.

    The matrix is returned as [out, in] (how expert_ffn takes it) whichever way it
    is stored: layout "in_out" stores each expert matrix transposed, [in, out].
    """

    def __init__(self, a: np.ndarray, dtype: str, layout: str = "out_in"):
        if layout not in ("out_in", "in_out"):
            raise ValueError(f"unknown weight layout {layout!r}")
        self.a, self.dtype, self.layout = a, dtype, layout

    def __getitem__(self, i: int) -> np.ndarray:
        m = decode(self.a[i], self.dtype)
        return m.T if self.layout == "in_out" else m

    @property
    def shape(self):
        L, r, c = self.a.shape
        return (L, c, r) if self.layout == "in_out" else (L, r, c)


def expert_views(inp: dict):
    """The gate, up and down weights of a layer's inputs as [out, in] views (any stored layout)."""
    lay = getattr(inp["spec"], "weight_layout", "out_in")
    dt = inp["spec"].dtype
    return tuple(_ExpertView(inp[k], dt, lay) for k in ("w_gate", "w_up", "w_down"))


# --------------------------------------------------------------------------- #
# expert ownership  ([HF] "How the sizes combine"; [UL] snippet's owner map)
# --------------------------------------------------------------------------- #
def ep_local_range(num_experts: int, ep_size: int, rank: int) -> tuple[int, int]:
    """Experts held by `rank`: block (rank mod ep_size) of ep_size equal blocks.

    ep_size consecutive ranks hold one full set, so the block index is the
    rank's position within its group.  ep_size must divide num_experts.
    """
    if ep_size <= 0 or num_experts <= 0 or rank < 0 or num_experts % ep_size != 0:
        raise ValueError("ep_size must be positive and divide num_experts; rank must be >= 0")
    per = num_experts // ep_size
    return (rank % ep_size) * per, per
