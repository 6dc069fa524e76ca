"""Pins for the CPU oracle: what the pages print, closed forms, invariants,
library special cases and brute force on tiny inputs.  CPU only.

Nothing here calls the HIP library.  Each pin is written independently of
the oracle's code (pure-Python loops, library routines, hand-derived values)
so that a plausible mistake in the oracle fails at least one of them; the
mutation tests at the end plant such mistakes and check that they are caught.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- #
# brute-force helpers: plain Python loops over scalars
# --------------------------------------------------------------------------- #
def bf_topk(logits_row, k):
    # full sort of (score descending, id ascending)
    pairs = sorted(range(len(logits_row)), key=lambda e: (-float(logits_row[e]), e))
    return pairs[:k]


def bf_silu(z):
    return z / (1.0 + math.exp(-z)) if z > -700 else 0.0 * z


def bf_expert(v, wg, wu, wd):
    I, H = wg.shape
    h = []
    for i in range(I):
        g = sum(v[c] * wg[i, c] for c in range(H))
        u = sum(v[c] * wu[i, c] for c in range(H))
        h.append(bf_silu(g) * u)
    return [sum(h[i] * wd[o, i] for i in range(I)) for o in range(H)]


def bf_layer(x, wr, br, wg, wu, wd, k, begin, L, cf, logits=None):
    """Whole layer by its definition, token by token (no permutation at all)."""
    T, H = x.shape
    E = wr.shape[0]
    if logits is None:
        logits = [[sum(x[t, c] * wr[e, c] for c in range(H)) + (br[e] if br is not None else 0.0)
                   for e in range(E)] for t in range(T)]
    ids = [bf_topk(logits[t], k) for t in range(T)]
    w = []
    for t in range(T):
        ls = [logits[t][e] for e in ids[t]]
        m = max(ls)
        z = [math.exp(v - m) for v in ls]
        s = sum(z)
        w.append([v / s for v in z])
    # capacity by brute force: for each expert list its pairs with keys
    keep = {}
    C = None if cf <= 0 else int(math.floor(cf * T * k / E))
    dropped = 0
    for e in range(begin, begin + L):
        members = [(t, j) for t in range(T) for j in range(k) if ids[t][j] == e]
        if C is not None and len(members) > C:
            ranked = sorted(members, key=lambda tj: (-logits[tj[0]][e], tj[0]))
            kept = set(ranked[:C])
            dropped += len(members) - C
        else:
            kept = set(members)
        for tj in members:
            keep[tj] = tj in kept
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = ids[t][j]
            if begin <= e < begin + L and keep[(t, j)]:
                y[t] += w[t][j] * np.array(bf_expert(x[t], wg[e - begin], wu[e - begin], wd[e - begin]))
    return {"ids": ids, "w": w, "y": y, "dropped": dropped, "logits": logits}


def tiny_inputs(seed, T=6, H=4, I=3, E=4, k=2, begin=0, L=None, bias=True):
    rng = np.random.default_rng(1000 + seed)
    L = E if L is None else L
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) / math.sqrt(H)
    br = rng.uniform(-0.5, 0.5, E) if bias else None
    wg = rng.standard_normal((L, I, H)) / math.sqrt(H)
    wu = rng.standard_normal((L, I, H)) / math.sqrt(H)
    wd = rng.standard_normal((L, H, I)) / math.sqrt(I)
    return x, wr, br, wg, wu, wd


def oracle_layer(x, wr, br, wg, wu, wd, k, begin, L, cf=0.0, logits=None):
    T, H = x.shape
    E = wr.shape[0]
    s = synth.LayerSpec("t", T=T, H=H, I=wg.shape[1], E=E, k=k, local_begin=begin, L=L,
                        dtype="f32", capacity_factor=cf)
    # float64 inputs go straight in: decode("f32") would round them, so pass a
    # float64-preserving dict through the staged functions directly.
    r = oracle.route(x, wr, br, k, logits=logits)
    d = oracle.dispatch(r["topk_ids"], r["topk_logit"], E, begin, L, cf, x=x)
    ys = oracle.grouped_ffn(d["x_sorted"], d["offsets"], wg, wu, wd)
    y = oracle.combine(ys, d["pair_row"], r["topk_w"])
    return {**r, **d, "y_sorted": ys, "y": y, "spec": s}


# --------------------------------------------------------------------------- #
# 1. the pages' routing simulation
# --------------------------------------------------------------------------- #
def _page_simulation_inputs():
    torch = pytest.importorskip("torch")
    g = _golden("routing_simulation_loads.json")
    torch.manual_seed(0)
    tokens = torch.randn(g["num_tokens"], g["hidden"])
    router = torch.nn.Linear(g["hidden"], g["num_experts"])
    return g, tokens, router


def test_page_routing_simulation_loads():
    """Per-expert and per-GPU loads of the glossary's snippet (printed extremes)."""
    g, tokens, router = _page_simulation_inputs()
    x = tokens.numpy().astype(np.float64)
    wr = router.weight.detach().numpy().astype(np.float64)
    br = router.bias.detach().numpy().astype(np.float64)
    r = oracle.route(x, wr, br, g["top_k"])
    counts = oracle.expert_counts(r["topk_ids"], g["num_experts"])
    assert counts.sum() == g["assignments"]
    assert counts.min() == g["per_expert_min"] and counts.max() == g["per_expert_max"]
    assert g["num_tokens"] * g["top_k"] // g["num_experts"] == g["even_share"]
    per_gpu = []
    for rank in range(g["num_gpus"]):
        b, n = oracle.ep_local_range(g["num_experts"], g["num_gpus"], rank)
        per_gpu.append(int(counts[b:b + n].sum()))
    assert min(per_gpu) == g["per_gpu_min"] and max(per_gpu) == g["per_gpu_max"]
    assert sum(per_gpu) == g["assignments"]


def test_page_routing_simulation_matches_library_topk():
    """The same snippet run through torch's own topk/bincount gives the oracle's loads."""
    import torch
    g, tokens, router = _page_simulation_inputs()
    with torch.no_grad():
        _, experts = router(tokens).topk(g["top_k"], dim=-1)
    lib = torch.bincount(experts.flatten(), minlength=g["num_experts"]).numpy()
    lib_gpu = torch.bincount((experts // (g["num_experts"] // g["num_gpus"])).flatten(),
                             minlength=g["num_gpus"]).numpy()
    x = tokens.numpy().astype(np.float64)
    r = oracle.route(x, router.weight.detach().numpy().astype(np.float64),
                     router.bias.detach().numpy().astype(np.float64), g["top_k"])
    counts = oracle.expert_counts(r["topk_ids"], g["num_experts"])
    np.testing.assert_array_equal(counts, lib)
    # torch orders the k results by score too: identical ids slot by slot
    np.testing.assert_array_equal(r["topk_ids"], experts.numpy())
    per_gpu = [counts[2 * i:2 * i + 2].sum() for i in range(4)]
    np.testing.assert_array_equal(per_gpu, lib_gpu)


# --------------------------------------------------------------------------- #
# 2. expert ownership: the eight-rank layout figure
# --------------------------------------------------------------------------- #
def test_rank_layout_figure():
    g = _golden("rank_layout_8ranks.json")
    for ep, table in g["experts_by_rank"].items():
        ep = int(ep)
        for rank, experts in enumerate(table):
            b, n = oracle.ep_local_range(g["num_experts"], ep, rank)
            assert list(range(b, b + n)) == experts
        assert g["fsdp_size"] * g["tp_size"] // ep == g["efsdp_size"][str(ep)]


def test_rank_layout_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.ep_local_range(8, 3, 0)
    with pytest.raises(ValueError):
        oracle.ep_local_range(8, 0, 0)


# --------------------------------------------------------------------------- #
# 3. brute force on tiny inputs
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("k,begin,L,cf", [(1, 0, 4, 0.0), (2, 0, 4, 0.0), (2, 1, 2, 0.0),
                                          (3, 0, 4, 0.0), (4, 0, 4, 0.0), (2, 0, 4, 1.0),
                                          (2, 1, 3, 0.75), (1, 0, 4, 0.5)])
def test_bruteforce_tiny(seed, k, begin, L, cf):
    x, wr, br, wg, wu, wd = tiny_inputs(seed, T=7, L=L)
    ref = bf_layer(x, wr, br, wg, wu, wd, k, begin, L, cf)
    got = oracle_layer(x, wr, br, wg, wu, wd, k, begin, L, cf)
    assert [list(r) for r in got["topk_ids"]] == ref["ids"]
    np.testing.assert_allclose(got["topk_w"], np.array(ref["w"]), rtol=0, atol=1e-14)
    assert got["num_dropped"] == ref["dropped"]
    np.testing.assert_allclose(got["y"], ref["y"], rtol=1e-12, atol=1e-13)


def test_bruteforce_ties_and_signed_zero():
    # equal scores: lower id first; -0.0 and +0.0 tie
    logits = np.array([[0.5, 0.5, 0.1, 0.5],
                       [-0.0, 0.0, -1.0, 0.0],
                       [1.0, 2.0, 2.0, -3.0]])
    for k in range(1, 5):
        ids = oracle.topk_select(logits, k)
        for t in range(3):
            assert list(ids[t]) == bf_topk(logits[t], k)
    assert list(oracle.topk_select(logits, 3)[0]) == [0, 1, 3]
    assert list(oracle.topk_select(logits, 3)[1]) == [0, 1, 3]


def test_topk_matches_lexsort():
    rng = np.random.default_rng(7)
    # quantised scores force many ties
    logits = np.round(rng.standard_normal((300, 16)) * 2) / 2
    for k in (1, 3, 8, 16):
        ids = oracle.topk_select(logits, k)
        for t in range(logits.shape[0]):
            ref = np.lexsort((np.arange(16), -logits[t]))[:k]
            np.testing.assert_array_equal(ids[t], ref)


# --------------------------------------------------------------------------- #
# 4. closed forms and special cases
# --------------------------------------------------------------------------- #
def test_decode_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = oracle.decode(bits, "bf16")
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    np.testing.assert_array_equal(vals, want)
    assert math.copysign(1.0, vals[4]) == -1.0


def test_generator_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], dtype=np.float32)
    got = oracle.decode(synth.f32_to_bf16_bits(f), "bf16")
    np.testing.assert_array_equal(got, [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5])


def test_swiglu_single_unit_closed_form():
    # H = I = 1: FFN(v) = silu(v*g) * (v*u) * d
    v, g, u, d = 1.5, 0.8, -2.0, 0.25
    y = oracle.expert_ffn(np.array([[v]]), np.array([[g]]), np.array([[u]]), np.array([[d]]))
    z = v * g
    assert y[0, 0] == pytest.approx(z * (1 / (1 + math.exp(-z))) * (v * u) * d, rel=1e-15)
    from scipy.special import expit
    zs = np.linspace(-30, 30, 61)
    s = oracle.expert_ffn(zs[:, None], np.ones((1, 1)), np.ones((1, 1)), np.ones((1, 1)))[:, 0]
    np.testing.assert_allclose(s, zs * expit(zs) * zs, rtol=1e-13, atol=1e-300)


def test_single_expert_is_dense_swiglu_mlp():
    # E = 1, k = 1: softmax over one score is 1, the layer is the plain MLP
    x, wr, br, wg, wu, wd = tiny_inputs(3, T=9, H=5, I=7, E=1)
    got = oracle_layer(x, wr, br, wg, wu, wd, 1, 0, 1)["y"]
    g = x @ wg[0].T
    want = (g / (1 + np.exp(-g)) * (x @ wu[0].T)) @ wd[0].T
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_k_equals_e_is_dense_soft_moe():
    # every expert chosen: y = sum_e softmax(logits)_e FFN_e(x), with scipy's softmax
    from scipy.special import softmax
    x, wr, br, wg, wu, wd = tiny_inputs(4, T=10, H=6, I=5, E=5)
    got = oracle_layer(x, wr, br, wg, wu, wd, 5, 0, 5)["y"]
    p = softmax(x @ wr.T + br, axis=1)
    want = np.zeros_like(x)
    for e in range(5):
        g = x @ wg[e].T
        want += p[:, e:e + 1] * ((g / (1 + np.exp(-g)) * (x @ wu[e].T)) @ wd[e].T)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_capacity_value():
    assert oracle.capacity_limit(1.25, 32768, 6, 64) == 3840
    assert oracle.capacity_limit(1.25, 4096, 2, 8) == 1280
    assert oracle.capacity_limit(0.0, 100, 2, 8) is None
    assert oracle.capacity_limit(-1.0, 100, 2, 8) is None
    assert oracle.capacity_limit(1.0, 7, 2, 4) == 3   # floor(3.5)


# --------------------------------------------------------------------------- #
# 5. invariants on a realistic-shape routing
# --------------------------------------------------------------------------- #
def _check_dispatch_invariants(r, d, T, k, E, begin, L, C):
    ids = r["topk_ids"]
    counts = d["counts"]
    assert counts.sum() == T * k
    np.testing.assert_array_equal(counts, [int((ids == e).sum()) for e in range(E)])
    local = (ids.ravel() >= begin) & (ids.ravel() < begin + L)
    kept = d["keep"]
    assert not np.any(kept & ~local)
    n_kept = int(kept.sum())
    assert d["offsets"][0] == 0 and d["offsets"][-1] == n_kept
    sp, pr = d["sorted_pairs"], d["pair_row"]
    # bijection onto the kept local pairs, and inverse of each other
    assert sorted(sp.tolist()) == np.flatnonzero(kept).tolist()
    np.testing.assert_array_equal(pr[sp], np.arange(n_kept))
    assert np.all(pr[~kept] == -1)
    # segment i holds expert begin+i's pairs in ascending pair order
    for i in range(L):
        seg = sp[d["offsets"][i]:d["offsets"][i + 1]]
        assert np.all(ids.ravel()[seg] == begin + i)
        assert np.all(np.diff(seg) > 0)
        n_e = counts[begin + i]
        assert len(seg) == (n_e if C is None else min(n_e, C))
    # closed form of the drop count
    want_drop = 0 if C is None else sum(max(0, int(counts[begin + i]) - C) for i in range(L))
    assert d["num_dropped"] == want_drop
    # the stable permutation is numpy's stable argsort of the expert id
    if C is None:
        kp = np.flatnonzero(kept)
        ref = kp[np.argsort(ids.ravel()[kp], kind="stable")]
        np.testing.assert_array_equal(sp, ref)


@pytest.mark.parametrize("name,over", [
    ("tiny_fp32", {}),
    ("gptoss_ep8_share", {"T": 2048, "H": 64}),
    ("decode_small", {}),
    ("skewed_capacity", {"T": 4096, "H": 64}),
    ("skewed_capacity", {"T": 4096, "H": 64, "local_begin": 16, "L": 32}),
])
def test_dispatch_invariants(name, over):
    s = synth.spec(name, **over)
    inp = synth.make_layer(s, with_experts=False)
    x = oracle.decode(inp["x"], s.dtype)
    wr = oracle.decode(inp["w_router"], s.dtype)
    br = None if inp["b_router"] is None else inp["b_router"].astype(np.float64)
    r = oracle.route(x, wr, br, s.k)
    np.testing.assert_allclose(r["topk_w"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(r["topk_logit"], axis=1) <= 0)
    d = oracle.dispatch(r["topk_ids"], r["topk_logit"], s.E, s.local_begin, s.L, s.capacity_factor, x=x)
    C = oracle.capacity_limit(s.capacity_factor, s.T, s.k, s.E)
    _check_dispatch_invariants(r, d, s.T, s.k, s.E, s.local_begin, s.L, C)
    # gathered rows are the tokens' rows
    np.testing.assert_array_equal(d["x_sorted"], x[d["sorted_pairs"] // s.k])


def test_capacity_kept_set_is_bruteforce_top_c():
    rng = np.random.default_rng(11)
    T, k, E = 200, 3, 6
    logits = np.round(rng.standard_normal((T, E)) * 4) / 4 + np.array([2.0, 1, 0, 0, 0, 0])
    r = oracle.route(None, None, None, k, logits=logits)
    d = oracle.dispatch(r["topk_ids"], r["topk_logit"], E, 0, E, capacity_factor=1.0)
    C = int(math.floor(1.0 * T * k / E))
    for e in range(E):
        members = [(t, j) for t in range(T) for j in range(k) if r["topk_ids"][t, j] == e]
        ranked = sorted(members, key=lambda tj: (-logits[tj[0], e], tj[0]))
        want = {t * k + j for (t, j) in ranked[:C]}
        got = {p for p in np.flatnonzero(d["keep"]) if r["topk_ids"].ravel()[p] == e}
        assert got == want


# --------------------------------------------------------------------------- #
# 6. combine with identity experts, decomposition over ranks and row slices
# --------------------------------------------------------------------------- #
def test_identity_experts_return_input():
    x, wr, br, *_ = tiny_inputs(5, T=50, H=8, E=6)
    r = oracle.route(x, wr, br, 3)
    d = oracle.dispatch(r["topk_ids"], r["topk_logit"], 6, 0, 6, x=x)
    y = oracle.combine(d["x_sorted"], d["pair_row"], r["topk_w"])
    np.testing.assert_allclose(y, x, rtol=1e-14, atol=1e-15)


def test_dropped_everywhere_gives_zero_rows():
    x, wr, br, wg, wu, wd = tiny_inputs(6, T=12, E=4)
    got = oracle_layer(x, wr, br, wg, wu, wd, 2, 0, 4, cf=0.25)   # C = floor(1.5) = 1
    kept_tok = set((np.flatnonzero(got["keep"]) // 2).tolist())
    for t in range(12):
        if t not in kept_tok:
            assert np.all(got["y"][t] == 0.0)
    assert got["num_dropped"] == 24 - int(got["keep"].sum())


def test_ep_ranges_sum_to_all_local():
    # no rank computes experts for tokens it does not own, and together they cover all
    x, wr, br, wg, wu, wd = tiny_inputs(8, T=40, H=6, I=5, E=8)
    full = oracle_layer(x, wr, br, wg, wu, wd, 2, 0, 8)["y"]
    for ep in (2, 4, 8):
        acc = np.zeros_like(full)
        for rank in range(ep):
            b, n = oracle.ep_local_range(8, ep, rank)
            acc += oracle_layer(x, wr, br, wg[b:b + n], wu[b:b + n], wd[b:b + n], 2, b, n)["y"]
        np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-13)


def test_row_slices_concatenate():
    # each tensor-parallel rank dispatches a disjoint slice of rows; slices may be uneven or empty
    x, wr, br, wg, wu, wd = tiny_inputs(9, T=23, H=6, I=5, E=4)
    full = oracle_layer(x, wr, br, wg, wu, wd, 2, 0, 4)["y"]
    parts = []
    for a, b in [(0, 0), (0, 10), (10, 11), (11, 23)]:
        if a == b:
            continue
        parts.append(oracle_layer(x[a:b], wr, br, wg, wu, wd, 2, 0, 4)["y"])
    np.testing.assert_allclose(np.concatenate(parts), full, rtol=1e-13, atol=1e-14)


def test_layer_forward_token_subset_matches_full():
    s = synth.spec("gptoss_ep8_share", T=256, H=64, I=32)
    inp = synth.make_layer(s)
    full = oracle.layer_forward(inp)
    sub = np.array([0, 5, 17, 255, 100])
    part = oracle.layer_forward(inp, tokens=sub)
    # BLAS may block a smaller product differently: equal up to rounding
    np.testing.assert_allclose(part["y"], full["y"][sub], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- #
# 6b. routing variants (Ultralytics glossary "Expert Parallelism", section "Load
#     balancing and capacity": bias-based balancing, node-limited routing)
# --------------------------------------------------------------------------- #
def test_variants_reduce_to_plain_routing():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((64, 16)).astype(np.float32).astype(np.float64)
    plain = oracle.route(None, None, None, 4, logits=lg)
    for kw in (dict(), dict(selection_bias=np.zeros(16, np.float32)), dict(num_groups=4, max_groups=4),
               dict(num_groups=1, max_groups=1)):
        r = oracle.route_with_options(lg, 4, **kw)
        np.testing.assert_array_equal(r["topk_ids"], plain["topk_ids"])
        np.testing.assert_array_equal(r["topk_w"], plain["topk_w"])


def test_selection_bias_worked_example():
    # logits 1.0 0.9 0.5 0.1, bias +0.6 on expert 2: choice by 1.0 0.9 1.1 0.1 -> experts 2, 0;
    # the weights are a softmax over their unbiased logits 0.5 and 1.0
    r = oracle.route_with_options(np.array([[1.0, 0.9, 0.5, 0.1]]), 2, np.array([0, 0, 0.6, 0], np.float32))
    assert r["topk_ids"].tolist() == [[2, 0]]
    assert r["topk_logit"].tolist() == [[0.5, 1.0]]
    w2 = 1.0 / (1.0 + math.exp(0.5))
    assert abs(r["topk_w"][0, 0] - w2) < 1e-15 and abs(r["topk_w"][0, 1] - (1.0 - w2)) < 1e-15


def test_group_limit_worked_example():
    # four groups of two: maxima 0.2 0.9 0.8 0.4.  One group: group 1 only, so 0.9 then
    # 0.0 although 0.8 and 0.7 score higher elsewhere; two groups: groups 1 and 2.
    lg = np.array([[0.1, 0.2, 0.9, 0.0, 0.8, 0.7, 0.3, 0.4]])
    assert oracle.route_with_options(lg, 2, None, 4, 1)["topk_ids"].tolist() == [[2, 3]]
    assert oracle.route_with_options(lg, 2, None, 4, 2)["topk_ids"].tolist() == [[2, 4]]
    # equal group maxima: the lower group wins
    lg = np.array([[0.5, 0.0, 0.0, 0.5, 0.1, 0.2]])
    assert oracle.route_with_options(lg, 2, None, 3, 1)["topk_ids"].tolist() == [[0, 1]]


@pytest.mark.parametrize("G,M", [(4, 1), (4, 2), (8, 3)])
def test_group_limit_invariants(G, M):
    rng = np.random.default_rng(G * 10 + M)
    T, E, k = 200, 32, 4
    lg = rng.standard_normal((T, E))
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    r = oracle.route_with_options(lg, k, bias, G, M)
    sc = lg.astype(np.float32) + bias
    for t in range(T):
        ids = [int(e) for e in r["topk_ids"][t]]
        assert len(set(ids)) == k
        # the best expert overall is always taken first (its group has the best score)
        assert ids[0] == bf_topk(sc[t].astype(np.float64), 1)[0]
        assert len({e // (E // G) for e in ids}) <= M
        # chosen scores never increase
        assert all(sc[t][ids[j]] >= sc[t][ids[j + 1]] for j in range(k - 1))
        # weights: a softmax over the chosen unbiased logits
        ex = [math.exp(lg[t, e] - max(lg[t, i] for i in ids)) for e in ids]
        assert np.allclose(r["topk_w"][t], [v / sum(ex) for v in ex], rtol=0, atol=1e-14)


def test_bias_step_closed_forms():
    # mean load 3.25: expert 3 is over, the others under; equal loads leave the bias alone
    g = 2.0 ** -10
    b = oracle.selection_bias_update(np.zeros(4, np.float32), np.array([3, 3, 3, 4]), g)
    assert b.dtype == np.float32 and b.tolist() == [g, g, g, -g]
    b0 = np.array([0.25, -1.5, 3.0], np.float32)
    assert oracle.selection_bias_update(b0, np.array([7, 7, 7]), g).tolist() == b0.tolist()
    # n steps at constant loads from zero: exactly -n*gamma*sign (multiples of 2^-10 are exact)
    c = np.array([10, 0, 5, 5, 20])
    b = np.zeros(5, np.float32)
    for _ in range(37):
        b = oracle.selection_bias_update(b, c, g)
    assert b.tolist() == [-37 * g, 37 * g, 37 * g, 37 * g, -37 * g]


def test_bias_steps_even_out_a_skewed_load():
    # the section's claim: the bias balances the load.  A router that favours expert 0
    # by one unit, 400 steps of choose-count-adjust; the largest load falls toward T*k/E.
    rng = np.random.default_rng(3)
    T, E, k = 256, 8, 2
    lg = rng.standard_normal((T, E))
    lg[:, 0] += 1.0
    b = np.zeros(E, np.float32)
    first = None
    for _ in range(400):
        ids = oracle.route_with_options(lg, k, b)["topk_ids"]
        c = np.bincount(ids.ravel(), minlength=E)
        first = c if first is None else first
        b = oracle.selection_bias_update(b, c, 0.01)
    assert first.max() > 1.8 * T * k / E
    assert c.max() < 1.25 * T * k / E
    assert b[0] < 0


# 7. planted mistakes must be caught by the pins above
# --------------------------------------------------------------------------- #
def _pins_pass():
    checks = [
        test_page_routing_simulation_loads,
        lambda: test_bruteforce_tiny(0, 2, 0, 4, 0.0),
        lambda: test_bruteforce_tiny(1, 2, 1, 3, 0.75),
        test_bruteforce_ties_and_signed_zero,
        test_identity_experts_return_input,
        test_capacity_kept_set_is_bruteforce_top_c,
        lambda: test_dispatch_invariants("skewed_capacity", {"T": 1024, "H": 64}),
        test_single_expert_is_dense_swiglu_mlp,
        test_k_equals_e_is_dense_soft_moe,
        test_selection_bias_worked_example,
        test_group_limit_worked_example,
        lambda: test_group_limit_invariants(4, 2),
        test_bias_step_closed_forms,
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def _mut_drop_bias(x, wr, br):
    return x @ wr.T


def _mut_ties_high(logits, k):
    order = np.argsort(-logits[:, ::-1], axis=1, kind="stable")
    return (logits.shape[1] - 1 - order[:, :k]).astype(np.int64)


def _mut_softmax_all(chosen):
    return np.exp(chosen) / np.exp(chosen).sum(axis=1, keepdims=True) * 0 + 1.0 / chosen.shape[1]


def _mut_silu_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _mut_ffn_swap(v, wg, wu, wd):
    return ((v @ wu.T) / (1 + np.exp(-(v @ wu.T))) * (v @ wg.T)) @ wd.T


def _mut_unstable_sort(topk_ids, keep, begin, L, offsets):
    sp, pr = _ORIG["counting_sort"](topk_ids, keep, begin, L, offsets)
    for i in range(L):
        a, b = int(offsets[i]), int(offsets[i + 1])
        sp[a:b] = sp[a:b][::-1].copy()
    pr[sp] = np.arange(len(sp))
    return sp, pr


def _mut_capacity_highest(topk_ids, topk_logit, begin, L, C):
    return _ORIG["capacity_keep"](topk_ids, -topk_logit, begin, L, C)


def _mut_weights_from_biased(logits, k, selection_bias=None, num_groups=0, max_groups=0):
    r = _ORIG["route_with_options"](logits, k, selection_bias, num_groups, max_groups)
    sc = oracle.selection_scores(logits, selection_bias)
    r["topk_w"] = oracle.softmax_over_k(np.take_along_axis(sc, r["topk_ids"], axis=1))
    return r


def _mut_bias_sign(bias, counts, gamma):
    return _ORIG["selection_bias_update"](bias, counts, -gamma)


def _mut_group_sum(scores, num_groups, max_groups):
    T, E = scores.shape
    if num_groups <= 1 or max_groups >= num_groups:
        return np.ones((T, E), dtype=bool)
    gs = E // num_groups
    best = np.argsort(-scores.reshape(T, num_groups, gs).sum(axis=2), axis=1, kind="stable")[:, :max_groups]
    keep = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(keep, best, True, axis=1)
    return np.repeat(keep, gs, axis=1)


def _mut_group_ties_high(scores, num_groups, max_groups):
    return _ORIG["group_allowed"](scores[:, ::-1], num_groups, max_groups)[:, ::-1]


_ORIG = {n: getattr(oracle.moe_oracle, n) for n in ("counting_sort", "capacity_keep", "route_with_options",
                                                     "selection_bias_update", "group_allowed")}


@pytest.mark.parametrize("target,mutant", [
    ("router_logits", _mut_drop_bias),
    ("topk_select", _mut_ties_high),
    ("softmax_over_k", _mut_softmax_all),
    ("_silu", _mut_silu_sigmoid),
    ("expert_ffn", _mut_ffn_swap),
    ("counting_sort", _mut_unstable_sort),
    ("capacity_keep", _mut_capacity_highest),
    ("route_with_options", _mut_weights_from_biased),
    ("selection_bias_update", _mut_bias_sign),
    ("group_allowed", _mut_group_sum),
    ("group_allowed", _mut_group_ties_high),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(oracle.moe_oracle, target, mutant)
    monkeypatch.setattr(oracle, target, mutant, raising=False)
    assert not _pins_pass(), f"a planted mistake in {target} went unnoticed"


def test_math_form_weight_layout():
    # the stacked layout of the workloads' math form (w_gate, w_up [L, H, I], w_down [L, I, H]):
    # with one expert and k = 1 the layer is (silu(x Wg) * (x Wu)) Wd written directly on
    # the stored arrays, and any layer equals the linear-layout layer on the same draws
    s1 = synth.spec("tiny_fp32", T=40, H=24, I=16, E=1, k=1, L=1, weight_layout="in_out")
    inp = synth.make_layer(s1)
    assert inp["w_gate"].shape == (1, 24, 16) and inp["w_down"].shape == (1, 16, 24)
    x = inp["x"].astype(np.float64)
    g = x @ inp["w_gate"][0].astype(np.float64)
    want = (g / (1 + np.exp(-g)) * (x @ inp["w_up"][0].astype(np.float64))) @ inp["w_down"][0].astype(np.float64)
    np.testing.assert_allclose(oracle.layer_forward(inp)["y"], want, rtol=1e-13, atol=1e-14)
    for name in ("skewed_capacity", "gptoss_ep8_share"):
        base = synth.spec(name, T=300, H=64, I=48)
        a = oracle.layer_forward(synth.make_layer(base))
        b = oracle.layer_forward(synth.make_layer(base.replace(weight_layout="in_out")))
        np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-13)
