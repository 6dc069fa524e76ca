"""GPU parity for the routing options of the Ultralytics glossary "Expert
Parallelism", section "Load balancing and capacity": a selection-only
per-expert bias (bias-based balancing), group-limited top-k (node-limited
routing) and the balancing step on the bias.  Decisions are compared bit for
bit with the oracle on the logits the GPU computed; weights within 2e-7.
"""

import numpy as np
import pytest

import oracle
import synth
from tests._harness import layer_of, np_of, row_error, say, tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import expert_token_dispatch_amd as etd  # noqa: E402


def _opts(E, bias_scale, G, M, seed):
    rng = np.random.default_rng(seed)
    bias = None
    if bias_scale:
        bias = (np.round(rng.standard_normal(E) * bias_scale * 4) / 4).astype(np.float32)
    return bias, G, M


CASES = [
    # E, k, G, M, bias scale, tied logits
    (8, 2, 0, 0, 1.0, False),
    (16, 2, 4, 1, 0.5, True),
    (64, 6, 8, 3, 0.0, False),
    (128, 4, 8, 4, 0.5, False),
    (128, 32, 8, 2, 0.5, True),
    (200, 5, 10, 2, 1.0, True),
    (256, 8, 16, 2, 0.25, False),
]


@pytest.mark.parametrize("E,k,G,M,bs,tied", CASES, ids=lambda v: str(v))
def test_route_with_options_bit_exact(E, k, G, M, bs, tied):
    s = synth.spec("mixtral_like", T=300, H=128, I=64, E=E, k=k, L=E)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    bias, G, M = _opts(E, bs, G, M, E + k)
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    o = etd.make_route_opts(bt, G, M)
    if tied:
        rng = np.random.default_rng(E)
        lg = (np.round(rng.standard_normal((s.T, E)) * 2) / 2).astype(np.float32)
        r = layer.route(x, logits_in=torch.from_numpy(lg).cuda(), want_topk_logit=True, opts=o)
    else:
        r = layer.route(x, want_logits=True, want_topk_logit=True, opts=o)
        lg = np_of(r["logits"])
    say(f"[options] E={E} k={k} groups {G}/{M} bias {bs} tied {tied}")
    ref = oracle.route_with_options(lg.astype(np.float64), k, bias, G, M)
    np.testing.assert_array_equal(np_of(r["topk_ids"]), ref["topk_ids"])
    np.testing.assert_array_equal(np_of(r["topk_logit"]), ref["topk_logit"].astype(np.float32))
    np.testing.assert_allclose(np_of(r["topk_w"]), ref["topk_w"], rtol=0, atol=2e-7)


def test_route_options_random_draws():
    # seeded random draws: E up to 256, k, a group count dividing E (up to 16), the most
    # groups a token may use (enough to hold k), a selection bias of random scale (or none),
    # and logits from the router or rounded so that many tie
    rng = np.random.default_rng(31337)
    for it in range(120):
        E = int(rng.choice([2, 4, 6, 8, 12, 16, 32, 48, 64, 96, 128, 160, 192, 256]))
        divs = [g for g in range(2, 17) if E % g == 0]
        G = int(rng.choice(divs)) if divs and rng.random() < 0.7 else 0
        k = int(rng.integers(1, min(E, 32) + 1))
        M = 0
        if G:
            M = int(rng.integers(1, G + 1))
            while M * (E // G) < k:
                M += 1
        bs = float(rng.choice([0.0, 0.25, 1.0, 4.0]))
        tied = bool(rng.random() < 0.4)
        T = int(rng.choice([1, 5, 64, 65, 257]))
        s = synth.spec("mixtral_like", T=T, H=64, I=64, E=E, k=k, L=E, seed=70000 + it)
        inp = synth.make_layer(s)
        layer, x = layer_of(inp)
        bias = (np.round(rng.standard_normal(E) * bs * 4) / 4).astype(np.float32) if bs else None
        bt = None if bias is None else torch.from_numpy(bias).cuda()
        o = etd.make_route_opts(bt, G, M)
        if tied:
            lg = (np.round(rng.standard_normal((T, E)) * 2) / 2).astype(np.float32)
            r = layer.route(x, logits_in=torch.from_numpy(lg).cuda(), want_topk_logit=True, opts=o)
        else:
            r = layer.route(x, want_logits=True, want_topk_logit=True, opts=o)
            lg = np_of(r["logits"])
        say(f"[options] draw {it}: T={T} E={E} k={k} groups {G}/{M} bias {bs} tied {tied}")
        ref = oracle.route_with_options(lg.astype(np.float64), k, bias, G, M)
        np.testing.assert_array_equal(np_of(r["topk_ids"]), ref["topk_ids"], err_msg=f"draw {it}")
        np.testing.assert_array_equal(np_of(r["topk_logit"]), ref["topk_logit"].astype(np.float32))
        np.testing.assert_allclose(np_of(r["topk_w"]), ref["topk_w"], rtol=0, atol=2e-7)


def test_layer_forward_with_options():
    s = synth.spec("gptoss_ep8_share", T=700, H=128, I=160, E=32, k=4, L=16, local_begin=8)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    bias = (np.random.default_rng(4).standard_normal(32) * 0.5).astype(np.float32)
    o = etd.make_route_opts(torch.from_numpy(bias).cuda(), 8, 2)
    lg = np_of(layer.route(x, want_logits=True).get("logits"))
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    counts = torch.empty((s.E,), dtype=torch.int32, device="cuda")
    y = np_of(layer.forward(x, topk_ids_out=ids, counts_out=counts, opts=o))
    ref = oracle.layer_forward(inp, logits=lg, route_opts={"selection_bias": bias, "num_groups": 8, "max_groups": 2})
    say(f"[options] layer with bias and 2 of 8 groups: {s}")
    np.testing.assert_array_equal(np_of(ids), ref["topk_ids"])
    np.testing.assert_array_equal(np_of(counts), ref["counts"])
    assert row_error(y, ref["y"], s.dtype) <= tol(s.dtype)


def test_selection_bias_update_bit_exact():
    rng = np.random.default_rng(9)
    for E in (1, 7, 128, 256):
        s = synth.spec("mixtral_like", T=64, H=64, I=64, E=E, k=1, L=E)
        layer, _ = layer_of(synth.make_layer(s))
        counts = rng.integers(0, 50, E).astype(np.int32)
        counts[: E // 3] = int(round(counts.mean()))       # some at (or near) the mean
        bias = rng.standard_normal(E).astype(np.float32)
        b = torch.from_numpy(bias.copy()).cuda()
        c = torch.from_numpy(counts).cuda()
        for g in (1e-3, 0.37):
            layer.update_selection_bias(c, b, g)
            bias = oracle.selection_bias_update(bias, counts, g)
        np.testing.assert_array_equal(np_of(b), bias)


def test_balancing_loop_matches_oracle():
    # choose (with the bias) - count - adjust, 40 steps on fixed logits that favour two
    # experts; the float32 bias after every step equals the oracle's bit for bit
    s = synth.spec("gptoss_ep8_share", T=512, H=64, I=64, E=16, k=2, L=16, local_begin=0)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((s.T, s.E)).astype(np.float32)
    lg[:, :2] += 1.0
    lgt = torch.from_numpy(lg).cuda()
    b = torch.zeros(s.E, dtype=torch.float32, device="cuda")
    bias = np.zeros(s.E, np.float32)
    o = etd.make_route_opts(b, 4, 2)
    first = None
    for step in range(40):
        r = layer.route(x, logits_in=lgt, opts=o)
        d = layer.dispatch(x, r["topk_ids"])
        layer.update_selection_bias(d["counts"], b, 0.02)
        ref = oracle.route_with_options(lg.astype(np.float64), s.k, bias, 4, 2)
        cnt = oracle.expert_counts(ref["topk_ids"], s.E)
        first = cnt if first is None else first
        bias = oracle.selection_bias_update(bias, cnt, 0.02)
        np.testing.assert_array_equal(np_of(r["topk_ids"]), ref["topk_ids"])
        np.testing.assert_array_equal(np_of(d["counts"]), cnt)
        np.testing.assert_array_equal(np_of(b), bias)
    say(f"[options] balancing loop: max load {first.max()} -> {cnt.max()} (even share {s.T * s.k // s.E})")
    assert cnt.max() < first.max()
