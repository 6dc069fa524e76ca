"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (moe_layer_forward, seed 0).

Routing and dispatch are checked on every token (ids, counts, offsets, drop
count and permutation bit for bit on identical logits; flips against the
oracle's own float64 logits only inside the allowed gap).  The layer output is
checked on every token against the oracle's whole layer, and every kept row of
the grouped FFN's output against the oracle's.
"""

import numpy as np
import pytest

import oracle
import synth
from tests._harness import FLIP_GAP, flips, layer_of, np_of, row_error, say, tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_size(name):
    s = synth.spec(name)
    say(f"[full] {name}: generating {s}")
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    say(f"[full] {name}: GPU forward")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    tw = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    cnt = torch.empty((s.E,), dtype=torch.int32, device="cuda")
    drop = torch.zeros((1,), dtype=torch.int64, device="cuda")
    y = layer.forward(x, topk_ids_out=ids, topk_w_out=tw, counts_out=cnt, num_dropped_out=drop)
    r = layer.route(x, want_logits=True, want_topk_logit=True)
    dd = layer.dispatch(x, r["topk_ids"], r["topk_logit"])
    torch.cuda.synchronize()
    y, ids, tw, cnt, drop = np_of(y), np_of(ids), np_of(tw), np_of(cnt), int(np_of(drop)[0])
    lg = np_of(r["logits"])
    np.testing.assert_array_equal(np_of(r["topk_ids"]), ids)

    say(f"[full] {name}: oracle routing and dispatch on the GPU's logits")
    ref = oracle.route(None, None, None, s.k, logits=lg.astype(np.float64))
    np.testing.assert_array_equal(ids, ref["topk_ids"])
    np.testing.assert_allclose(tw, ref["topk_w"], rtol=0, atol=2e-7)
    d = oracle.dispatch(ref["topk_ids"], ref["topk_logit"], s.E, s.local_begin, s.L, s.capacity_factor)
    np.testing.assert_array_equal(cnt, d["counts"])
    assert drop == d["num_dropped"]
    assert int(cnt.sum()) == s.T * s.k
    P = int(d["offsets"][-1])
    np.testing.assert_array_equal(np_of(dd["offsets"]), d["offsets"])
    np.testing.assert_array_equal(np_of(dd["sorted_pairs"])[:P], d["sorted_pairs"])
    np.testing.assert_array_equal(np_of(dd["pair_row"]), d["pair_row"])
    say(f"[full] {name}: counts {cnt.tolist() if s.E <= 16 else (cnt.min(), cnt.max())}, P={P}, dropped={drop}")

    say(f"[full] {name}: flips against float64 logits")
    xr = oracle.decode(inp["x"], s.dtype)
    wr = oracle.decode(inp["w_router"], s.dtype)
    br = None if inp["b_router"] is None else inp["b_router"].astype(np.float64)
    lg64 = oracle.router_logits(xr, wr, br)
    assert np.abs(lg - lg64).max() <= 1e-5 * max(1.0, np.abs(lg64).max())
    bad, gaps = flips(ids, oracle.topk_select(lg64, s.k), lg64, s.k)
    say(f"[full] {name}: {len(bad)} flips (gaps {gaps[:8]})")
    assert np.all(gaps < FLIP_GAP)
    del xr

    say(f"[full] {name}: oracle layer on every token")
    o = oracle.layer_forward(inp, logits=lg)
    err = row_error(y, o["y"], s.dtype)
    say(f"[full] {name}: row error over all {s.T} tokens {err:.3g}")
    assert err <= tol(s.dtype)
    if s.capacity_factor > 0:
        # tokens whose pairs were all cut get exactly zero (the row measure also demands it)
        all_cut = np.flatnonzero(np.all(d["pair_row"].reshape(s.T, s.k) < 0, axis=1))
        say(f"[full] {name}: {len(all_cut)} tokens with every pair cut")
        assert np.all(y[all_cut] == 0)
    # every kept row of the grouped FFN's output, on the dispatch's x_sorted (bit-equal to the oracle's)
    ys = np_of(layer.grouped_ffn(dd["x_sorted"], dd["offsets"]))[:P]
    np.testing.assert_array_equal(np_of(dd["x_sorted"])[:P], oracle.decode(inp["x"], s.dtype)[d["sorted_pairs"] // s.k])
    err_s = row_error(ys, o["y_sorted"][:P], s.dtype)
    say(f"[full] {name}: row error over all {P} rows of y_sorted {err_s:.3g}")
    assert err_s <= tol(s.dtype)
