"""Pins of the backward oracle against mathematics it does not share code with.

* Central finite differences of the (separately pinned) forward oracle, on
  tiny float64 layers, for every entry of every gradient: the derivative is
  fixed by the forward alone, so a dropped term, a wrong sign, a wrong index
  or a transposed operand anywhere in the backward fails here.  Each check
  first asserts that the perturbations leave every routing, capacity and
  placement decision unchanged (the gradient of a piecewise-constant choice
  is taken with the choice held fixed).
* k = E = 1 reduces the layer to a dense SwiGLU MLP with weight 1: torch's
  autograd (an independent differentiation engine) on that MLP in float64.
* Invariants: softmax shift invariance (router gradients sum to zero over
  experts), homogeneity (y is linear in Wd and in Wu, so sum <W, dW> = <dy, y>),
  linearity in dy, fully dropped tokens get dx = 0, empty experts get 0.
* Planted mistakes in the oracle (on the CPU) must fail these pins.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.moe_backward as B
import synth


def tiny(T, H, I, E, k, lb, L, cf=0.0, seed=0, bias=True):
    """A float64 layer: inputs are taken exactly (storage type "f64")."""
    rng = np.random.default_rng(seed)
    s = synth.LayerSpec(name="tiny_f64", T=T, H=H, I=I, E=E, k=k, local_begin=lb, L=L, dtype="f64",
                        capacity_factor=cf, seed=seed)
    inp = {"spec": s,
           "x": rng.standard_normal((T, H)),
           "w_router": rng.standard_normal((E, H)),
           "b_router": rng.standard_normal(E) * 0.3 if bias else None,
           "w_gate": rng.standard_normal((L, I, H)) / np.sqrt(H),
           "w_up": rng.standard_normal((L, I, H)) / np.sqrt(H),
           "w_down": rng.standard_normal((L, H, I)) / np.sqrt(I)}
    dy = rng.standard_normal((T, H))
    return inp, dy


GRAD_OF = {"x": "dx", "w_router": "dw_router", "b_router": "db_router",
           "w_gate": "dw_gate", "w_up": "dw_up", "w_down": "dw_down"}


def decisions(f):
    return (f["topk_ids"].copy(), f["pair_row"].copy(), f["offsets"].copy())


def fd_check(inp, dy, route_opts=None, eps=1e-6, rtol=1e-7):
    """Every gradient entry against a central difference of <dy, y>."""
    g = B.layer_backward(inp, dy, route_opts=route_opts)
    base = decisions(g["forward"])
    for name, gname in GRAD_OF.items():
        if inp.get(name) is None:
            assert g.get(gname) is None
            continue
        a = inp[name]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            vals = []
            for sgn in (1.0, -1.0):
                old = a[idx]
                a[idx] = old + sgn * eps
                f = oracle.layer_forward(inp, route_opts=route_opts)
                a[idx] = old
                for u, v in zip(decisions(f), base):
                    assert np.array_equal(u, v), f"perturbing {name}{idx} changed a routing decision"
                vals.append(float((dy * f["y"]).sum()))
            fd[idx] = (vals[0] - vals[1]) / (2 * eps)
        got = g[gname]
        scale = max(np.abs(fd).max(), 1e-30)
        err = np.abs(got - fd).max() / scale
        assert err < rtol, f"{gname}: max error {err:.3e} relative to max |grad| {scale:.3e}"
    return g


# ---------------------------------------------------------------------------
# finite differences
# ---------------------------------------------------------------------------
def test_fd_plain_layer_with_nonlocal_experts():
    # experts 1..2 of 4 are local: some slots are not local, all take part in the softmax
    inp, dy = tiny(T=7, H=6, I=5, E=4, k=2, lb=1, L=2, seed=1)
    g = fd_check(inp, dy)
    assert np.any(g["forward"]["pair_row"] < 0)


def test_fd_all_experts_local_k_equals_e():
    inp, dy = tiny(T=5, H=4, I=3, E=3, k=3, lb=0, L=3, seed=2)
    fd_check(inp, dy)


def test_fd_with_capacity_drops():
    # C = floor(0.5 * 8 * 2 / 4) = 2 rows per expert: many pairs drop
    inp, dy = tiny(T=8, H=5, I=4, E=4, k=2, lb=0, L=4, cf=0.5, seed=3)
    g = fd_check(inp, dy)
    assert g["forward"]["num_dropped"] > 0


def test_fd_with_selection_bias_and_groups():
    inp, dy = tiny(T=6, H=5, I=3, E=4, k=2, lb=0, L=4, seed=4)
    opts = {"selection_bias": np.array([0.4, -0.2, 0.1, -0.3], dtype=np.float32), "num_groups": 2, "max_groups": 1}
    g = fd_check(inp, dy, route_opts=opts)
    # with one group of two experts allowed, a token's two experts share a group
    ids = g["forward"]["topk_ids"]
    assert np.all(ids[:, 0] // 2 == ids[:, 1] // 2)


def test_fd_without_router_bias():
    inp, dy = tiny(T=6, H=4, I=4, E=5, k=2, lb=2, L=3, seed=5, bias=False)
    fd_check(inp, dy)


# ---------------------------------------------------------------------------
# k = E = 1: a dense SwiGLU MLP, differentiated by torch's autograd
# ---------------------------------------------------------------------------
def test_single_expert_is_dense_mlp_autograd():
    torch = pytest.importorskip("torch")
    inp, dy = tiny(T=9, H=6, I=7, E=1, k=1, lb=0, L=1, seed=6)
    g = B.layer_backward(inp, dy)
    x = torch.tensor(inp["x"], requires_grad=True)
    wg = torch.tensor(inp["w_gate"][0], requires_grad=True)
    wu = torch.tensor(inp["w_up"][0], requires_grad=True)
    wd = torch.tensor(inp["w_down"][0], requires_grad=True)
    y = (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(g["dx"], x.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dw_gate"][0], wg.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dw_up"][0], wu.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(g["dw_down"][0], wd.grad.numpy(), rtol=1e-12, atol=1e-13)
    # one expert: its weight is exactly 1 and the router gets exactly nothing
    assert np.all(g["dl"] == 0) and np.all(g["dw_router"] == 0) and np.all(g["db_router"] == 0)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def mid():
    inp, dy = tiny(T=64, H=16, I=12, E=8, k=3, lb=0, L=8, seed=7)
    return inp, dy, B.layer_backward(inp, dy)


def test_router_gradients_sum_to_zero_over_experts(mid):
    # adding a constant to every logit of a token leaves its softmax unchanged
    _, _, g = mid
    assert np.abs(g["dl"].sum(axis=1)).max() < 1e-13
    assert abs(g["db_router"].sum()) < 1e-12
    assert np.abs(g["dw_router"].sum(axis=0)).max() < 1e-12


def test_homogeneity_in_down_and_up_weights(mid):
    inp, dy, g = mid
    ydy = float((dy * g["forward"]["y"]).sum())
    assert abs(float((inp["w_down"] * g["dw_down"]).sum()) - ydy) < 1e-10 * max(1.0, abs(ydy))
    assert abs(float((inp["w_up"] * g["dw_up"]).sum()) - ydy) < 1e-10 * max(1.0, abs(ydy))


def test_linear_in_upstream_gradient(mid):
    inp, dy, g = mid
    rng = np.random.default_rng(8)
    dy2 = rng.standard_normal(dy.shape)
    g2 = B.layer_backward(inp, dy2, fwd_out=g["forward"])
    g12 = B.layer_backward(inp, 2.0 * dy - dy2, fwd_out=g["forward"])
    for k in GRAD_OF.values():
        np.testing.assert_allclose(g12[k], 2.0 * g[k] - g2[k], rtol=1e-10, atol=1e-11)


def test_dropped_tokens_and_empty_experts_get_zero():
    # capacity 1 per expert, 6 tokens, all routed to 2 of 4 experts by the bias
    inp, dy = tiny(T=6, H=4, I=3, E=4, k=1, lb=0, L=4, cf=0.7, seed=9)
    inp["b_router"] = np.array([50.0, 40.0, -50.0, -50.0])
    g = B.layer_backward(inp, dy)
    f = g["forward"]
    kept = (f["pair_row"] >= 0).reshape(6, 1).any(axis=1)
    assert (~kept).sum() >= 3
    assert np.all(g["dx"][~kept] == 0)
    assert np.all(g["dw_gate"][2:] == 0) and np.all(g["dw_up"][2:] == 0) and np.all(g["dw_down"][2:] == 0)
    fd_check(inp, dy)


# ---------------------------------------------------------------------------
# planted mistakes must fail a pin
# ---------------------------------------------------------------------------
def _mutant_ffn_missing_dsilu_term(v, wg, wu, wd, dout):
    r = B.__dict__["_orig_expert_ffn_backward"](v, wg, wu, wd, dout)
    g, u = r["g"], r["u"]
    s = 1.0 / (1.0 + np.exp(-g))
    dg = (dout @ wd) * u * s  # drops the g (1 - s) term of d silu / dg
    r["dwg"] = dg.T @ v
    r["dv"] = dg @ wg + r["du"] @ wu
    return r


def _mutant_dispatch_no_router(dx_sorted, pair_row, topk_ids, dl, w_router):
    return B.__dict__["_orig_dispatch_backward"](dx_sorted, pair_row, topk_ids, dl * 0.0, w_router)


def _mutant_softmax_no_inner(topk_w, d_topk_w):
    return topk_w * d_topk_w


def _mutant_combine_no_weight(dy, y_sorted, pair_row, topk_w):
    return B.__dict__["_orig_combine_backward"](dy, y_sorted, pair_row, np.ones_like(topk_w))


def _mutant_route_wrong_slot(x, topk_ids, dl, num_experts):
    return B.__dict__["_orig_route_backward"](x, topk_ids[:, ::-1], dl, num_experts)


@pytest.mark.parametrize("fn,mutant", [
    ("expert_ffn_backward", _mutant_ffn_missing_dsilu_term),
    ("dispatch_backward", _mutant_dispatch_no_router),
    ("softmax_over_k_backward", _mutant_softmax_no_inner),
    ("combine_backward", _mutant_combine_no_weight),
    ("route_backward", _mutant_route_wrong_slot),
])
def test_planted_mistakes_fail_finite_differences(monkeypatch, fn, mutant):
    monkeypatch.setitem(B.__dict__, "_orig_" + fn, getattr(B, fn))
    monkeypatch.setattr(B, fn, mutant)
    inp, dy = tiny(T=6, H=4, I=3, E=4, k=2, lb=0, L=4, seed=10)
    with pytest.raises(AssertionError):
        fd_check(inp, dy)


def test_weight_gradients_take_the_weights_layout():
    # math-form weights (w_gate, w_up [L, H, I], w_down [L, I, H]): the same layer, so the
    # same gradients (up to the BLAS summation order of transposed operands), with each
    # expert's weight gradient stored transposed
    import oracle as fwd_oracle
    base = synth.spec("gptoss_ep8_share", T=200, H=40, I=24, E=16, k=4, L=8, local_begin=4)
    dy = fwd_oracle.decode(synth.make_upstream_grad(base), base.dtype)
    a = B.layer_backward(synth.make_layer(base), dy)
    b = B.layer_backward(synth.make_layer(base.replace(weight_layout="in_out")), dy)
    for k in ("dw_gate", "dw_up", "dw_down"):
        assert b[k].shape == a[k].transpose(0, 2, 1).shape
        np.testing.assert_allclose(b[k], a[k].transpose(0, 2, 1), rtol=1e-12, atol=1e-12)
    for k in ("dx", "dw_router", "dx_sorted"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-12, atol=1e-12)
