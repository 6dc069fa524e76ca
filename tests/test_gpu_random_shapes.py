"""Seeded random layer shapes through the whole path, against the oracles.

Each case draws a dtype, E (1..256), k, a local expert range, T, H and I (multiples
of 64, which the large-tile kernel takes, or any multiple of 8), an optional
capacity factor, the weight layout and the router bias, then checks what the fixed
cases check: routing, counts, offsets and the permutation bit for bit against the
oracle (which routes on the GPU's own float32 logits), the fused forward equal to
the staged one, the output rows within the forward's tolerance; for the training
step, the stage gradients and weight gradients within the backward's measures.

The router's weight gradient sums the chosen slots' logit gradients, each a
difference of dot products scaled through the softmax: its error is bounded by the
terms, not by the result (one token gives a rank-one matrix whose norm can cancel).
It is checked against the logit-gradient rounding bound (the one the combine
backward test uses) carried through dWr = sum over tokens of dlogits x, plus the
output rounding.
"""

import numpy as np
import pytest

import oracle
import oracle.moe_backward as B
import synth
from tests._harness import layer_of, np_of, row_error, say, tol
from tests.test_gpu_backward import mat_ok, rows_ok, run_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _draw(rng, pairs_max, seed):
    dtype = str(rng.choice(["bf16", "f32"]))
    E = int(rng.choice([1, 2, 3, 5, 8, 16, 32, 64, 100, 128, 200, 256]))
    k = int(min(E, rng.choice([1, 2, 3, 4, 6, 8, 16, 32])))
    L = int(rng.integers(1, E + 1))
    begin = int(rng.integers(0, E - L + 1))
    T = int(rng.choice([1, 7, 64, 65, 300, 1000, 2500]))
    while T * k > pairs_max and T > 1:
        T //= 2
    grid = rng.random() < 0.5
    H = int(64 * rng.integers(1, 9)) if grid else int(8 * rng.integers(1, 65))
    I = int(64 * rng.integers(1, 9)) if grid else int(8 * rng.integers(1, 65))
    cf = float(rng.uniform(0.3, 2.0)) if rng.random() < 0.3 else 0.0
    return synth.spec("gptoss_ep8_share", T=T, H=H, I=I, E=E, k=k, local_begin=begin, L=L, dtype=dtype,
                      capacity_factor=cf, weight_layout=str(rng.choice(["out_in", "in_out"])),
                      bias=str(rng.choice(["none", "linear_default", "zipf"])), seed=seed)


def test_random_shapes_forward():
    rng = np.random.default_rng(20261)
    for it in range(200):
        s = _draw(rng, 8000, 50000 + it)
        say(f"[random] forward {it}: {s}")
        inp = synth.make_layer(s)
        layer, x = layer_of(inp)
        g = layer.staged(x)
        y = layer.forward(x)
        torch.cuda.synchronize()
        gpu = {kk: (np_of(v) if isinstance(v, torch.Tensor) else v) for kk, v in g.items()}
        ref = oracle.layer_forward(inp, logits=gpu["logits"])
        np.testing.assert_array_equal(gpu["topk_ids"], ref["topk_ids"])
        np.testing.assert_array_equal(gpu["counts"], ref["counts"])
        np.testing.assert_array_equal(gpu["offsets"], ref["offsets"])
        P = int(ref["offsets"][-1])
        np.testing.assert_array_equal(gpu["sorted_pairs"][:P], ref["sorted_pairs"])
        np.testing.assert_array_equal(gpu["pair_row"], ref["pair_row"])
        assert int(gpu["num_dropped"][0]) == ref["num_dropped"]
        np.testing.assert_array_equal(np_of(y), gpu["y"])
        err = row_error(gpu["y"], ref["y"], s.dtype)
        assert err <= tol(s.dtype), f"case {it}: row error {err:.3g}"


def test_random_shapes_training_step():
    rng = np.random.default_rng(20262)
    for it in range(100):
        s = _draw(rng, 8000, 60000 + it)
        if s.bias == "zipf":
            s = s.replace(bias="linear_default")
        say(f"[random] training step {it}: {s}")
        inp = synth.make_layer(s)
        layer, x, dy_h, gpu, fused = run_gpu(s, inp)
        dy = oracle.decode(dy_h, s.dtype)
        ref = B.layer_backward(inp, dy, logits=gpu["logits"].astype(np.float64))
        f = ref["forward"]
        P = int(f["offsets"][-1])
        np.testing.assert_array_equal(gpu["y"], gpu["y_inference"])
        rows_ok("y", gpu["y"], f["y"], s.dtype)
        rows_ok("dy_sorted", gpu["dy_sorted"][:P], ref["dy_sorted"][:P], s.dtype)
        rows_ok("dx_sorted", gpu["dx_sorted"][:P], ref["dx_sorted"][:P], s.dtype)
        mat_ok("dw_gate", gpu["dw_gate"], ref["dw_gate"], s.dtype)
        mat_ok("dw_up", gpu["dw_up"], ref["dw_up"], s.dtype)
        mat_ok("dw_down", gpu["dw_down"], ref["dw_down"], s.dtype)
        rows_ok("dx", gpu["dx"], ref["dx"], s.dtype)
        # router weight gradient against the propagated logit-gradient bound
        T, k = f["topk_w"].shape
        pr = f["pair_row"].reshape(T, k)
        has = pr >= 0
        ynorm = np.zeros((T, k))
        ynorm[has] = np.linalg.norm(f["y_sorted"][pr[has]], axis=1)
        scale = np.linalg.norm(dy, axis=1) * ynorm.max(axis=1)
        b = 2 * tol(s.dtype) * f["topk_w"] * scale[:, None]
        xd = oracle.decode(inp["x"], s.dtype)
        bound = tol(s.dtype) * np.abs(ref["dw_router"])
        for j in range(k):
            np.add.at(bound, f["topk_ids"][:, j], b[:, j:j + 1] * np.abs(xd))
        err = np.abs(gpu["dw_router"] - ref["dw_router"])
        assert np.all(err <= bound), f"case {it}: router weight gradient above its bound"
        for kk, v in fused.items():
            if v is not None:
                np.testing.assert_array_equal(v, gpu[kk], err_msg=f"case {it}: {kk}")
