"""GPU parity of the per-token row kernels (combine, combine backward, dispatch
backward) on rows whose 16-byte slices do not fill the wave's last pass.

These kernels give each token one wave: lane j holds slot j's sorted row and
weight, every lane takes 16-byte slices of the row, and the slots are
broadcast across the wave.  Rows of H elements are vec = H * dtype / 16
slices; when vec leaves a remainder of 1..k-1 slices in the last pass (or is
itself below k), lanes past the remainder still hold slots, so every lane
must run every pass.  The shapes below put that remainder in every position
the kernels' pass widths allow: bf16 H = 64 with k = 16 (8 slices), bf16
H = 8 with k = 2 (one slice), bf16 H = 2056 with k = 4 (257 slices), f32
H = 1032 with k = 4 (258 slices).  Forward and backward against the float64
oracles (Ultralytics glossary "Expert Parallelism", "How tokens move between
GPUs", step 4; Transformers "Expert parallelism", "Token dispatch").
"""

import numpy as np
import pytest

import oracle
import oracle.moe_backward as B
import synth
from tests._harness import layer_of, np_of, row_error, say, tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SHAPES = {
    "bf16-H64-k16": synth.spec("mixtral_like", T=200, H=64, I=64, E=64, k=16, L=64),
    "bf16-H8-k2": synth.spec("mixtral_like", T=150, H=8, I=16, E=8, k=2, L=8),
    "bf16-H2056-k4": synth.spec("gptoss_ep8_share", T=160, H=2056, I=96, E=16, k=4, L=16),
    "f32-H1032-k4": synth.spec("tiny_fp32", T=160, H=1032, I=64, E=8, k=4, L=8),
    "bf16-H2056-k3-local-range": synth.spec("gptoss_ep8_share", T=130, H=2056, I=64, E=16, k=3,
                                            local_begin=4, L=8),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_forward_row_tails(name):
    s = SHAPES[name]
    say(f"[tails] forward {name}: {s}")
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    g = layer.staged(x)
    y_fused = layer.forward(x)
    torch.cuda.synchronize()
    gpu = {k: (np_of(v) if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    ref = oracle.layer_forward(inp, logits=gpu["logits"])
    np.testing.assert_array_equal(gpu["topk_ids"], ref["topk_ids"])
    np.testing.assert_array_equal(gpu["pair_row"], ref["pair_row"])
    P = int(ref["offsets"][-1])
    # combine on the GPU's own y_sorted, in float64: the combine alone within its rounding
    own = oracle.combine(gpu["y_sorted"][:P].astype(np.float64), gpu["pair_row"], gpu["topk_w"].astype(np.float64))
    e_comb = row_error(gpu["y"], own, s.dtype)
    e_layer = row_error(gpu["y"], ref["y"], s.dtype)
    say(f"[tails]   combine on own rows {e_comb:.2e}, layer {e_layer:.2e}")
    assert e_comb <= tol(s.dtype) and e_layer <= tol(s.dtype)
    np.testing.assert_array_equal(np_of(y_fused), gpu["y"])


@pytest.mark.parametrize("name", list(SHAPES))
def test_backward_row_tails(name):
    s = SHAPES[name]
    say(f"[tails] backward {name}: {s}")
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    from expert_token_dispatch_amd.layer import to_device
    dy_h = synth.make_upstream_grad(s)
    dy = to_device(dy_h, s.dtype)
    logits = layer.route(x, want_logits=True)["logits"]
    y, saved = layer.forward_train(x)
    st = layer.staged_backward(x, saved, dy)
    torch.cuda.synchronize()
    gpu = {k: np_of(v) for k, v in saved._tensors.items()}
    gpu.update({k: (None if v is None else np_of(v)) for k, v in st.items()})
    lg = np_of(logits).astype(np.float64)
    ref = B.layer_backward(inp, oracle.decode(dy_h, s.dtype), logits=lg)
    P = int(ref["forward"]["offsets"][-1])
    e = row_error(gpu["dy_sorted"][:P], ref["dy_sorted"][:P], s.dtype)
    say(f"[tails]   dy_sorted {e:.2e}")
    assert e <= tol(s.dtype)
    # rows >= P of dy_sorted are never written by the combine backward; row 0 belongs to a pair
    # (with P > 0) and must hold that pair's gradient, not another slot's
    f = ref["forward"]
    dyd = oracle.decode(dy_h, s.dtype)
    T, k = f["topk_w"].shape
    pr = f["pair_row"].reshape(T, k)
    ynorm = np.zeros((T, k))
    has = pr >= 0
    ynorm[has] = np.linalg.norm(f["y_sorted"][pr[has]], axis=1)
    bound = 2 * tol(s.dtype) * f["topk_w"] * (np.linalg.norm(dyd, axis=1) * ynorm.max(axis=1))[:, None]
    err = np.abs(gpu["dl"] - ref["dl"])
    say(f"[tails]   dl: max error / bound {float((err / np.maximum(bound, 1e-300)).max()):.2e}")
    assert np.all(err <= bound)
    e = row_error(gpu["dx"], ref["dx"], s.dtype)
    say(f"[tails]   dx {e:.2e}")
    assert e <= tol(s.dtype)
