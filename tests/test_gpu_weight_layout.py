"""GPU parity with the expert weights in the math-form layout (w_gate, w_up
[L, H, I], w_down [L, I, H]: the stacked [in, out] matrices of the workloads'
"W_gate H x I"; Transformers "Expert parallelism": grouped_gemm experts stacked
along the expert dimension) against the float64 oracle, on every kernel path:
the large-tile kernel (four and eight waves, K cut into pieces, wide tail
tiles), the skinny decode kernel, and the general kernel (float32 and shapes
off the large tile's grid).

The kernels read those k-major weights with transposing LDS reads (or, in the
general kernel, transpose (k, k+1) pairs on the way into LDS), which hands the
matrix cores the very operands the linear layout gives, in the same order: so
the forward must equal the linear-layout forward on the same values bit for
bit, as well as the oracle within tolerance.  The backward reads each weight
in place in either layout and writes the weight gradients in the weights'
layout; it is checked against the backward oracle.
"""

import numpy as np
import pytest

import oracle
import oracle.moe_backward as B
import synth
from tests._harness import layer_of, np_of, row_error, say, tol
from tests.test_gpu_backward import SMALL, mat_ok, rows_ok, run_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = dict(SMALL)
CASES.update({
    "off-grid-bf16": synth.spec("gptoss_ep8_share", T=257, H=136, I=200, E=16, k=3, L=16),
    "large-eight-waves-cut": synth.spec("gptoss_ep8_share", T=300, H=2880, I=2880, E=4, k=2, L=4),
    "large-four-waves-cut": synth.spec("mixtral_like", T=400, H=4096, I=4608, E=4, k=2, L=4),
    "large-I320": synth.spec("gptoss_ep8_share", T=2048, H=320, I=320),
    "decode-I288": synth.spec("decode_small", T=16, H=512, I=288, E=32, k=4, L=32),
})


def _forward(s):
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    g = layer.staged(x)
    y = layer.forward(x)
    torch.cuda.synchronize()
    gpu = {k: (np_of(v) if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    return inp, gpu, np_of(y)


@pytest.mark.parametrize("name", list(CASES))
def test_math_form_forward(name):
    s = CASES[name].replace(weight_layout="in_out")
    say(f"[layout] forward {name}: {s}")
    inp, gpu, y = _forward(s)
    _, gpu_lin, y_lin = _forward(s.replace(weight_layout="out_in"))
    np.testing.assert_array_equal(y, gpu["y"])          # fused = staged
    P = int(gpu["offsets"][-1])
    np.testing.assert_array_equal(gpu["y_sorted"][:P], gpu_lin["y_sorted"][:P])
    np.testing.assert_array_equal(y, y_lin)
    ref = oracle.layer_forward(inp, logits=gpu["logits"])
    err = row_error(y, ref["y"], s.dtype)
    say(f"[layout]   equal to the linear layout bit for bit; layer row error {err:.2e}")
    assert err <= tol(s.dtype)


@pytest.mark.parametrize("name", list(SMALL) + ["large-eight-waves-cut", "decode-I288"])
def test_math_form_backward(name):
    s = CASES[name].replace(weight_layout="in_out")
    say(f"[layout] backward {name}: {s}")
    inp = synth.make_layer(s)
    layer, x, dy_h, gpu, fused = run_gpu(s, inp)
    assert gpu["dw_gate"].shape == (s.L, s.H, s.I) and gpu["dw_down"].shape == (s.L, s.I, s.H)
    ref = B.layer_backward(inp, oracle.decode(dy_h, s.dtype), logits=gpu["logits"].astype(np.float64))
    np.testing.assert_array_equal(gpu["y"], gpu["y_inference"])
    P = int(ref["forward"]["offsets"][-1])
    rows_ok("dx_sorted", gpu["dx_sorted"][:P], ref["dx_sorted"][:P], s.dtype)
    for k in ("dw_gate", "dw_up", "dw_down", "dw_router"):
        mat_ok(k, gpu[k], ref[k], s.dtype)
    rows_ok("dx", gpu["dx"], ref["dx"], s.dtype)
    for k, v in fused.items():
        if v is not None:
            np.testing.assert_array_equal(v, gpu[k], err_msg=k)
