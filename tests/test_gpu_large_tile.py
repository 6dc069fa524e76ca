"""GPU parity of every variant of the large-tile grouped GEMM, on scaled
layers that select each variant the full-size workloads run.

The large-tile kernel (Ultralytics glossary "Expert Parallelism", "How tokens
move between GPUs", step 3: each GPU runs its local experts; Transformers
"Expert parallelism": the grouped_gemm expert rule) has these launch-time
variants:
  * four waves (products of 64 k steps or more) or eight waves (fewer);
  * each XCD's partly filled last round cut along K into pieces plus a fixup
    pass that adds them (K of 32 steps or more, few enough leftover tiles);
  * regular 256-row tiles and wide 128-row tail tiles.
The gpt-oss-like share (H = I = 2880: 45 steps) and the skewed layer's gate/up
(H = 2048: 32 steps) take eight waves with the cut; the mixtral-like layer
takes four waves.  Each case below asserts, from the kernel names the library
reports, that the variant it is meant for ran, then checks every row of the
grouped FFN output against the float64 oracle on the GPU's own x_sorted, the
layer output against the oracle layer, and the backward (whose dgrad products
run on the same kernel) against the backward oracle.
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

CASES = {
    # gpt-oss-like share with I a multiple of 64: 5-step products, eight waves, no cut
    "gptoss-I320": (synth.spec("gptoss_ep8_share", T=2048, H=320, I=320), {"ffn_plan"}, set()),
    # K = 2880 (45 steps) for both products, few tiles: eight waves, every last-round tile cut in two
    "K2880-cut": (synth.spec("gptoss_ep8_share", T=300, H=2880, I=2880, E=4, k=2, L=4),
                  {"ffn_plan", "ffn_gate_up_fixup", "ffn_down_fixup"}, set()),
    # the skewed layer's gate/up K = 2048 (32 steps) with capacity: eight waves, gate/up cut,
    # down (K = 1408, 22 steps) not cut
    "K2048-capacity-cut": (synth.spec("skewed_capacity", T=600, H=2048, I=1408, E=8, k=2, L=8),
                           {"ffn_plan", "ffn_gate_up_fixup"}, {"ffn_down_fixup"}),
    # four waves (K = 4096, 64 steps) with a cut of the down product (K = 4608)
    "K4096-four-waves": (synth.spec("mixtral_like", T=400, H=4096, I=4608, E=4, k=2, L=4),
                         {"ffn_plan", "ffn_down_fixup"}, set()),
}


def _kernel_names():
    import expert_token_dispatch_amd as etd
    return [etd.moe_profile_kernel_name(i) for i in range(etd.moe_profile_kernel_count())]


@pytest.mark.parametrize("name", list(CASES))
def test_large_tile_variant_forward(name):
    s, must, must_not = CASES[name]
    say(f"[large] {name}: {s}")
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    g = layer.staged(x)
    torch.cuda.synchronize()
    # the grouped FFN again on its own, to read the kernels it launched
    ys2 = layer.grouped_ffn(g["x_sorted"], g["offsets"])
    names = set(_kernel_names())
    torch.cuda.synchronize()
    say(f"[large]   kernels {sorted(names)}")
    assert must <= names, f"expected {must - names} to run"
    assert not (must_not & names), f"{must_not & names} ran"
    gpu = {k: (np_of(v) if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    offs = gpu["offsets"].astype(np.int64)
    P = int(offs[-1])
    np.testing.assert_array_equal(np_of(ys2)[:P], gpu["y_sorted"][:P])
    view = oracle.moe_oracle._ExpertView
    ref_ys = oracle.grouped_ffn(gpu["x_sorted"][:P].astype(np.float64), offs, view(inp["w_gate"], s.dtype),
                                view(inp["w_up"], s.dtype), view(inp["w_down"], s.dtype))
    e_ffn = row_error(gpu["y_sorted"][:P], ref_ys, s.dtype)
    ref = oracle.layer_forward(inp, logits=gpu["logits"])
    np.testing.assert_array_equal(gpu["offsets"], ref["offsets"])
    np.testing.assert_array_equal(gpu["pair_row"], ref["pair_row"])
    e_layer = row_error(gpu["y"], ref["y"], s.dtype)
    say(f"[large]   P={P} segments {np.diff(offs).tolist()}: every y_sorted row {e_ffn:.2e}, layer {e_layer:.2e}")
    assert e_ffn <= tol(s.dtype) and e_layer <= tol(s.dtype)


@pytest.mark.parametrize("name", ["K2880-cut", "K2048-capacity-cut"])
def test_large_tile_variant_backward(name):
    s, _, _ = CASES[name]
    say(f"[large] backward {name}: {s}")
    inp = synth.make_layer(s)
    layer, x, dy_h, gpu, fused = run_gpu(s, inp)
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
