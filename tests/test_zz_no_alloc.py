"""moe_dispatch_noalloc (the dispatch for callers that cannot allocate device
memory: its scratch is a static device array of the library) against
moe_dispatch with a caller workspace, through the C ABI.

Integer and index work and row copies, so the bar is bit-exact: counts,
offsets, the permutation, pair rows, the drop count and every gathered row.
Calls run back to back on one GPU, a large one and then smaller ones, with and
without the capacity cut, so each call finds the previous call's contents in
the shared scratch.
"""

import numpy as np
import pytest

import synth
from tests._harness import layer_of, np_of, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _both(s):
    import expert_token_dispatch_amd as etd
    inp = synth.make_layer(s, with_experts=False)
    inp["w_gate"] = inp["w_up"] = np.zeros((s.L, s.I, s.H), dtype=np.uint16 if s.dtype == "bf16" else np.float32)
    inp["w_down"] = np.zeros((s.L, s.H, s.I), dtype=inp["w_gate"].dtype)
    layer, x = layer_of(inp)
    r = layer.route(x, want_topk_logit=True)
    ref = layer.dispatch(x, r["topk_ids"], r["topk_logit"] if s.capacity_factor > 0 else None)
    d = layer.desc
    pm = max(layer.max_pairs, 1)
    out = {
        "counts": torch.full((s.E,), -7, dtype=torch.int32, device="cuda"),
        "offsets": torch.full((s.L + 1,), -7, dtype=torch.int32, device="cuda"),
        "sorted_pairs": torch.full((pm,), -1, dtype=torch.int32, device="cuda"),
        "pair_row": torch.full((s.T * s.k,), -7, dtype=torch.int32, device="cuda"),
        "x_sorted": torch.zeros((pm, s.H), dtype=x.dtype, device="cuda"),
        "num_dropped": torch.full((1,), -7, dtype=torch.int64, device="cuda"),
    }
    etd.moe_dispatch_noalloc(d, x, r["topk_ids"], r["topk_logit"] if s.capacity_factor > 0 else None,
                             out["counts"], out["offsets"], out["sorted_pairs"], out["pair_row"], out["x_sorted"],
                             out["num_dropped"])
    torch.cuda.synchronize()
    P = int(np_of(ref["offsets"])[-1])
    for k in ("counts", "offsets", "pair_row", "num_dropped"):
        np.testing.assert_array_equal(np_of(out[k]), np_of(ref[k]), err_msg=k)
    np.testing.assert_array_equal(np_of(out["sorted_pairs"])[:P], np_of(ref["sorted_pairs"])[:P])
    assert torch.equal(out["x_sorted"][:P], ref["x_sorted"][:P])
    say(f"[noalloc] {s.name} T={s.T}: P={P}, dropped {int(np_of(ref['num_dropped'])[0])}: bit-exact")
    return P


def test_noalloc_dispatch_matches_workspace_dispatch_call_after_call():
    # capacity path (scatter with the scan folded in, slice histograms, capacity cut over a
    # hot expert's two 4096-row slices, gather), then a smaller call of the same kind, then
    # the fused no-capacity path, then a smaller one of that
    cases = [
        synth.spec("skewed_capacity", T=6000, H=256, I=64),
        synth.spec("skewed_capacity", T=900, H=256, I=64),
        synth.spec("gptoss_ep8_share", T=5000, H=320, I=64),
        synth.spec("gptoss_ep8_share", T=700, H=320, I=64),
        synth.spec("decode_small", H=512, I=64),
    ]
    for s in cases:
        _both(s)


def test_noalloc_dispatch_rejects_sizes_past_its_buffer():
    import expert_token_dispatch_amd as etd
    from expert_token_dispatch_amd import _lib as L
    # 2^20 tokens of 256 experts: per-chunk histograms alone need 16 MiB + the local bases
    d = etd.make_desc(1 << 20, 64, 64, 256, 2)
    t = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(L.MoeError) as e:
        etd.moe_dispatch_noalloc(d, t, t, None, t, t, t, t, t, t)
    assert e.value.status == L.MOE_ERR_UNSUPPORTED
    assert "static buffer" in str(e.value)
