"""The C ABI without a GPU: the library loads, exports every declared symbol,
its host helpers follow the pages, and bad arguments are rejected before any
work is enqueued (every call here fails validation or is a T == 0 no-op, so
no kernel is launched)."""

import ctypes
import json
import os
import re

import pytest

import expert_token_dispatch_amd as etd
from expert_token_dispatch_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(L.lib_path)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert etd.moe_version().startswith("libmoe")


def test_ep_local_range_matches_layout_figure():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "rank_layout_8ranks.json")))
    for ep, table in g["experts_by_rank"].items():
        for rank, experts in enumerate(table):
            b, n = etd.moe_ep_local_range(g["num_experts"], int(ep), rank)
            assert list(range(b, b + n)) == experts


@pytest.mark.parametrize("E,ep,rank", [(8, 3, 0), (8, 0, 0), (0, 1, 0), (8, 2, -1)])
def test_ep_local_range_rejects(E, ep, rank):
    with pytest.raises(L.MoeError) as e:
        etd.moe_ep_local_range(E, ep, rank)
    assert e.value.status == L.MOE_ERR_INVALID_ARG


def test_capacity_and_max_pairs():
    d = etd.make_desc(32768, 2048, 1408, 64, 6, capacity_factor=1.25)
    assert etd.moe_capacity(d) == 3840
    assert etd.moe_max_pairs(d) == min(32768 * 6, 64 * 3840)
    d = etd.make_desc(32768, 2048, 1408, 64, 6, local_begin=8, local_count=16, capacity_factor=1.25)
    assert etd.moe_max_pairs(d) == 16 * 3840
    d = etd.make_desc(8192, 4096, 14336, 8, 2)
    assert etd.moe_capacity(d) == -1
    assert etd.moe_max_pairs(d) == 16384
    d = etd.make_desc(100, 64, 64, 8, 2, capacity_factor=10.0)   # limit above T*k
    assert etd.moe_capacity(d) == 250
    assert etd.moe_max_pairs(d) == 200


def test_workspace_sizes_cover_buffers():
    d = etd.make_desc(8192, 4096, 14336, 8, 2)
    ffn = etd.moe_workspace_size(d, L.MOE_STAGE_FFN)
    assert ffn >= 16384 * 14336 * 2
    layer = etd.moe_workspace_size(d, L.MOE_STAGE_LAYER)
    assert layer >= ffn + 2 * 16384 * 4096 * 2
    assert etd.moe_workspace_size(d, L.MOE_STAGE_ROUTE) >= 8192 * 8 * 4   # per-slice partial logits
    assert etd.moe_workspace_size(d, L.MOE_STAGE_DISPATCH) > 0


BAD = [
    dict(num_tokens=-1),
    dict(hidden=0), dict(hidden=12), dict(intermediate=4),
    dict(num_experts=0), dict(top_k=0), dict(top_k=9),
    dict(local_begin=-1), dict(local_count=0), dict(local_begin=4, local_count=5),
    dict(dtype=7), dict(capacity_factor=float("nan")),
]


@pytest.mark.parametrize("over", BAD)
def test_invalid_descriptor_rejected_before_launch(over):
    base = dict(num_tokens=16, hidden=64, intermediate=64, num_experts=8, top_k=2, local_begin=0,
                local_count=8, capacity_factor=0.0, dtype=L.MOE_BF16)
    base.update(over)
    d = L.LayerDesc(**base)
    lib = L.lib()
    st = lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None)
    assert st == L.MOE_ERR_INVALID_ARG, L.moe_last_error()
    assert L.moe_last_error()
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_capacity(ctypes.byref(d)) == -1


def test_unsupported_sizes():
    lib = L.lib()
    d = etd.make_desc(16, 64, 64, 300, 2)     # router handles E <= 256
    st = lib.moe_route(ctypes.byref(d), 16, 16, None, None, None, 16, 16, None, None, 0, None)
    assert st == L.MOE_ERR_UNSUPPORTED
    d = etd.make_desc(16, 64, 64, 64, 33)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(d), 4, ctypes.byref(n)) == L.MOE_ERR_UNSUPPORTED


def test_null_and_misaligned_pointers_rejected():
    lib = L.lib()
    d = etd.make_desc(16, 64, 64, 8, 2)
    # NULL x
    assert lib.moe_route(ctypes.byref(d), None, 256, None, None, None, 256, 256, None, None, 0, None) \
        == L.MOE_ERR_INVALID_ARG
    assert "x is NULL" in L.moe_last_error()
    # misaligned router weight
    assert lib.moe_route(ctypes.byref(d), 256, 258, None, None, None, 256, 256, None, None, 0, None) \
        == L.MOE_ERR_INVALID_ARG
    assert "aligned" in L.moe_last_error()
    # combine: misaligned output
    assert lib.moe_combine(ctypes.byref(d), 256, 256, 256, 264, None) == L.MOE_ERR_INVALID_ARG
    # capacity needs the chosen logits
    dc = etd.make_desc(16, 64, 64, 8, 2, capacity_factor=1.0)
    st = lib.moe_dispatch(ctypes.byref(dc), 256, 256, None, 256, 256, 256, 256, 256, None, 256, 1 << 20, None)
    assert st == L.MOE_ERR_INVALID_ARG and "topk_logit" in L.moe_last_error()


def test_workspace_too_small():
    lib = L.lib()
    d = etd.make_desc(16, 64, 64, 8, 2)
    st = lib.moe_dispatch(ctypes.byref(d), 256, 256, None, 256, 256, 256, 256, 256, None, 256, 4, None)
    assert st == L.MOE_ERR_WORKSPACE
    st = lib.moe_grouped_ffn(ctypes.byref(d), 256, 256, 256, 256, 256, 256, None, 0, None)
    assert st == L.MOE_ERR_WORKSPACE
    st = lib.moe_layer_forward(ctypes.byref(d), 256, 256, None, 256, 256, 256, 256, None, None, None, None,
                               None, 0, None)
    assert st == L.MOE_ERR_WORKSPACE


def test_zero_tokens_is_a_noop():
    lib = L.lib()
    d = etd.make_desc(0, 64, 64, 8, 2)
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, None, None, None, None, None, 0, None) == L.MOE_OK
    assert lib.moe_dispatch(ctypes.byref(d), *([None] * 10), 0, None) == L.MOE_OK
    assert lib.moe_grouped_ffn(ctypes.byref(d), *([None] * 7), 0, None) == L.MOE_OK
    assert lib.moe_combine(ctypes.byref(d), None, None, None, None, None) == L.MOE_OK
    assert lib.moe_layer_forward(ctypes.byref(d), *([None] * 12), 0, None) == L.MOE_OK
    assert lib.moe_profile_kernel_count() == 0


@pytest.mark.parametrize("G,M,code", [(3, 1, "INVALID_ARG"), (32, 1, "UNSUPPORTED"), (4, 0, "INVALID_ARG"),
                                      (4, 5, "INVALID_ARG"), (8, 1, "INVALID_ARG")])
def test_route_options_rejected_before_launch(G, M, code):
    # groups must divide E (8 here), at most 16 of them, 1 <= max_groups <= num_groups, and
    # the groups a token may use must hold at least k experts (8 groups of one, k = 2)
    lib = L.lib()
    d = etd.make_desc(16, 64, 64, 8, 2)
    opts = L.make_route_opts(None, G, M)
    st = lib.moe_route_ex(ctypes.byref(d), ctypes.addressof(opts), 256, 256, None, None, None, 256, 256, None, None,
                          0, None)
    assert st == getattr(L, "MOE_ERR_" + code), L.moe_last_error()
    assert "route options" in L.moe_last_error()
    st = lib.moe_layer_forward_ex(ctypes.byref(d), ctypes.addressof(opts), 256, 256, None, 256, 256, 256, 256, None,
                                  None, None, None, 256, 1 << 30, None)
    assert st == getattr(L, "MOE_ERR_" + code), L.moe_last_error()


def test_selection_bias_update_arguments_checked():
    lib = L.lib()
    d = etd.make_desc(16, 64, 64, 8, 2)
    assert lib.moe_selection_bias_update(ctypes.byref(d), None, 256, 0.001, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_selection_bias_update(ctypes.byref(d), 256, None, 0.001, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_selection_bias_update(ctypes.byref(d), 256, 256, float("nan"), None) == L.MOE_ERR_INVALID_ARG


def _saved(**null):
    v = L.Saved(*[None if n in null else 256 for n, _ in L.Saved._fields_])
    return v


def test_backward_workspace_sizes():
    d = etd.make_desc(1000, 512, 896, 8, 2)
    pm = 2000
    assert etd.moe_workspace_size(d, L.MOE_STAGE_FFN_BACKWARD) >= 2 * pm * 896 * 2
    assert etd.moe_workspace_size(d, L.MOE_STAGE_ROUTE_BACKWARD) >= 1000 * 8 * (2 + 4)
    lb = etd.moe_workspace_size(d, L.MOE_STAGE_LAYER_BACKWARD)
    assert lb >= (etd.moe_workspace_size(d, L.MOE_STAGE_FFN_BACKWARD) + etd.moe_workspace_size(d, L.MOE_STAGE_ROUTE_BACKWARD)
                  + 2 * pm * 512 * 2 + 1000 * 2 * 4)
    n = ctypes.c_size_t()
    assert L.lib().moe_workspace_size(ctypes.byref(d), 8, ctypes.byref(n)) == L.MOE_ERR_INVALID_ARG


def test_backward_arguments_rejected_before_launch():
    lib = L.lib()
    d = etd.make_desc(16, 64, 64, 8, 2)
    b = ctypes.byref
    # the fused backward needs the saved intermediates
    st = lib.moe_layer_backward(b(d), 256, 256, 256, 256, 256, None, 256, 256, 256, None, 256, 256, 256, 256, 1 << 30,
                                None)
    assert st == L.MOE_ERR_INVALID_ARG and "saved is NULL" in L.moe_last_error()
    v = _saved(gate=1)
    st = lib.moe_layer_backward(b(d), 256, 256, 256, 256, 256, ctypes.addressof(v), 256, 256, 256, None, 256, 256, 256,
                                256, 1 << 30, None)
    assert st == L.MOE_ERR_INVALID_ARG and "gate" in L.moe_last_error()
    v = _saved()
    st = lib.moe_layer_backward(b(d), 256, 256, 256, 256, 256, ctypes.addressof(v), 256, 256, 256, None, 256, 256, 256,
                                256, 16, None)
    assert st == L.MOE_ERR_WORKSPACE
    v = _saved(h=1)
    st = lib.moe_layer_forward_train(b(d), None, 256, 256, None, 256, 256, 256, 256, ctypes.addressof(v),
                                     None, None, 256, 1 << 30, None)
    assert st == L.MOE_ERR_INVALID_ARG and "h is NULL" in L.moe_last_error()
    # stage calls
    assert lib.moe_combine_backward(b(d), None, 256, 256, 256, 256, 256, None) == L.MOE_ERR_INVALID_ARG
    assert "dy is NULL" in L.moe_last_error()
    st = lib.moe_grouped_ffn_backward(b(d), *([256] * 13), 256, 16, None)
    assert st == L.MOE_ERR_WORKSPACE
    st = lib.moe_route_backward(b(d), 256, 256, 256, 264, None, 256, 1 << 20, None)
    assert st == L.MOE_ERR_INVALID_ARG and "dw_router" in L.moe_last_error()
    assert lib.moe_dispatch_backward(b(d), 256, 256, 256, 256, None, 256, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_grouped_ffn_train(b(d), 256, 256, 256, 256, 256, 256, 256, None, 256, 256, 1 << 30, None) \
        == L.MOE_ERR_INVALID_ARG


def test_backward_with_zero_tokens():
    # no rows: the stage calls that only touch rows are no-ops; the weight gradients of a
    # layer that saw no tokens are zero, so those calls still need their buffers
    lib = L.lib()
    d = etd.make_desc(0, 64, 64, 8, 2)
    b = ctypes.byref
    assert lib.moe_combine_backward(b(d), *([None] * 6), None) == L.MOE_OK
    assert lib.moe_dispatch_backward(b(d), *([None] * 6), None) == L.MOE_OK
    assert lib.moe_grouped_ffn_train(b(d), *([None] * 10), 0, None) == L.MOE_OK
    assert lib.moe_layer_forward_train(b(d), *([None] * 12), 0, None) == L.MOE_OK
    assert lib.moe_grouped_ffn_backward(b(d), *([None] * 13), None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route_backward(b(d), None, None, None, None, None, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_backward(b(d), *([None] * 14), 0, None) == L.MOE_ERR_INVALID_ARG
