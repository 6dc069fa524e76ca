"""ctypes binding of libmoe (include/moe.h).  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_WEIGHTS_OUT_IN, MOE_WEIGHTS_IN_OUT = 0, 1
MOE_STAGE_ROUTE, MOE_STAGE_DISPATCH, MOE_STAGE_FFN, MOE_STAGE_COMBINE, MOE_STAGE_LAYER = 0, 1, 2, 3, 4
MOE_STAGE_FFN_BACKWARD, MOE_STAGE_ROUTE_BACKWARD, MOE_STAGE_LAYER_BACKWARD = 5, 6, 7

_STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED", -3: "MOE_ERR_WORKSPACE",
           -4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("local_begin", ctypes.c_int32),
        ("local_count", ctypes.c_int32),
        ("capacity_factor", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("weight_layout", ctypes.c_int32),
    ]


class RouteOpts(ctypes.Structure):
    """moe_route_opts: selection-only expert bias and groups per token (include/moe.h)."""
    _fields_ = [
        ("selection_bias", ctypes.c_void_p),
        ("num_groups", ctypes.c_int32),
        ("max_groups", ctypes.c_int32),
    ]


class Saved(ctypes.Structure):
    """moe_saved: what the training forward keeps for the backward (include/moe.h)."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_ids", "topk_w", "offsets", "pair_row", "x_sorted", "gate", "up", "h", "y_sorted")]


def make_saved(t: dict) -> Saved:
    """t: a dict of device tensors under the moe_saved field names.  The struct
    keeps a reference to the dict, so the pointers stay valid while it lives."""
    v = Saved(*[_p(t[n]) for n, _ in Saved._fields_])
    v._tensors = t
    return v


def make_route_opts(selection_bias=None, num_groups: int = 0, max_groups: int = 0) -> RouteOpts:
    """selection_bias: float32 [E] device tensor or None.  The options keep a
    reference to it, so the pointer stays valid while they are alive."""
    o = RouteOpts(_p(selection_bias), int(num_groups), int(max_groups))
    o._bias = selection_bias
    return o


def make_desc(num_tokens: int, hidden: int, intermediate: int, num_experts: int, top_k: int,
              local_begin: int = 0, local_count: Optional[int] = None, capacity_factor: float = 0.0,
              dtype="bf16", weight_layout="out_in") -> LayerDesc:
    """weight_layout: "out_in" (w_gate, w_up [L, I, H], w_down [L, H, I]) or "in_out"
    (w_gate, w_up [L, H, I], w_down [L, I, H]), or the MOE_WEIGHTS_* value."""
    if isinstance(dtype, str):
        dtype = {"bf16": MOE_BF16, "f32": MOE_F32}[dtype]
    if isinstance(weight_layout, str):
        weight_layout = {"out_in": MOE_WEIGHTS_OUT_IN, "in_out": MOE_WEIGHTS_IN_OUT}[weight_layout]
    return LayerDesc(num_tokens, hidden, intermediate, num_experts, top_k, local_begin,
                     num_experts if local_count is None else local_count, capacity_factor, dtype, weight_layout)


_LIB = None
_VP = ctypes.c_void_p
_DP = ctypes.POINTER(LayerDesc)
_OP = ctypes.c_void_p  # moe_route_opts*, NULL allowed


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built: run `python -m expert_token_dispatch_amd.build`")
        # torch first: its HIP runtime then serves libmoe too (one runtime per process)
        import torch  # noqa: F401
        L = ctypes.CDLL(lib_path)
        st = ctypes.c_int
        sig = {
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_version": (ctypes.c_char_p, []),
            "moe_ep_local_range": (st, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
            "moe_capacity": (ctypes.c_int64, [_DP]),
            "moe_max_pairs": (ctypes.c_int64, [_DP]),
            "moe_workspace_size": (st, [_DP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
            "moe_profile_events": (st, [ctypes.POINTER(_VP), ctypes.c_int32]),
            "moe_profile_kernel_name": (ctypes.c_char_p, [ctypes.c_int32]),
            "moe_profile_kernel_count": (ctypes.c_int32, []),
            "moe_route": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "moe_dispatch": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "moe_dispatch_noalloc": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
            "moe_grouped_ffn": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "moe_combine": (st, [_DP, _VP, _VP, _VP, _VP, _VP]),
            "moe_layer_forward": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                       ctypes.c_size_t, _VP]),
            "moe_route_ex": (st, [_DP, _OP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "moe_layer_forward_ex": (st, [_DP, _OP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          ctypes.c_size_t, _VP]),
            "moe_selection_bias_update": (st, [_DP, _VP, _VP, ctypes.c_float, _VP]),
            "moe_grouped_ffn_train": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                           _VP]),
            "moe_layer_forward_train": (st, [_DP, _OP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                             ctypes.c_size_t, _VP]),
            "moe_combine_backward": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
            "moe_grouped_ffn_backward": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                              _VP, ctypes.c_size_t, _VP]),
            "moe_route_backward": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
            "moe_dispatch_backward": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
            "moe_layer_backward": (st, [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                        ctypes.c_size_t, _VP]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _p(t) -> Optional[int]:
    """Device pointer of a torch tensor (None stays NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoe must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _s(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ws(ws):
    return (None, 0) if ws is None else (_p(ws), ws.numel() * ws.element_size())


# ---- host helpers ------------------------------------------------------------
def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_ep_local_range(num_experts: int, ep_size: int, rank: int) -> tuple[int, int]:
    b, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().moe_ep_local_range(num_experts, ep_size, rank, ctypes.byref(b), ctypes.byref(c)))
    return b.value, c.value


def moe_capacity(d: LayerDesc) -> int:
    return lib().moe_capacity(ctypes.byref(d))


def moe_max_pairs(d: LayerDesc) -> int:
    return lib().moe_max_pairs(ctypes.byref(d))


def moe_workspace_size(d: LayerDesc, stage: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(d), stage, ctypes.byref(n)))
    return n.value


def moe_profile_events(handles) -> None:
    """handles: list of hipEvent_t values (ints; None for both of a kernel's pair skips it),
    or None/[] to switch timing off."""
    if not handles:
        _check(lib().moe_profile_events(None, 0))
        return
    arr = (_VP * len(handles))(*handles)
    _check(lib().moe_profile_events(arr, len(handles)))
    moe_profile_events._keep = arr  # the library keeps the handles, not the array


def moe_profile_kernel_count() -> int:
    return lib().moe_profile_kernel_count()


def moe_profile_kernel_name(i: int) -> Optional[str]:
    r = lib().moe_profile_kernel_name(i)
    return None if r is None else r.decode()


# ---- the five stage calls ------------------------------------------------------
def moe_route(d, x, w_router, b_router, topk_ids, topk_w, topk_logit=None, logits_in=None, logits_out=None,
              ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_route(ctypes.byref(d), _p(x), _p(w_router), _p(b_router), _p(logits_in), _p(logits_out),
                           _p(topk_ids), _p(topk_w), _p(topk_logit), wp, wn, _s(stream)))


def moe_dispatch(d, x, topk_ids, topk_logit, counts, offsets, sorted_pairs, pair_row, x_sorted, num_dropped=None,
                 ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_dispatch(ctypes.byref(d), _p(x), _p(topk_ids), _p(topk_logit), _p(counts), _p(offsets),
                              _p(sorted_pairs), _p(pair_row), _p(x_sorted), _p(num_dropped), wp, wn, _s(stream)))


def moe_dispatch_noalloc(d, x, topk_ids, topk_logit, counts, offsets, sorted_pairs, pair_row, x_sorted,
                         num_dropped=None, stream=None) -> None:
    _check(lib().moe_dispatch_noalloc(ctypes.byref(d), _p(x), _p(topk_ids), _p(topk_logit), _p(counts), _p(offsets),
                                      _p(sorted_pairs), _p(pair_row), _p(x_sorted), _p(num_dropped), _s(stream)))


def moe_grouped_ffn(d, x_sorted, offsets, w_gate, w_up, w_down, y_sorted, ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_ffn(ctypes.byref(d), _p(x_sorted), _p(offsets), _p(w_gate), _p(w_up), _p(w_down),
                                 _p(y_sorted), wp, wn, _s(stream)))


def moe_combine(d, y_sorted, pair_row, topk_w, y, stream=None) -> None:
    _check(lib().moe_combine(ctypes.byref(d), _p(y_sorted), _p(pair_row), _p(topk_w), _p(y), _s(stream)))


def moe_layer_forward(d, x, w_router, b_router, w_gate, w_up, w_down, y, ws, topk_ids_out=None, topk_w_out=None,
                      counts_out=None, num_dropped_out=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_layer_forward(ctypes.byref(d), _p(x), _p(w_router), _p(b_router), _p(w_gate), _p(w_up),
                                   _p(w_down), _p(y), _p(topk_ids_out), _p(topk_w_out), _p(counts_out),
                                   _p(num_dropped_out), wp, wn, _s(stream)))


# ---- routing options (glossary "Load balancing and capacity") --------------------
def _opts(opts) -> Optional[int]:
    return None if opts is None else ctypes.addressof(opts)


def moe_route_ex(d, opts, x, w_router, b_router, topk_ids, topk_w, topk_logit=None, logits_in=None, logits_out=None,
                 ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_route_ex(ctypes.byref(d), _opts(opts), _p(x), _p(w_router), _p(b_router), _p(logits_in),
                              _p(logits_out), _p(topk_ids), _p(topk_w), _p(topk_logit), wp, wn, _s(stream)))


def moe_layer_forward_ex(d, opts, x, w_router, b_router, w_gate, w_up, w_down, y, ws, topk_ids_out=None,
                         topk_w_out=None, counts_out=None, num_dropped_out=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_layer_forward_ex(ctypes.byref(d), _opts(opts), _p(x), _p(w_router), _p(b_router), _p(w_gate),
                                      _p(w_up), _p(w_down), _p(y), _p(topk_ids_out), _p(topk_w_out),
                                      _p(counts_out), _p(num_dropped_out), wp, wn, _s(stream)))


def moe_selection_bias_update(d, counts, bias, gamma: float, stream=None) -> None:
    _check(lib().moe_selection_bias_update(ctypes.byref(d), _p(counts), _p(bias), float(gamma), _s(stream)))


# ---- training: the backward pass (Transformers "Expert parallelism", "Token dispatch") ----
def _saved(v) -> Optional[int]:
    return None if v is None else ctypes.addressof(v)


def moe_grouped_ffn_train(d, x_sorted, offsets, w_gate, w_up, w_down, y_sorted, h, gate, up, ws=None,
                          stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_ffn_train(ctypes.byref(d), _p(x_sorted), _p(offsets), _p(w_gate), _p(w_up), _p(w_down),
                                       _p(y_sorted), _p(h), _p(gate), _p(up), wp, wn, _s(stream)))


def moe_layer_forward_train(d, opts, x, w_router, b_router, w_gate, w_up, w_down, y, saved, ws, counts_out=None,
                            num_dropped_out=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_layer_forward_train(ctypes.byref(d), _opts(opts), _p(x), _p(w_router), _p(b_router), _p(w_gate),
                                         _p(w_up), _p(w_down), _p(y), _saved(saved), _p(counts_out),
                                         _p(num_dropped_out), wp, wn, _s(stream)))


def moe_combine_backward(d, dy, y_sorted, pair_row, topk_w, dy_sorted, dl, stream=None) -> None:
    _check(lib().moe_combine_backward(ctypes.byref(d), _p(dy), _p(y_sorted), _p(pair_row), _p(topk_w),
                                      _p(dy_sorted), _p(dl), _s(stream)))


def moe_grouped_ffn_backward(d, x_sorted, offsets, w_gate, w_up, w_down, gate, up, h, dy_sorted, dx_sorted, dw_gate,
                             dw_up, dw_down, ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_grouped_ffn_backward(ctypes.byref(d), _p(x_sorted), _p(offsets), _p(w_gate), _p(w_up),
                                          _p(w_down), _p(gate), _p(up), _p(h), _p(dy_sorted), _p(dx_sorted),
                                          _p(dw_gate), _p(dw_up), _p(dw_down), wp, wn, _s(stream)))


def moe_route_backward(d, x, topk_ids, dl, dw_router, db_router=None, ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_route_backward(ctypes.byref(d), _p(x), _p(topk_ids), _p(dl), _p(dw_router), _p(db_router),
                                    wp, wn, _s(stream)))


def moe_dispatch_backward(d, dx_sorted, pair_row, topk_ids, dl, w_router, dx, stream=None) -> None:
    _check(lib().moe_dispatch_backward(ctypes.byref(d), _p(dx_sorted), _p(pair_row), _p(topk_ids), _p(dl),
                                       _p(w_router), _p(dx), _s(stream)))


def moe_layer_backward(d, x, w_router, w_gate, w_up, w_down, saved, dy, dx, dw_router, db_router, dw_gate, dw_up,
                       dw_down, ws, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_layer_backward(ctypes.byref(d), _p(x), _p(w_router), _p(w_gate), _p(w_up), _p(w_down),
                                    _saved(saved), _p(dy), _p(dx), _p(dw_router), _p(db_router), _p(dw_gate),
                                    _p(dw_up), _p(dw_down), wp, wn, _s(stream)))
