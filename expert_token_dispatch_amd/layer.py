"""Buffer management around the C ABI: one MoE layer's device tensors.

MoELayer owns the weights (torch device tensors in the library's layout), the
workspace, and the stage outputs, and calls the libmoe entry points on the
current torch stream.  It computes nothing itself.
"""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L


def to_device(a: Optional[np.ndarray], dtype: str, device="cuda") -> Optional[torch.Tensor]:
    """Host array -> device tensor.  bf16 arrays arrive as uint16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class MoELayer:
    def __init__(self, desc: L.LayerDesc, w_router, b_router, w_gate, w_up, w_down, device="cuda"):
        self.desc = desc
        self.device = torch.device(device)
        self.dtype = "bf16" if desc.dtype == L.MOE_BF16 else "f32"
        self.w_router, self.b_router = w_router, b_router
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        self.max_pairs = L.moe_max_pairs(desc)
        self._ws = {}

    @classmethod
    def from_host(cls, desc: L.LayerDesc, inp: dict, device="cuda") -> "MoELayer":
        dt = "bf16" if desc.dtype == L.MOE_BF16 else "f32"
        return cls(desc, to_device(inp["w_router"], dt, device), to_device(inp.get("b_router"), "f32", device),
                   to_device(inp["w_gate"], dt, device), to_device(inp["w_up"], dt, device),
                   to_device(inp["w_down"], dt, device), device)

    def workspace(self, stage: int) -> Optional[torch.Tensor]:
        if stage not in self._ws:
            n = L.moe_workspace_size(self.desc, stage)
            # 256-byte aligned: torch's caching allocator hands out 512-byte aligned blocks
            self._ws[stage] = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device) if n else None
        return self._ws[stage]

    def _empty(self, shape, dtype):
        return torch.empty(shape, dtype=dtype, device=self.device)

    # ---- stages ------------------------------------------------------------
    def route(self, x, logits_in=None, want_logits=False, want_topk_logit=None, opts=None):
        d = self.desc
        T, k, E = d.num_tokens, d.top_k, d.num_experts
        out = {"topk_ids": self._empty((T, k), torch.int32), "topk_w": self._empty((T, k), torch.float32)}
        if want_topk_logit is None:
            want_topk_logit = d.capacity_factor > 0
        out["topk_logit"] = self._empty((T, k), torch.float32) if want_topk_logit else None
        out["logits"] = self._empty((T, E), torch.float32) if want_logits else None
        L.moe_route_ex(d, opts, x, self.w_router, self.b_router, out["topk_ids"], out["topk_w"], out["topk_logit"],
                       logits_in=logits_in, logits_out=out["logits"], ws=self.workspace(L.MOE_STAGE_ROUTE))
        return out

    def dispatch(self, x, topk_ids, topk_logit=None):
        d = self.desc
        T, k, E, Lc, H = d.num_tokens, d.top_k, d.num_experts, d.local_count, d.hidden
        pm = max(self.max_pairs, 1)
        out = {
            "counts": self._empty((E,), torch.int32),
            "offsets": self._empty((Lc + 1,), torch.int32),
            "sorted_pairs": torch.full((pm,), -1, dtype=torch.int32, device=self.device),
            "pair_row": self._empty((T * k,), torch.int32),
            "x_sorted": self._empty((pm, H), x.dtype),
            "num_dropped": torch.zeros((1,), dtype=torch.int64, device=self.device),
        }
        L.moe_dispatch(d, x, topk_ids, topk_logit, out["counts"], out["offsets"], out["sorted_pairs"],
                       out["pair_row"], out["x_sorted"], out["num_dropped"], ws=self.workspace(L.MOE_STAGE_DISPATCH))
        return out

    def grouped_ffn(self, x_sorted, offsets):
        d = self.desc
        y_sorted = self._empty((max(self.max_pairs, 1), d.hidden), x_sorted.dtype)
        L.moe_grouped_ffn(d, x_sorted, offsets, self.w_gate, self.w_up, self.w_down, y_sorted,
                          ws=self.workspace(L.MOE_STAGE_FFN))
        return y_sorted

    def combine(self, y_sorted, pair_row, topk_w):
        d = self.desc
        y = self._empty((d.num_tokens, d.hidden), y_sorted.dtype)
        L.moe_combine(d, y_sorted, pair_row, topk_w, y)
        return y

    def forward(self, x, y=None, topk_ids_out=None, topk_w_out=None, counts_out=None, num_dropped_out=None,
                opts=None):
        """opts: an L.RouteOpts (selection bias, groups per token) or None."""
        d = self.desc
        if y is None:
            y = self._empty((d.num_tokens, d.hidden), x.dtype)
        L.moe_layer_forward_ex(d, opts, x, self.w_router, self.b_router, self.w_gate, self.w_up, self.w_down, y,
                               self.workspace(L.MOE_STAGE_LAYER), topk_ids_out, topk_w_out, counts_out,
                               num_dropped_out)
        return y

    def update_selection_bias(self, counts, bias, gamma):
        """One balancing step on the float32 [E] bias from a batch's [E] int32 expert loads."""
        L.moe_selection_bias_update(self.desc, counts, bias, gamma)
        return bias

    def staged(self, x, logits_in=None, opts=None):
        """The four stage calls one after another; returns every intermediate."""
        r = self.route(x, logits_in=logits_in, want_logits=True, want_topk_logit=True, opts=opts)
        dd = self.dispatch(x, r["topk_ids"], r["topk_logit"])
        ys = self.grouped_ffn(dd["x_sorted"], dd["offsets"])
        y = self.combine(ys, dd["pair_row"], r["topk_w"])
        return {**r, **dd, "y_sorted": ys, "y": y}

    # ---- training (Transformers "Expert parallelism", "Token dispatch") ----------
    def saved_buffers(self, x_dtype) -> dict:
        """Device buffers for the intermediates the training forward keeps."""
        d = self.desc
        T, k, Lc, H, I = d.num_tokens, d.top_k, d.local_count, d.hidden, d.intermediate
        pm = max(self.max_pairs, 1)
        return {
            "topk_ids": self._empty((max(T, 1), k), torch.int32),
            "topk_w": self._empty((max(T, 1), k), torch.float32),
            "offsets": self._empty((Lc + 1,), torch.int32),
            "pair_row": self._empty((max(T * k, 1),), torch.int32),
            "x_sorted": self._empty((pm, H), x_dtype),
            "gate": self._empty((pm, I), x_dtype),
            "up": self._empty((pm, I), x_dtype),
            "h": self._empty((pm, I), x_dtype),
            "y_sorted": self._empty((pm, H), x_dtype),
        }

    def forward_train(self, x, opts=None, saved=None, y=None, counts_out=None, num_dropped_out=None):
        """The layer forward that keeps what the backward needs; returns (y, saved)."""
        d = self.desc
        if y is None:
            y = self._empty((d.num_tokens, d.hidden), x.dtype)
        if saved is None:
            saved = L.make_saved(self.saved_buffers(x.dtype))
        L.moe_layer_forward_train(d, opts, x, self.w_router, self.b_router, self.w_gate, self.w_up, self.w_down, y,
                                  saved, self.workspace(L.MOE_STAGE_LAYER), counts_out, num_dropped_out)
        return y, saved

    def grad_buffers(self, x_dtype) -> dict:
        d = self.desc
        T, E, Lc, H, I = d.num_tokens, d.num_experts, d.local_count, d.hidden, d.intermediate
        return {
            "dx": self._empty((max(T, 1), H), x_dtype),
            "dw_router": self._empty((E, H), x_dtype),
            "db_router": self._empty((E,), torch.float32) if self.b_router is not None else None,
            # the weight gradients take the weights' layout
            "dw_gate": self._empty(tuple(self.w_gate.shape), x_dtype),
            "dw_up": self._empty(tuple(self.w_up.shape), x_dtype),
            "dw_down": self._empty(tuple(self.w_down.shape), x_dtype),
        }

    def backward(self, x, saved, dy, grads=None) -> dict:
        """Gradients of the layer given dy, from forward_train's saved intermediates."""
        if grads is None:
            grads = self.grad_buffers(dy.dtype)
        L.moe_layer_backward(self.desc, x, self.w_router, self.w_gate, self.w_up, self.w_down, saved, dy,
                             grads["dx"], grads["dw_router"], grads["db_router"], grads["dw_gate"], grads["dw_up"],
                             grads["dw_down"], self.workspace(L.MOE_STAGE_LAYER_BACKWARD))
        return grads

    def staged_backward(self, x, saved, dy) -> dict:
        """The four backward stage calls one after another; returns every intermediate."""
        d = self.desc
        T, k, H = d.num_tokens, d.top_k, d.hidden
        pm = max(self.max_pairs, 1)
        t = saved._tensors
        g = self.grad_buffers(dy.dtype)
        dys = self._empty((pm, H), dy.dtype)
        dl = self._empty((max(T, 1), k), torch.float32)
        L.moe_combine_backward(d, dy, t["y_sorted"], t["pair_row"], t["topk_w"], dys, dl)
        dxs = self._empty((pm, H), dy.dtype)
        L.moe_grouped_ffn_backward(d, t["x_sorted"], t["offsets"], self.w_gate, self.w_up, self.w_down, t["gate"],
                                   t["up"], t["h"], dys, dxs, g["dw_gate"], g["dw_up"], g["dw_down"],
                                   ws=self.workspace(L.MOE_STAGE_FFN_BACKWARD))
        L.moe_route_backward(d, x, t["topk_ids"], dl, g["dw_router"], g["db_router"],
                             ws=self.workspace(L.MOE_STAGE_ROUTE_BACKWARD))
        L.moe_dispatch_backward(d, dxs, t["pair_row"], t["topk_ids"], dl, self.w_router, g["dx"])
        return {**g, "dy_sorted": dys, "dl": dl, "dx_sorted": dxs}
