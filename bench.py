"""Benchmark: one MoE layer forward (route -> dispatch -> grouped SwiGLU FFN ->
combine) on one MI355X through the libmoe C ABI.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--backward]

A step is one moe_layer_forward over one batch of seeded synthetic input that
is already resident in HBM (with --backward: one training step of the layer,
moe_layer_forward_train then moe_layer_backward on a seeded upstream gradient).  W untimed steps, then exactly K timed steps
between two device synchronisations.  Every kernel of every timed step is
also bracketed by HIP events on the launch stream (the library records them),
which gives each kernel's average duration; the roofline entry uses the
dominant kernel.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer (1 GPU, bf16) + grouped-GEMM % MFMA peak"
METRIC_TRAIN = "routed tokens/s per MoE layer training step (forward keeping activations + backward; 1 GPU)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime that torch already loaded.  They are created
    timing-only (hipEventDisableSystemFence): recording one does not write back and invalidate
    the caches, which would otherwise add a few microseconds to every kernel the events bracket
    (most for kernels that leave much dirty data in L2)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(e.value)
        return out

    def record(self, e, stream) -> None:
        """Record event e on the hipStream_t stream (an int handle, e.g. a torch stream's cuda_stream)."""
        if self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_work(name: str, s, P: int, touched_tokens: int, touched_experts: int, nblk: int,
                train: bool = False) -> tuple[float, float]:
    """Algorithmic (bytes, flops) of one launch of a libmoe kernel (train: the
    training forward, whose gate/up kernel also writes the pre-activations)."""
    dt = 2 if s.dtype == "bf16" else 4
    T, H, I, E, k = s.T, s.H, s.I, s.E, s.k
    cap = s.capacity_factor > 0
    if name == "route_logits":
        return (T * H + E * H) * dt + T * E * 4, 2.0 * T * H * E
    if name == "route_topk":
        return T * E * 4 * 2 + T * k * (12 if cap else 8), 0.0
    if name == "dispatch_count":
        return T * k * 4 + nblk * E * 4, 0.0
    if name == "dispatch_scan":
        return nblk * E * 4 * 2, 0.0
    if name == "dispatch_scatter":  # ids, logits, chunk counts in; pair_row, pre-capacity permutation and keys out
        return T * k * 4 * 5 + nblk * E * 4, 0.0
    if name == "dispatch_cap_hist":  # the keys of the experts over capacity (at most all of them)
        return T * k * 4, 0.0
    if name == "dispatch_capacity":
        return T * k * 4 * 3, 0.0
    if name == "dispatch_gather":
        return (touched_tokens + P) * H * dt + P * 4, 0.0
    if name == "dispatch_place":
        # ranks from the pair ids and chunk bases, both permutation arrays, and the row copy
        return T * k * 4 * 2 + nblk * E * 4 + P * 4 + (touched_tokens + P) * H * dt, 0.0
    if name == "ffn_gate_up":
        return P * H * dt + 2 * touched_experts * I * H * dt + (3 if train else 1) * P * I * dt, 4.0 * P * H * I
    if name == "ffn_down":
        return P * I * dt + touched_experts * H * I * dt + P * H * dt, 2.0 * P * H * I
    if name == "combine":
        return P * H * dt + T * k * 8 + T * H * dt, 0.0
    # backward (training): dy_sorted, dl; dh -> dg, du; dW; dx_sorted; router; dx
    Ep = (E + 7) // 8 * 8
    Lc = s.L
    if name == "combine_bwd":
        return (T * H + 2 * P * H) * dt + T * k * 12, 0.0
    if name == "ffn_down_dgrad":
        return (P * H + touched_experts * H * I + 4 * P * I) * dt, 2.0 * P * H * I
    if name == "ffn_down_wgrad":
        return (P * H + P * I + Lc * H * I) * dt, 2.0 * P * H * I
    if name == "ffn_gate_up_dgrad":
        return (2 * P * I + 2 * touched_experts * I * H + P * H) * dt, 4.0 * P * H * I
    if name == "ffn_gate_up_wgrad":
        return (2 * P * I + P * H + 2 * Lc * I * H) * dt, 4.0 * P * H * I
    if name == "ffn_bwd_transpose":  # one expert matrix stack read and written per launch
        return 2 * Lc * H * I * dt, 0.0
    if name == "ffn_bwd_seg_transpose":  # dy_sorted, h, dg|du, x_sorted: (2H + 3I) columns over 4 launches
        return 2 * P * (2 * H + 3 * I) * dt / 4, 0.0
    if name == "route_bwd_dlogits":
        return T * k * 8 + T * Ep * (dt + 4), 0.0
    if name == "route_bwd_wgrad":
        return (T * H + T * Ep + E * H) * dt, 2.0 * T * k * H
    if name == "route_bwd_bias":
        return T * Ep * 4, 0.0
    if name == "dispatch_bwd":
        return (P * H + T * H + E * H) * dt + T * k * 12, 0.0
    return 0.0, 0.0


def source_digest(paths) -> str:
    """First 16 hex digits of the SHA-256 of the named files' bytes, concatenated in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str, training: bool = False):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel's source file and
    the local headers it builds on still match the recorded digest (training-step runs are recorded
    under their own keys: their kernels are other instantiations)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{workload}:{kernel}" + (":training" if training else ""))
    except (OSError, ValueError):
        return None
    if not rec or not isinstance(rec.get("sources"), list):
        return None
    srcs = [os.path.join(ROOT, "expert_token_dispatch_amd", "csrc", f) for f in rec["sources"]]
    if not all(os.path.exists(f) for f in srcs) or source_digest(srcs) != rec["source_sha"]:
        return None
    return rec["bytes_per_launch"]


def _oracle_forward_steps(sub) -> tuple[dict, dict]:
    """The oracle layer forward step by step (its own functions, in the order of its
    layer_forward), with the seconds each step took."""
    import oracle
    from oracle.moe_oracle import expert_views
    s = sub["spec"]
    dt = s.dtype
    sec = {}
    t0 = time.perf_counter()
    x = oracle.decode(sub["x"], dt)
    wr = oracle.decode(sub["w_router"], dt)
    br = sub.get("b_router")
    br = None if br is None else br.astype("float64")
    r = oracle.route(x, wr, br, s.k)
    t1 = time.perf_counter()
    sec["route"] = t1 - t0
    d = oracle.dispatch(r["topk_ids"], r["topk_logit"], s.E, s.local_begin, s.L, s.capacity_factor, x=x)
    t2 = time.perf_counter()
    sec["dispatch"] = t2 - t1
    ys = oracle.grouped_ffn(d["x_sorted"], d["offsets"], *expert_views(sub))
    t3 = time.perf_counter()
    sec["grouped_ffn"] = t3 - t2
    y = oracle.combine(ys, d["pair_row"], r["topk_w"])
    sec["combine"] = time.perf_counter() - t3
    return {**r, **d, "y_sorted": ys, "y": y, "tokens": None}, sec


def cpu_baseline(inp, tokens: int, backward: bool = False) -> dict:
    """The oracle as it stands, on the first `tokens` tokens of the same layer
    (with backward: its forward and backward, a training step), timed per step."""
    import numpy as np
    import oracle
    import oracle.moe_backward as ob
    import synth
    from threadpoolctl import threadpool_info
    s = inp["spec"]
    sub = dict(inp)
    sub["spec"] = s.replace(T=tokens)
    sub["x"] = np.ascontiguousarray(inp["x"][:tokens])
    dy = oracle.decode(synth.make_upstream_grad(s)[:tokens], s.dtype) if backward else None
    t0 = time.perf_counter()
    fwd, sec = _oracle_forward_steps(sub)
    if backward:
        tb = time.perf_counter()
        ob.layer_backward(sub, dy, fwd_out=fwd)
        sec["backward"] = time.perf_counter() - tb
    dt = time.perf_counter() - t0
    info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    blas = [i.get("num_threads", 1) for i in info]
    lib = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip() for i in info})) or "none"
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    nth = int(max(blas) if blas else 1)
    return {"value": tokens / dt, "unit": "tokens/s", "cores": nth, "kind": "oracle",
            "seconds_per_step": {k: round(v, 3) for k, v in sec.items()},
            "blas": lib,
            "sample": f"first {tokens} of {s.T} tokens of the same layer, all {s.L} experts' weights; "
                      f"whole oracle {'forward + backward' if backward else 'path'} (float64) in {dt:.1f} s; "
                      f"host has {os.cpu_count()} CPUs ({model}); BLAS ({lib}) threads {nth} in the expert "
                      f"products; routing, counting-sort and combine loops single-threaded NumPy"}


def routing_report(inp, ids_gpu, counts_gpu, dropped: int, P: int, with_oracle: bool) -> dict:
    """The realised routing of the timed layer: per-expert loads (all E, before any capacity
    cut), per-rank loads of an expert-parallel split when this GPU holds one block, the drop
    count; and, from the oracle's float64 logits, the top-k flips (tokens whose chosen set
    differs) with the smallest and largest logit gap among them."""
    import numpy as np
    s = inp["spec"]
    cnt = np.asarray(counts_gpu, dtype=np.int64)
    out = {"expert_load_min": int(cnt.min()), "expert_load_max": int(cnt.max()),
           "even_share": s.T * s.k / s.E, "experts_empty": int((cnt == 0).sum()),
           "local_pairs_routed": int(cnt[s.local_begin:s.local_begin + s.L].sum()),
           "pairs_kept": P, "pairs_dropped": dropped}
    if s.L < s.E and s.E % s.L == 0:
        ranks = cnt.reshape(s.E // s.L, s.L).sum(axis=1)
        out["rank_loads"] = {"ranks": s.E // s.L, "min": int(ranks.min()), "max": int(ranks.max())}
    if with_oracle:
        import oracle
        x = oracle.decode(inp["x"], s.dtype)
        wr = oracle.decode(inp["w_router"], s.dtype)
        br = None if inp["b_router"] is None else inp["b_router"].astype(np.float64)
        lg64 = oracle.router_logits(x, wr, br)
        del x
        ref = oracle.topk_select(lg64, s.k)
        bad = np.flatnonzero(np.any(np.sort(ids_gpu, axis=1) != np.sort(ref, axis=1), axis=1))
        if s.k < s.E:
            srt = -np.sort(-lg64, axis=1)
            gap = srt[:, s.k - 1] - srt[:, s.k]
        else:
            gap = np.full(s.T, np.inf)
        out["topk_flips"] = int(len(bad))
        out["flip_gap_min"] = float(gap[bad].min()) if len(bad) else None
        out["flip_gap_max"] = float(gap[bad].max()) if len(bad) else None
        out["flip_gap_allowed"] = 1e-5
    return out


def copy_probe(s, P: int) -> dict:
    """Library copy kernels with the byte mixes of the layer's memory-bound stages:
    torch.index_select gathering P rows of [T, H] (reads T*H, writes P*H: dispatch_place's
    mix) and torch.add of two [T, H] halves of a [P, H] buffer (reads P*H, writes T*H:
    combine's mix, for k = 2).  Eight buffer sets rotate so the 256 MB Infinity Cache holds
    none of the next call's inputs.  Timed per call with the same timing-only HIP events as
    the library's kernels (median of 20)."""
    import torch
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    esz = 2 if s.dtype == "bf16" else 4
    nset = 8
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    xs = [torch.empty((s.T, s.H), dtype=dt, device="cuda").normal_(generator=g) for _ in range(nset)]
    idx = torch.randperm(P, device="cuda", generator=g) % s.T
    outs = [torch.empty((P, s.H), dtype=dt, device="cuda") for _ in range(nset)]
    res = {}
    for name, fn, rd, wr in (
            ("gather (dispatch_place mix)", lambda i: torch.index_select(xs[i], 0, idx, out=outs[i]), s.T, P),
            ("add (combine mix)", lambda i: torch.add(outs[i][:P // 2], outs[i][P // 2:2 * (P // 2)],
                                                       out=xs[i][:P // 2]), 2 * (P // 2), P // 2)):
        for i in range(nset):
            fn(i)
        torch.cuda.synchronize()
        ms = []
        hip = HipEvents()
        st = torch.cuda.current_stream().cuda_stream
        for r in range(20):
            ev = hip.create(2)
            hip.record(ev[0], st)
            fn(r % nset)
            hip.record(ev[1], st)
            torch.cuda.synchronize()
            ms.append(hip.elapsed_ms(ev[0], ev[1]))
            hip.destroy(ev)
        ms.sort()
        med = ms[len(ms) // 2]
        by = (rd + wr) * s.H * esz
        res[name] = {"us": round(med * 1e3, 2), "bytes": by, "GB/s": round(by / (med * 1e-3) / 1e9, 1),
                     "hbm_frac": round(by / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del xs, outs
    return res


def gemm_probe(s, P: int) -> dict:
    """The library's grouped FFN and the vendor library on the dense products with the grouped
    products' flops: one expert holding all P rows ([P, H] through gate/up [2I, H] and down
    [H, I]), first through this library (offsets [0, P]; its gate/up also applies SwiGLU and
    writes [P, I]), then torch.matmul (hipBLASLt) on the same shapes ([P, H] x [H, 2I] and
    [P, I] x [I, H], bf16 out, float32 accumulation).  A dense product has no segment tails
    and reads one weight matrix instead of L.  Timed per call with the same timing-only HIP events
    as the library's kernels (median of 10)."""
    import torch
    import synth
    import expert_token_dispatch_amd as etd
    from expert_token_dispatch_amd.layer import MoELayer
    if s.dtype != "bf16":
        return {}
    res = {}
    d1 = synth.spec(s.name, T=P, E=1, k=1, local_begin=0, L=1, capacity_factor=0.0)
    lay = MoELayer.from_host(etd.make_desc(d1.T, d1.H, d1.I, 1, 1, 0, 1, 0.0, "bf16"), synth.make_layer(d1))
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    xs = torch.empty((P, s.H), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    offs = torch.tensor([0, P], dtype=torch.int32, device="cuda")
    hip = HipEvents()
    for _ in range(2):
        lay.grouped_ffn(xs, offs)
    torch.cuda.synchronize()
    per = {}
    for _ in range(10):
        ev = hip.create(16)
        etd.moe_profile_events(ev)
        lay.grouped_ffn(xs, offs)
        etd.moe_profile_events(None)
        torch.cuda.synchronize()
        for i in range(etd.moe_profile_kernel_count()):
            per.setdefault(etd.moe_profile_kernel_name(i), []).append(hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]))
        hip.destroy(ev)
    flops = {"ffn_gate_up": 4.0 * P * s.H * s.I, "ffn_down": 2.0 * P * s.H * s.I}
    for n, ts in per.items():
        med = sorted(ts)[len(ts) // 2]
        e = {"us": round(med * 1e3, 2)}
        if n in flops:
            tf = flops[n] / (med * 1e-3) / 1e12
            e.update({"TFLOP/s": round(tf, 1), "mfma_frac": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4)})
        res[f"library {n}, one expert of {P} rows"] = e
    del lay, xs
    for name, M, N, K in (("gate_up", P, 2 * s.I, s.H), ("down", P, s.H, s.I)):
        a = torch.empty((M, K), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
        w = torch.empty((N, K), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            torch.matmul(a, w.t(), out=c)
        torch.cuda.synchronize()
        ms = []
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(10):
            ev = hip.create(2)
            hip.record(ev[0], st)
            torch.matmul(a, w.t(), out=c)
            hip.record(ev[1], st)
            torch.cuda.synchronize()
            ms.append(hip.elapsed_ms(ev[0], ev[1]))
            hip.destroy(ev)
        ms.sort()
        med = ms[len(ms) // 2]
        tf = 2.0 * M * N * K / (med * 1e-3) / 1e12
        res[f"hipBLASLt {name} [{M}x{K}]x[{K}x{N}]"] = {"us": round(med * 1e3, 2), "TFLOP/s": round(tf, 1),
                                                        "mfma_frac": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4)}
        del a, w, c
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_like")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--weight-layout", choices=["out_in", "in_out"], default="out_in",
                    help="expert weights as a linear layer stores them ([L, I, H] gate/up) or in the math form "
                         "([L, H, I] gate/up, [L, I, H] down)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--route-groups", type=int, nargs=2, default=None, metavar=("G", "M"),
                    help="group-limited routing: E experts in G contiguous groups, at most M per token")
    ap.add_argument("--balance-gamma", type=float, default=None, metavar="GAMMA",
                    help="route with a selection bias (zero at the start) and take one balancing step on it "
                         "per layer step, from that step's expert loads")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step of the layer: the forward that keeps its activations, "
                         "then the backward on a seeded upstream gradient")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the benchmark, time library copy kernels with the byte mix of dispatch_place "
                         "(read the token rows once, write each kept pair's row) and of combine (read the "
                         "pairs' rows, write the token rows) on this workload, buffers rotated past the "
                         "Infinity Cache; reported under copy_probe")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="after the benchmark, time the library's grouped FFN on one expert holding all the "
                         "pairs' rows and torch.matmul (hipBLASLt) on the same dense products; reported under "
                         "gemm_probe")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run one plain device copy of BYTES bytes (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              f"(the multi-GPU exchange is not part of this library)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import expert_token_dispatch_amd as etd
    from expert_token_dispatch_amd.layer import MoELayer, to_device

    s = synth.spec(args.workload, seed=args.seed, weight_layout=args.weight_layout)
    log(f"[bench] generating {s}")
    inp = synth.make_layer(s)
    desc = etd.make_desc(s.T, s.H, s.I, s.E, s.k, s.local_begin, s.L, s.capacity_factor, s.dtype, s.weight_layout)
    layer = MoELayer.from_host(desc, inp)
    x = to_device(inp["x"], s.dtype)
    y = torch.empty_like(x)
    counts = torch.empty((s.E,), dtype=torch.int32, device="cuda")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    dropped = torch.zeros((1,), dtype=torch.int64, device="cuda")

    # routing options (glossary "Load balancing and capacity"): a step is then the layer
    # forward with the options plus, with a bias, one balancing step on it
    opts, sel_bias, step_counts = None, None, None
    if args.route_groups is not None or args.balance_gamma is not None:
        if args.balance_gamma is not None:
            sel_bias = torch.zeros((s.E,), dtype=torch.float32, device="cuda")
            step_counts = torch.zeros((s.E,), dtype=torch.int32, device="cuda")
        G, M = args.route_groups if args.route_groups is not None else (0, 0)
        opts = etd.make_route_opts(sel_bias, G, M)

    # a step is a list of library calls; each call gets its own profiling event array
    if args.backward:
        dy = to_device(synth.make_upstream_grad(s), s.dtype)
        saved = etd.make_saved(layer.saved_buffers(x.dtype))
        grads = layer.grad_buffers(x.dtype)

    def calls(**kw):
        if step_counts is not None and "counts_out" not in kw:
            kw["counts_out"] = step_counts
        if args.backward:
            out = [lambda: layer.forward_train(x, opts=opts, saved=saved, y=y, **kw),
                   lambda: layer.backward(x, saved, dy, grads=grads)]
        else:
            out = [lambda: layer.forward(x, y=y, opts=opts, **kw)]
        if sel_bias is not None:  # the balancing step, never timed on its own
            out.append(lambda: layer.update_selection_bias(kw["counts_out"], sel_bias, args.balance_gamma))
        return out

    ncalls = len(calls()) - (1 if sel_bias is not None else 0)  # calls whose kernels are profiled
    names = []  # names[c]: the kernels of call c, in launch order

    def step(ev=None, capture_names=False, **kw):
        """ev: per profiled call, a list of hipEvent_t (or None)."""
        for c, fn in enumerate(calls(**kw)):
            etd.moe_profile_events(ev[c] if ev is not None and c < ncalls else None)
            fn()
            if capture_names and c < ncalls:
                names.append([etd.moe_profile_kernel_name(i) for i in range(etd.moe_profile_kernel_count())])
        etd.moe_profile_events(None)

    if args.copy_calibration > 0:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {n} bytes done")

    # one run to learn the routing (pairs kept, experts touched) for the work model
    if args.backward:
        step(capture_names=True, counts_out=counts, num_dropped_out=dropped)
        torch.cuda.synchronize()
        ids_h = saved._tensors["topk_ids"].cpu().numpy()
    else:
        step(capture_names=True, topk_ids_out=ids, counts_out=counts, num_dropped_out=dropped)
        torch.cuda.synchronize()
        ids_h = ids.cpu().numpy()
    cnt_h = counts.cpu().numpy()
    C = etd.moe_capacity(desc)
    local = cnt_h[s.local_begin:s.local_begin + s.L]
    kept = np.minimum(local, C) if C >= 0 else local
    P = int(kept.sum())
    touched_experts = int((kept > 0).sum())
    is_local = (ids_h >= s.local_begin) & (ids_h < s.local_begin + s.L)
    touched_tokens = int(np.any(is_local, axis=1).sum())  # upper bound when capacity cuts pairs
    nblk = -(-s.T * s.k // 1024)
    log(f"[bench] kernels {names}; P={P}, experts touched {touched_experts}, dropped {int(dropped.item())}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = HipEvents()

    def kernel_entry(n, us, count):
        b, f = kernel_work(n, s, P, touched_tokens, touched_experts, nblk, args.backward)
        b, f = b * count, f * count
        gbs = b / (us * 1e-6) / 1e9 if us > 0 else 0.0
        tfl = f / (us * 1e-6) / 1e12 if us > 0 else 0.0
        return {"us": round(us, 2), "GB/s": round(gbs, 1), "TFLOP/s": round(tfl, 2),
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                "mfma_frac": round(tfl / MFMA_PEAK_TFLOPS[s.dtype], 4) if f else None}

    # breakdown: a few more steps with every kernel between HIP events (each event pair
    # costs the stream a little time, so the timed steps below carry only one kernel's)
    nbd = max(3, min(args.steps, 10))
    evs = [[hip.create(2 * len(nc)) for nc in names] for _ in range(nbd)]
    for i in range(nbd):
        step(evs[i])
    torch.cuda.synchronize()
    per_kernel = {}
    for c, nc in enumerate(names):
        for j, n in enumerate(nc):
            ts = [hip.elapsed_ms(evs[i][c][2 * j], evs[i][c][2 * j + 1]) for i in range(nbd)]
            per_kernel.setdefault(n, []).append(sum(ts) / len(ts))
    for e in evs:
        for ec in e:
            hip.destroy(ec)
    # a name launched twice in a step adds up
    kern = {n: kernel_entry(n, sum(ts) * 1e3, len(ts)) for n, ts in per_kernel.items()}
    dom = max(kern, key=lambda n: kern[n]["us"])

    # timed steps: HIP events around the dominant kernel's launches only
    where = [(c, j) for c, nc in enumerate(names) for j, n in enumerate(nc) if n == dom]
    tev = []
    for _ in range(args.steps):
        h = [[None] * (2 * len(nc)) for nc in names]
        for c, j in where:
            h[c][2 * j], h[c][2 * j + 1] = hip.create(2)
        tev.append(h)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(tev[i])
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    dom_ms = sum(hip.elapsed_ms(h[c][2 * j], h[c][2 * j + 1]) for h in tev for c, j in where) / args.steps
    for h in tev:
        for hc in h:
            hip.destroy([e for e in hc if e is not None])
    kern[dom] = kernel_entry(dom, dom_ms * 1e3, len(where))

    # per-step durations (median and minimum), from K more steps each between two events
    # of its own, after the timed region
    cur = torch.cuda.current_stream().cuda_stream
    pev = [hip.create(2) for _ in range(args.steps)]
    for a_, b_ in pev:
        hip.record(a_, cur)
        step()
        hip.record(b_, cur)
    torch.cuda.synchronize()
    per_step = sorted(hip.elapsed_ms(a_, b_) for a_, b_ in pev)
    for e in pev:
        hip.destroy(e)
    step_median = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    step_min = per_step[0]

    b, f = kernel_work(dom, s, P, touched_tokens, touched_experts, nblk, args.backward)
    us = kern[dom]["us"]
    gemm_bound_hbm = dom.startswith("ffn") and (f / (MFMA_PEAK_TFLOPS[s.dtype] * 1e12) < b / (HBM_PEAK_GBS * 1e9))
    if f > 0 and not gemm_bound_hbm:
        achieved = f / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS[s.dtype],
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS[s.dtype], 4)}
    else:
        achieved = b / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    tb = traffic_for(dom, s.name, args.backward)
    roof["traffic"] = tb
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = f if roof["bound"] == "mfma" else b

    # grouped GEMM: all ffn kernels (plan and fixups included) against their flops
    gemm_us = sum(kern[n]["us"] for n in kern if n.startswith("ffn"))
    gemm_fl = sum(kernel_work(n, s, P, touched_tokens, touched_experts, nblk, args.backward)[1] * len(per_kernel[n])
                  for n in kern if n.startswith("ffn"))
    gemm_frac = gemm_fl / (gemm_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[s.dtype] if gemm_us else None
    stage = lambda pre: round(sum(kern[n]["us"] for n in kern if n.startswith(pre)), 2)  # noqa: E731

    out = {
        "metric": METRIC_TRAIN if args.backward else METRIC,
        "value": round(s.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(step_median, 4),
        "ms_per_step_min": round(step_min, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic (seeded numpy draws; random-init router and experts)",
        "config": {"workload": s.name, "tokens": s.T, "hidden": s.H, "intermediate": s.I, "experts": s.E,
                   "top_k": s.k, "local_experts": [s.local_begin, s.local_begin + s.L],
                   "capacity_factor": s.capacity_factor, "pairs_kept": P, "seed": s.seed,
                   "weight_layout": s.weight_layout,
                   **({"route_groups": args.route_groups} if args.route_groups else {}),
                   **({"balance_gamma": args.balance_gamma} if args.balance_gamma is not None else {})},
        "grouped_gemm_mfma_frac": round(gemm_frac, 4) if gemm_frac else None,
        "stages_us": {"route": stage("route"), "dispatch": stage("dispatch"), "grouped_ffn": stage("ffn"),
                      "combine": stage("combine")},
        **({"mode": "training step (forward keeping activations + backward)"} if args.backward else {}),
        "kernels": kern,
        "roofline": roof,
    }
    if args.copy_probe:
        out["copy_probe"] = copy_probe(s, P)
    if args.gemm_probe:
        out["gemm_probe"] = gemm_probe(s, P)
    out["routing"] = routing_report(inp, ids_h, cnt_h, int(dropped.item()), P, not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(inp, min(args.cpu_tokens, s.T), backward=args.backward)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
