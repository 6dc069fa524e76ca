"""GPU edge cases the pages name or the method implies: single tokens and
uneven slices (Transformers "With tensor parallelism": slices may be uneven or
empty, even in single-token decoding), experts that receive nothing, capacity
overflow with tied scores (glossary "Load balancing and capacity"), shapes off
the tile grid, and the decomposition identities over expert ranges and token
slices."""

import numpy as np
import pytest

import oracle
import synth
from tests._harness import layer_of, np_of, row_error, say, tol

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run(s, logits=None):
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    lg_in = None if logits is None else torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    g = layer.staged(x, logits_in=lg_in)
    torch.cuda.synchronize()
    gpu = {k: (np_of(v) if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    return inp, layer, x, gpu


def _check(s, inp, gpu, logits=None):
    ref = oracle.layer_forward(inp, logits=gpu["logits"] if logits is None else logits)
    np.testing.assert_array_equal(gpu["topk_ids"], ref["topk_ids"])
    np.testing.assert_array_equal(gpu["counts"], ref["counts"])
    np.testing.assert_array_equal(gpu["offsets"], ref["offsets"])
    P = int(ref["offsets"][-1])
    np.testing.assert_array_equal(gpu["sorted_pairs"][:P], ref["sorted_pairs"])
    np.testing.assert_array_equal(gpu["pair_row"], ref["pair_row"])
    assert int(gpu["num_dropped"][0]) == ref["num_dropped"]
    err = row_error(gpu["y"], ref["y"], s.dtype)
    assert err <= tol(s.dtype), err
    return ref


@pytest.mark.parametrize("over", [
    dict(T=1), dict(T=2, k=1), dict(T=3, k=8, E=8, L=8), dict(T=5, E=1, k=1, L=1),
    dict(T=130, H=72, I=40), dict(T=257, H=136, I=200, E=16, k=3, L=16),
    dict(T=300, E=32, k=4, local_begin=31, L=1), dict(T=300, E=32, k=4, local_begin=5, L=11),
])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_shapes(over, dtype):
    s = synth.spec("gptoss_ep8_share", H=64, I=96, E=8, k=2, local_begin=0, L=8, dtype=dtype,
                   bias="linear_default").replace(**over)
    say(f"[edge] {s}")
    inp, layer, x, gpu = _run(s)
    _check(s, inp, gpu)


def test_all_tokens_to_one_expert_and_empty_experts():
    s = synth.spec("gptoss_ep8_share", T=700, H=128, I=160, E=16, k=2, L=16)
    lg = np.full((s.T, s.E), -5.0, dtype=np.float32)
    lg[:, 3] = 2.0
    lg[:, 7] = 1.0 + np.arange(s.T, dtype=np.float32) * 1e-3
    inp, layer, x, gpu = _run(s, logits=lg)
    ref = _check(s, inp, gpu, logits=lg)
    assert ref["counts"][3] == s.T and ref["counts"][7] == s.T
    assert (ref["counts"] == 0).sum() == 14


@pytest.mark.parametrize("E,k", [(5, 5), (64, 8), (128, 1), (128, 32), (200, 4), (256, 17), (256, 32)],
                         ids=lambda v: str(v))
def test_top_k_on_tied_logits(E, k):
    # Top-k over given logits with many equal scores (rounded to 0.5): descending order,
    # equal scores to the lower expert id.  The expert counts cover 8 and 16 logits per
    # lane of the row kernel (E <= 128, <= 256, the most the router takes), k past 16 (two
    # entries per lane) and k = E.
    s = synth.spec("mixtral_like", T=130, H=64, I=64, E=E, k=k, L=E)
    rng = np.random.default_rng(E * 100 + k)
    lg = (np.round(rng.standard_normal((s.T, E)) * 2) / 2).astype(np.float32)
    lg[:3] = 1.5                                   # whole rows tied
    lg[3, ::7] = 9.0                               # a tie at the top across the row
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    r = layer.route(x, logits_in=torch.from_numpy(lg).cuda(), want_topk_logit=True)
    ref = oracle.route(None, None, None, k, logits=lg.astype(np.float64))
    say(f"[edges] top-k on tied logits E={E} k={k}")
    np.testing.assert_array_equal(np_of(r["topk_ids"]), ref["topk_ids"])
    np.testing.assert_array_equal(np_of(r["topk_logit"]), ref["topk_logit"].astype(np.float32))
    np.testing.assert_allclose(np_of(r["topk_w"]), ref["topk_w"], rtol=0, atol=2e-7)


def test_capacity_with_tied_scores():
    # expert 0 is everyone's first choice with the same score: the lower tokens win
    s = synth.spec("skewed_capacity", T=2000, H=64, I=64, E=8, k=2, L=8, capacity_factor=1.0)
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((s.T, s.E)).astype(np.float32)
    lg[:, 0] = 7.0
    lg[::3, 1] = 7.0       # ties across experts too: lower id first
    inp, layer, x, gpu = _run(s, logits=lg)
    ref = _check(s, inp, gpu, logits=lg)
    C = oracle.capacity_limit(1.0, s.T, s.k, s.E)
    kept0 = [p // s.k for p in ref["sorted_pairs"][ref["offsets"][0]:ref["offsets"][1]]]
    assert kept0 == list(range(C))
    assert ref["num_dropped"] > 0


def test_capacity_drops_everything_for_some_tokens():
    s = synth.spec("skewed_capacity", T=1024, H=64, I=64, E=8, k=1, L=8, capacity_factor=0.5)
    lg = np.zeros((s.T, s.E), dtype=np.float32)
    lg[:, 2] = np.linspace(0, 1, s.T, dtype=np.float32)[::-1] + 1
    inp, layer, x, gpu = _run(s, logits=lg)
    ref = _check(s, inp, gpu, logits=lg)
    C = oracle.capacity_limit(0.5, s.T, 1, s.E)
    assert ref["num_dropped"] == s.T - C
    assert np.all(gpu["y"][C:] == 0)


@pytest.mark.parametrize("case", ["max_segment", "ragged_clustered", "many_slices"])
def test_capacity_cut_large_segments(case):
    # The capacity cut keeps a segment's keys 32 per thread of a 1024-thread block and
    # ranks them in slices of 4096 rows, one block per slice: a segment of the most
    # tokens a call takes (32768, every register full, no padding, eight slices),
    # segments of several thousand keys that are not multiples of 1024 (padding rows)
    # whose logits share a handful of values (many keys per radix digit, ties ranked by
    # token across slice edges), and a local range past expert 0 with hot experts of
    # 2 to 5 slices, experts within capacity and one that receives nothing between them.
    if case == "many_slices":
        s = synth.spec("skewed_capacity", T=20000, H=64, I=64, E=16, k=3, local_begin=2, L=12,
                       capacity_factor=1.0)
        rng = np.random.default_rng(13)
        lg = rng.standard_normal((s.T, s.E)).astype(np.float32)
        lg[:, 5] = -50.0                                   # local expert 3 (id 5) gets nothing
        lg[:, 3] += 2.5                                    # hot: in most tokens' top 3
        lg[:, 7] += 1.5
        lg[: s.T // 2, 9] = np.round(lg[: s.T // 2, 9] * 2) / 2 + 3.0  # ties, half the tokens
        lg[:, 13] = np.where(np.arange(s.T) % 7 < 3, 4.0, lg[:, 13])   # one tied score, 3/7 of tokens
    elif case == "max_segment":
        s = synth.spec("skewed_capacity", T=32768, H=64, I=64, E=8, k=1, L=8, capacity_factor=0.5)
        rng = np.random.default_rng(11)
        lg = np.zeros((s.T, s.E), dtype=np.float32)
        lg[:, 0] = rng.choice(np.array([1.0, 1.5, 2.0], dtype=np.float32), size=s.T)
    else:
        s = synth.spec("skewed_capacity", T=9001, H=64, I=64, E=4, k=2, L=4, capacity_factor=0.9)
        rng = np.random.default_rng(12)
        lg = (3.0 + 1e-3 * np.round(rng.standard_normal((s.T, s.E)) * 3)).astype(np.float32)
        lg[:, 1] += 0.5   # expert 1 in nearly every token's top 2
    say(f"[edge] capacity cut {case}: {s}")
    inp, layer, x, gpu = _run(s, logits=lg)
    ref = _check(s, inp, gpu, logits=lg)
    C = oracle.capacity_limit(s.capacity_factor, s.T, s.k, s.E)
    assert int(np.max(ref["counts"])) > C and ref["num_dropped"] > 0


def test_zero_capacity_drops_every_pair():
    # a capacity factor so small that C = floor(cf * T * k / E) = 0: every pair is cut
    # and every output row is zero
    s = synth.spec("skewed_capacity", T=1000, H=64, I=64, E=8, k=2, L=8, capacity_factor=0.001)
    assert oracle.capacity_limit(s.capacity_factor, s.T, s.k, s.E) == 0
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    y = np_of(layer.forward(x))
    ref = oracle.layer_forward(inp)
    assert ref["num_dropped"] == s.T * s.k
    assert np.all(y == 0) and np.all(ref["y"] == 0)


@pytest.mark.parametrize("E,L,begin,cf,T", [(2048, 2048, 0, 0.0, 3000), (4096, 1500, 100, 0.0, 3000),
                                             (4096, 3000, 1000, 2.0, 3000), (4096, 2000, 50, 40.0, 16384)],
                         ids=lambda v: str(v))
def test_dispatch_with_thousands_of_experts(E, L, begin, cf, T):
    # Dispatch on given top-k ids with more experts than the router takes (up to the 4096
    # the descriptor allows, up to 3000 local): the chunk histogram table is past the
    # size the place and scatter kernels sum themselves, so the scan runs as its own
    # launch over column groups of 1024 experts (and writes the capacity slice table);
    # with a capacity factor, the cut runs over segments of a few pairs, and with 16384
    # tokens the crowded expert's ~5460 pairs span two 4096-row slices with equal scores
    # across the slice edge.
    s = synth.spec("gptoss_ep8_share", T=T, H=64, I=32, E=E, k=4, local_begin=begin, L=L, capacity_factor=cf)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    rng = np.random.default_rng(E + L)
    ids = np.argsort(rng.random((s.T, E)), axis=1)[:, : s.k].astype(np.int32)   # k distinct experts per token
    crowd = (np.arange(s.T) < s.T // 3) & ~(ids[:, 1:] == begin + 7).any(axis=1)
    ids[crowd, 0] = begin + 7                                                     # one crowded local expert
    lgt = np.round(rng.standard_normal((s.T, s.k)) * 4).astype(np.float32) / 4   # many equal scores
    say(f"[edge] dispatch E={E} L={L} begin={begin} cf={cf}")
    g = layer.dispatch(x, torch.from_numpy(ids).cuda(), torch.from_numpy(lgt).cuda() if cf > 0 else None)
    torch.cuda.synchronize()
    d = oracle.dispatch(ids.astype(np.int64), lgt.astype(np.float64), E, begin, L, cf)
    np.testing.assert_array_equal(np_of(g["counts"]), d["counts"])
    np.testing.assert_array_equal(np_of(g["offsets"]), d["offsets"])
    P = int(d["offsets"][-1])
    np.testing.assert_array_equal(np_of(g["sorted_pairs"])[:P], d["sorted_pairs"])
    np.testing.assert_array_equal(np_of(g["pair_row"]), d["pair_row"])
    assert int(np_of(g["num_dropped"])[0]) == d["num_dropped"]
    np.testing.assert_array_equal(np_of(g["x_sorted"])[:P], np_of(x)[d["sorted_pairs"] // s.k])
    if cf > 0:
        assert d["num_dropped"] > 0
    if T > 3000:
        assert d["counts"][begin + 7] > 4096 > oracle.capacity_limit(cf, s.T, s.k, s.E)


@pytest.mark.parametrize("H,I", [(128, 512), (512, 128)], ids=["gate_up_128", "down_128"])
def test_float32_layer_on_128_tiles(H, I):
    # A float32 layer whose 64 x 64 tiles would fill the CUs unevenly takes 128 x 128
    # tiles (six-slot ring) for the product with 512 output columns: gate/up for
    # H=128, I=512; down for H=512, I=128 (the tile picker's cost: rounds of 256 CUs x
    # tile area, 64 x 64 only when 10% cheaper).
    s = synth.spec("tiny_fp32", T=3000, H=H, I=I, E=8, k=2, L=8)
    say(f"[edge] float32 128x128 tiles: {s}")
    inp, layer, x, gpu = _run(s)
    _check(s, inp, gpu)


def test_expert_ranges_sum_to_all_local():
    base = synth.spec("gptoss_ep8_share", T=512, H=128, I=96, E=16, k=4, L=16, dtype="f32", bias="none")
    inp = synth.make_layer(base)
    layer, x = layer_of(inp)
    full = np_of(layer.forward(x))
    for ep in (2, 4):
        acc = np.zeros_like(full, dtype=np.float64)
        for rank in range(ep):
            b, n = oracle.ep_local_range(16, ep, rank)
            part = dict(inp)
            part["spec"] = base.replace(local_begin=b, L=n)
            for w in ("w_gate", "w_up", "w_down"):
                part[w] = inp[w][b:b + n]
            pl, px = layer_of(part)
            acc += np_of(pl.forward(px))
        assert row_error(acc, full.astype(np.float64), "f32") <= 1e-5


def test_token_slices_concatenate_bit_exact():
    s = synth.spec("mixtral_like", T=900, H=256, I=384)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    full = np_of(layer.forward(x))
    parts = []
    for a, b in [(0, 1), (1, 450), (450, 451), (451, 900)]:
        sub = dict(inp)
        sub["spec"] = s.replace(T=b - a)
        sub["x"] = inp["x"][a:b]
        pl, px = layer_of(sub)
        parts.append(np_of(pl.forward(px)))
    np.testing.assert_array_equal(np.concatenate(parts), full)


def test_zero_tokens_leave_outputs_untouched():
    s = synth.spec("mixtral_like", T=0, H=64, I=64)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    y = torch.full((0, s.H), 1.0, dtype=torch.bfloat16, device="cuda")
    layer.forward(x, y=y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("H,I", [(512, 8192), (8192, 512)], ids=["long-I-down", "long-H-gate-up"])
def test_long_k_split_tiles(H, I):
    # K of 8192 or more (128 steps of 64) lets the large-tile kernel cut each XCD's
    # partly filled last round along K; with this few tiles every XCD has one or two
    # tiles left over, so every tile goes through the pieces and the fixup pass
    s = synth.spec("mixtral_like", T=300, H=H, I=I, E=4, L=4)
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    g = layer.staged(x)
    torch.cuda.synchronize()
    offs = np_of(g["offsets"]).astype(np.int64)
    P = int(offs[-1])
    xs = np_of(g["x_sorted"])[:P].astype(np.float64)
    view = oracle.moe_oracle._ExpertView
    ref = oracle.grouped_ffn(xs, offs, view(inp["w_gate"], s.dtype), view(inp["w_up"], s.dtype),
                             view(inp["w_down"], s.dtype))
    got = np_of(g["y_sorted"])[:P]
    err = row_error(got, ref, s.dtype)
    say(f"[parity] long K H={H} I={I}: grouped FFN row error {err:.3g}")
    assert err <= tol(s.dtype)
    # the same call again gives the same bits (the pieces are added in a fixed order)
    y2 = np_of(layer.grouped_ffn(g["x_sorted"], g["offsets"]))[:P]
    np.testing.assert_array_equal(y2, got)


def test_segment_tails_on_the_large_tile_path():
    # hand-made segments whose tails take every tile shape of the large-tile kernel:
    # 257 rows (full tile + 1-row wide tail), 128 (a wide tile alone), 129 (regular tail),
    # 0 (empty), 256 (exactly one full tile) and 384 (full + 128-row wide tail); I = 448 and
    # H = 320 leave the last n-tile of both products partly past N
    s = synth.spec("mixtral_like", T=600, H=320, I=448, E=6, L=6)
    inp = synth.make_layer(s)
    layer, _ = layer_of(inp)
    counts = np.array([257, 128, 129, 0, 256, 384])
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = int(offs[-1])
    assert layer.max_pairs >= P and layer.max_pairs >= 128 * s.L
    rng = np.random.default_rng(7)
    xs = np.zeros((layer.max_pairs, s.H), dtype=np.float32)
    xs[:P] = rng.standard_normal((P, s.H)).astype(np.float32)
    xs_bits = synth.f32_to_bf16_bits(xs)
    x_dev = torch.from_numpy(xs_bits.view(np.int16)).cuda().view(torch.bfloat16)
    y = np_of(layer.grouped_ffn(x_dev, torch.from_numpy(offs).cuda()))[:P]
    view = oracle.moe_oracle._ExpertView
    x64 = np_of(x_dev)[:P].astype(np.float64)
    ref = oracle.grouped_ffn(x64, offs.astype(np.int64), view(inp["w_gate"], s.dtype), view(inp["w_up"], s.dtype),
                             view(inp["w_down"], s.dtype))
    err = row_error(y, ref, s.dtype)
    say(f"[parity] segment tails 257/128/129/0/256/384: grouped FFN row error {err:.3g}")
    assert err <= tol(s.dtype)


@pytest.mark.parametrize("over", [dict(T=16256, H=128, I=128, E=4, k=2, L=4), dict(T=4096, H=512, I=256, E=8, k=2, L=8),
                                  dict(T=300, H=136, I=200, E=8, k=2, L=8)],
                         ids=["ring-128x128-tiles", "ring-64x64-tiles", "general-off-grid"])
def test_fp32_tile_shapes(over):
    # the float32 grouped GEMM's tile shapes: 128 x 128 tiles when they fill the CUs in
    # whole rounds (32512 pairs over 4 experts, N = 128), 64 x 64 tiles for the tiny
    # layer's shape, and the general kernel for k off the 16-element grid
    s = synth.spec("tiny_fp32").replace(**over)
    say(f"[edge] float32 {s}")
    inp, layer, x, gpu = _run(s)
    _check(s, inp, gpu)
