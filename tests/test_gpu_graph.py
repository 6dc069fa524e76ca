"""The layer forward captured in a HIP graph (torch.cuda.graph over the library's
launches on the current stream) and replayed: every replay must equal the eager
forward bit for bit, with eager work and synchronisations between the replays.

The library launches no memset or copy and allocates nothing inside a forward
that is given its workspace, so a captured step is the same kernels with the
launch gaps removed (bench.py reports it as ms_per_step_graph).  Scaled copies of
the workloads cover the fused place path, the capacity path (scan, scatter,
capacity cut, gather) and the float32 kernels.
"""

import numpy as np
import pytest

import synth
from tests._harness import layer_of, np_of, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    "mixtral-small": synth.spec("mixtral_like", T=512, H=256, I=512, E=8, k=2, L=8),
    "gptoss-share-small": synth.spec("gptoss_ep8_share", T=600, H=320, I=320, E=32, k=4, local_begin=8, L=8),
    "skewed-capacity-small": synth.spec("skewed_capacity", T=700, H=256, I=192, E=16, k=3, L=16),
    "tiny-f32": synth.spec("tiny_fp32", T=300),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_matches_eager(name):
    s = CASES[name]
    say(f"[graph] {name}: {s}")
    inp = synth.make_layer(s)
    layer, x = layer_of(inp)
    y_eager = layer.forward(x)
    torch.cuda.synchronize()
    ref = np_of(y_eager)

    y_g = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, y=y_g)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x, y=y_g)
    torch.cuda.synchronize()

    other = torch.empty_like(x)
    for r in range(3):
        y_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np_of(y_g), ref, err_msg=f"replay {r}")
        # eager work between replays: a forward of its own and a reduction
        layer.forward(x, y=other)
        _ = float(other.float().abs().sum().item())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np_of(other), ref)
    say(f"[graph]   three replays equal to the eager forward")
