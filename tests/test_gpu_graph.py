"""The one-call layer captured in a HIP graph and replayed.

moe_layer_forward enqueues kernels only (no allocation, copy, memset or host
synchronization), so a caller can capture it.  Each replay here follows eager
work on other buffers, a sentinel fill of every output and a device
synchronization, and must reproduce the eager call bit for bit."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_08_amd import inputs as minp
from mixture_experts_ffn_08_amd.inputs import SOFTMAX_THEN_TOPK as SM_TK, TOPK_THEN_SOFTMAX as TK_SM
from mixture_experts_ffn_08_amd.layer import Buffers, DeviceWeights, MoeLayer, to_device
from support import host, log

pytestmark = pytest.mark.gpu

S = minp.LayerShape
CASES = [
    # decode batch: one-block selection, dispatch and statistics; skewed router, so the expert
    # GEMMs' tiled launch for groups of more than 16 rows has work
    S("graph_decode_zipf", "bf16", 64, 256, 128, 8, 128, 0, SM_TK, True, None, True),
    # many tokens: router blocks write the dispatch histograms and the statistics' partial sums
    S("graph_prefill_hist", "bf16", 4133, 256, 128, 8, 128, 0, SM_TK, True, None, False),
    # separate route and permute launches, capacity dropping, shared expert
    S("graph_shared_capacity", "bf16", 300, 256, 16, 4, 256, 512, TK_SM, False, 1.0, False),
]

_FLOAT = ("logits", "topk_w", "a", "y_perm", "y", "f", "P", "l_aux", "max_over_mean", "shared_y")
_INT = ("topk_idx", "near_tie", "counts", "offsets", "row_of", "perm_token")


def _outputs(b):
    return {name: getattr(b, name) for name in _FLOAT + _INT if getattr(b, name, None) is not None}


def _snapshot(b, R):
    out = {name: host(t) for name, t in _outputs(b).items()}
    for name in ("perm_token", "a", "y_perm"):
        out[name] = out[name][:R]
    return out


@pytest.mark.parametrize("shape", CASES, ids=lambda s: s.name)
def test_graph_replay_matches_eager(shape):
    inp = minp.LayerInputs(shape, seed=8)
    layer = MoeLayer(DeviceWeights(inp, "cuda"))
    x = to_device(inp.x, shape.dtype, "cuda")
    b = Buffers(shape, shape.T, "cuda")
    other = Buffers(shape, shape.T, "cuda")
    layer.forward(x, b)
    torch.cuda.synchronize()
    R = int(host(b.offsets)[-1])
    ref = _snapshot(b, R)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, b)  # the capture stream's first call outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        layer.forward(x, b)
    torch.cuda.synchronize()

    for rep in range(4):
        for name, t in _outputs(b).items():
            t.fill_(float("nan") if name in _FLOAT else -7)
        layer.forward(x, other)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(b, R)
        for name in ref:
            assert np.array_equal(got[name], ref[name]), (rep, name)
    eager = _snapshot(other, R)
    for name in ref:
        assert np.array_equal(eager[name], ref[name]), name
    log(f"[{shape.name}] 4 graph replays bit-identical to the eager call")
