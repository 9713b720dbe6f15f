"""moe_forward captured in a HIP graph: every replay equals the eager result bit for bit.

Replays are interleaved with eager calls of the same layer on other inputs and
with host synchronizations, as a graph is used in a real serving loop.
"""
import pytest
import torch

import gpu_harness as H
import sparse_mixture_experts_48_amd as moe
from sparse_mixture_experts_48_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("cfg", [
    W.LayerShape("graph_decode", 16, 512, 8, 2, 1376, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 41),
    W.LayerShape("graph_prefill", 600, 256, 8, 2, 384, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 42),
    W.LayerShape("graph_switch", 300, 256, 16, 1, 344, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16, "zipf1.1", 43),
    W.LayerShape("graph_f32", 200, 128, 8, 2, 256, W.ACT_GELU, W.GATE_RENORM, W.DT_F32, "normal2", 44),
], ids=lambda c: c.name)
def test_graph_replays_match_eager(cfg):
    H.say("[gpu] graph case %s" % (cfg,))
    layer = moe.MoELayer(cfg, W.make_inputs(cfg))
    other = W.make_inputs(cfg, seed=cfg.seed + 100)["h"].cuda()
    y0, a0, c0 = (t.clone() for t in layer.forward())
    torch.cuda.synchronize()
    static_h = layer.p["h"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(static_h)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(static_h)
    for rep in range(4):
        layer.forward(other)          # eager work on other data between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(layer.y), _bits(y0)), "replay %d: y differs" % rep
        assert torch.equal(layer.aux, a0) and torch.equal(layer.counts, c0), "replay %d" % rep
