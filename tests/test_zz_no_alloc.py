"""moe_forward_noalloc (the entry point that allocates nothing: its scratch is
the library's static device array) against moe_forward on the same inputs:
two calls in a row, the second on a smaller layer, each bitwise equal to
moe_forward's y, aux, counts and z-loss; and the first layer's result again
after the second call reused the array."""
import numpy as np
import pytest
import torch

import gpu_harness as H
import sparse_mixture_experts_48_amd as moe
from sparse_mixture_experts_48_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the CPU suite deselects these
    pytest.skip("needs a GPU", allow_module_level=True)

L = W.LayerShape
FIRST = L("noalloc_big", 600, 512, 16, 2, 1032, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "normal2", 71)
SECOND = L("noalloc_small", 40, 256, 8, 1, 264, W.ACT_GELU, W.GATE_RAW, W.DT_BF16, "zipf1.1", 72)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _pair(cfg, dev, noise):
    desc = moe.desc_of(cfg)
    assert moe.workspace_size(desc) <= moe.binding.NOALLOC_SCRATCH_BYTES
    y = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device="cuda")
    aux = torch.empty(1, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    z = torch.empty(1, device="cuda")
    moe.forward_noalloc(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"], dev["W2"], dev["b2"],
                        y, aux=aux, counts=counts, noise=noise, z_loss=z)
    z_ref = torch.empty(1, device="cuda")
    y_ref, aux_ref, counts_ref = moe.forward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"],
                                             dev["W2"], dev["b2"], noise=noise, z_loss=z_ref)
    torch.cuda.synchronize()
    return (y, aux, counts, z), (y_ref, aux_ref, counts_ref, z_ref)


def _same(got, want, what):
    for g, w, name in zip(got, want, ("y", "aux", "counts", "z_loss")):
        assert torch.equal(_bits(g), _bits(w)), "%s: %s differs from moe_forward" % (what, name)


def test_noalloc_matches_forward_twice():
    H.say("[gpu] moe_forward_noalloc: %s then %s" % (FIRST, SECOND))
    inp1 = H.to_dev(W.make_inputs(FIRST))
    noise1 = torch.from_numpy((np.random.default_rng(3).standard_normal((FIRST.T, FIRST.E)) * 0.3)
                              .astype(np.float32)).cuda()
    got1, want1 = _pair(FIRST, inp1, noise1)
    _same(got1, want1, "first call")
    inp2 = H.to_dev(W.make_inputs(SECOND))
    got2, want2 = _pair(SECOND, inp2, None)
    _same(got2, want2, "second (smaller) call")
    # the first layer again, after the smaller call left its own contents in the array
    again, _ = _pair(FIRST, inp1, noise1)
    _same(again, want1, "first layer after the second call")
