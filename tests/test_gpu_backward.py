"""Backward pass of the layer on the GPU (moe_backward) against the CPU
oracle's float64 backward, on the same seeded inputs and upstream gradient.

The oracle's backward is pinned on the CPU against central differences of the
float64 layer and against autograd of the dense E = 1 case. Routing is
recomputed bit for bit, so both sides differentiate the same choice.

Bar, per gradient tensor: |got - want|_2 <= 2e-2 |want|_2. Between the
bfloat16 inputs and any term the path rounds to bfloat16 up to five times
(the pre-activations, the hidden activation, dO, dZ, and for dh the output),
2^-9 relative each, so the typical element is off by well under 1 %; a
per-element bar does not suit gradients, whose elements are sums with
cancellation at several levels (a pre-activation near 0 makes its SiLU
gradient's relative error large). The router's bias gradient is judged per
element against the sum of its terms' magnitudes (which the oracle returns):
with renormalised gates a token's terms sum to zero over the experts, so the
whole vector is small next to its terms. That per-element figure is printed
for every gradient.
Float32 layers keep every intermediate in float32, so their bar is 1e-4
(per tensor, and per element of db_r against its terms): each gradient is a
chain of a few float32 sums over at most max(d, width, T) terms, whose
rounding (2^-24 per operation, growing like the square root of the terms)
stays near 1e-6 at these sizes.
Also: a second call gives the same bits, and with no tokens every gradient is
zero.
"""
import numpy as np
import pytest
import torch

import gpu_harness as H
import sparse_mixture_experts_48_amd as moe
from oracle import moe_oracle as O
from sparse_mixture_experts_48_amd import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the CPU suite deselects these
    pytest.skip("needs a GPU", allow_module_level=True)

L = W.LayerShape
TOL = 2e-2
TOL_F32 = 1e-4
CASES = {
    # name: (shape, daux, capacity, bias_mode)
    "swiglu_renorm": (L("bw_swiglu", 200, 128, 8, 2, 256, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "normal2", 81),
                      0.5, 0, 0),
    "gelu_raw_bias": (L("bw_gelu", 150, 64, 6, 2, 96, W.ACT_GELU, W.GATE_RAW, W.DT_BF16, "normal2", 82), 0.3, 0, 0),
    "switch_top1": (L("bw_switch", 300, 128, 16, 1, 128, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16, "zipf1.1", 83),
                    1.0, 0, 0),
    "capacity": (L("bw_cap", 120, 64, 8, 2, 128, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "normal2", 84), 0.0, 20,
                 0),
    "select_bias": (L("bw_sel", 96, 64, 8, 2, 64, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16, "normal2", 85), 0.2, 0, 1),
    "decode_T16": (L("bw_dec", 16, 256, 8, 2, 512, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 86), 0.1, 0, 0),
    "tiles_e4": (L("bw_tiles", 2048, 256, 4, 2, 512, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 87), 0.0, 0,
                 0),
    # shapes whose backward GEMMs run on the tiles of the full-size layers
    # (see TILES): the recompute and dZ GEMMs on 256 x 256 ...
    "tiles_256_swiglu": (L("bw_t256", 4096, 256, 4, 2, 4096, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 92),
                         0.25, 0, 0),
    # ... on 128 x 256 (about 100 rows per expert, top-1) ...
    "tiles_128x256_k1": (L("bw_t128x256", 1600, 128, 16, 1, 4608, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16, "zipf1.1",
                           93), 0.5, 0, 0),
    # ... and the dX GEMM on 256 x 256 (d = 4096)
    "tiles_256_dx_gelu": (L("bw_t256dx", 4096, 4096, 4, 2, 512, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16, "normal2", 94),
                          0.1, 0, 0),
    # ... and with a reduction of 2 width = 1024 (four stages per part), so that
    # the dX GEMM splits the experts' short tails along k
    "tiles_256_dx_split": (L("bw_t256split", 4096, 4096, 8, 2, 512, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none",
                             97), 0.2, 0, 0),
    # float32 layers: the micro workload itself (GELU with biases), SwiGLU with
    # raw gates and capacity drops, top-1 with a selection-only bias
    "f32_micro": (W.WORKLOADS["micro"], 0.5, 0, 0),
    "f32_swiglu_raw_cap": (L("bw_f32_sw", 300, 96, 6, 2, 160, W.ACT_SWIGLU, W.GATE_RAW, W.DT_F32, "normal2", 95),
                           0.3, 80, 0),
    "f32_top1_select": (L("bw_f32_k1", 200, 64, 16, 1, 128, W.ACT_GELU, W.GATE_RAW, W.DT_F32, "zipf1.1", 96), 1.0,
                        0, 1),
}

# Tile (rows x weight rows) each backward GEMM must run on, for the cases that
# are there to cover the larger tiles: (recompute, dZ, dX).
TILES = {
    "tiles_256_swiglu": ((256, 256), (256, 256), (128, 128)),
    "tiles_128x256_k1": ((128, 256), (128, 256), (128, 128)),
    "tiles_256_dx_gelu": ((128, 128), (128, 128), (256, 256)),
    "tiles_256_dx_split": ((128, 128), (128, 128), (256, 256)),
}


def test_dx_split_tails_case():
    """The tiles_256_dx_split case has experts whose last 256-row tile holds
    at most 64 rows, which the dX GEMM (reduction 2 width = 1024, at least 16
    stages) splits into four parts."""
    cfg = CASES["tiles_256_dx_split"][0]
    assert (2 * cfg.width + 63) // 64 >= 16
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    g = moe.route(moe.desc_of(cfg), dev["h"], dev["W_r"], dev["b_r"])
    counts = H.to_np(g["counts"]).astype(np.int64)
    assert ((counts % 256 > 0) & (counts % 256 <= 64)).any(), counts


def _tile(S, E, N, nmat):
    """The tile shape the library picks for a grouped GEMM of S rows over E
    experts and N output columns (nmat = 2 when W1 and W3 share a tile): 256 x
    256 with at least 512 rows per expert on average and two blocks per CU,
    else 128 x 256 with two blocks per CU, else 128 x 128."""
    def blocks(bm, bn):
        return ((S + bm - 1) // bm + min(E, S)) * ((N + bn // nmat - 1) // (bn // nmat))
    if S // max(E, 1) >= 512 and blocks(256, 256) >= 2 * 256:
        return (256, 256)
    if blocks(128, 256) >= 2 * 256:
        return (128, 256)
    return (128, 128)


def _backward_tiles(cfg):
    nmat = 2 if cfg.act == W.ACT_SWIGLU else 1
    return (_tile(cfg.S, cfg.E, cfg.width, nmat), _tile(cfg.S, cfg.E, cfg.width, 1),
            _tile(cfg.S, cfg.E, cfg.d, 1))


def _dy(cfg, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((cfg.T, cfg.d), generator=g).to(cfg.torch_dtype)


def _run(cfg, dev, dy, daux, cap, bias_mode):
    desc = moe.desc_of(cfg, capacity=cap, bias_mode=bias_mode)
    out = moe.backward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"], dev["W2"], dev["b2"],
                       dy, daux)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name):
    cfg, daux, cap, bias_mode = CASES[name]
    H.say("[gpu] backward %s %s daux=%g capacity=%d bias_mode=%d" % (name, cfg, daux, cap, bias_mode))
    if name in TILES:
        assert _backward_tiles(cfg) == TILES[name], (name, _backward_tiles(cfg))
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    dy = _dy(cfg, cfg.seed + 1000)
    out = _run(cfg, dev, dy.cuda(), daux, cap, bias_mode)
    again = _run(cfg, dev, dy.cuda(), daux, cap, bias_mode)
    for k, v in out.items():
        if v is not None:
            assert torch.equal(v.view(torch.int16) if v.dtype == torch.bfloat16 else v,
                               again[k].view(torch.int16) if v.dtype == torch.bfloat16 else again[k]), k
    ref = O.moe_backward(H.oracle_params(inp), cfg.T, cfg.d, cfg.E, cfg.K, cfg.act, cfg.gate,
                         W.as_float32(dy).astype(np.float64), daux=daux, capacity=cap if cap > 0 else None,
                         bias_select_only=bias_mode == 1, with_scales=True)
    bad = []
    for k in ("dh", "dW_r", "db_r", "dW1", "db1", "dW3", "dW2", "db2"):
        got, want = out[k], ref[k]
        if got is None or want is None:  # not requested, or a bias the layer does not have
            continue
        g = H.to_np(got).astype(np.float64)
        if k == "db_r" and bias_mode == 1:
            assert not g.any(), "a selection-only bias has no gradient"
            continue
        err = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-30))
        scale = ref["scale"][k]
        floor = 1e-6 * max(float(scale.max()), 1e-30)
        per_elem = float(np.max(np.abs(g - want) / np.maximum(scale, floor)))
        H.say("[gpu] %s %s: |d|/|ref| = %.5f (max |d|/sum|terms| %.4f, max|d|/rms %.4f)" % (
            name, k, err, per_elem, H.rel_err(g, want)))
        H.record("grad", "%s %s" % (name, k), rel=err, per_term=per_elem)
        tol = TOL if cfg.dtype == W.DT_BF16 else TOL_F32
        if (per_elem if k == "db_r" else err) > tol:
            bad.append((k, err, per_elem))
    assert not bad, bad


def test_backward_z_loss_and_noise():
    """loss = sum(dy y) + daux aux + dz z_loss with noise on the router logits
    (an input, held fixed): both router layouts, both bias modes."""
    for cfg, bias_mode, dz, cap in ((L("bw_znoise", 160, 128, 8, 2, 192, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16,
                                       "normal2", 89), 0, 0.7, 0),
                                    (L("bw_znoise_sel", 300, 64, 24, 2, 96, W.ACT_GELU, W.GATE_RAW, W.DT_BF16,
                                       "normal2", 90), 1, 2.0, 0),
                                    # everything at once: top-1 raw gates, drops, selection-only bias, noise, dz
                                    (L("bw_znoise_cap", 240, 64, 16, 1, 64, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                                       "zipf1.1", 91), 1, 1.3, 24)):
        H.say("[gpu] backward z-loss/noise %s bias_mode=%d dz=%g capacity=%d" % (cfg, bias_mode, dz, cap))
        inp = W.make_inputs(cfg)
        dev = H.to_dev(inp)
        dy = _dy(cfg, cfg.seed + 1000)
        noise = (np.random.default_rng(cfg.seed).standard_normal((cfg.T, cfg.E)) * 0.5).astype(np.float32)
        desc = moe.desc_of(cfg, capacity=cap, bias_mode=bias_mode)
        out = moe.backward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"], dev["W2"],
                           dev["b2"], dy.cuda(), 0.3, noise=torch.from_numpy(noise).cuda(), dz=dz)
        torch.cuda.synchronize()
        ref = O.moe_backward(H.oracle_params(inp), cfg.T, cfg.d, cfg.E, cfg.K, cfg.act, cfg.gate,
                             W.as_float32(dy).astype(np.float64), daux=0.3, capacity=cap if cap > 0 else None,
                             bias_select_only=bias_mode == 1, with_scales=True, noise=noise, dz_loss=dz)
        for k in ("dh", "dW_r", "db_r", "dW1", "db1", "dW3", "dW2", "db2"):
            got, want = out[k], ref[k]
            if got is None or want is None:
                continue
            g = H.to_np(got).astype(np.float64)
            if k == "db_r" and bias_mode == 1:
                assert not g.any()
                continue
            err = float(np.linalg.norm(g - want) / max(np.linalg.norm(want), 1e-30))
            scale = ref["scale"][k]
            per_elem = float(np.max(np.abs(g - want) / np.maximum(scale, 1e-6 * max(float(scale.max()), 1e-30))))
            H.say("[gpu] %s %s: |d|/|ref| = %.5f (max |d|/sum|terms| %.4f)" % (cfg.name, k, err, per_elem))
            H.record("grad", "%s %s" % (cfg.name, k), rel=err, per_term=per_elem)
            assert (per_elem if k == "db_r" else err) <= TOL, (k, err, per_elem)


def test_backward_no_tokens():
    cfg = CASES["gelu_raw_bias"][0]
    cfg0 = L("bw_empty", 0, cfg.d, cfg.E, cfg.K, cfg.width, cfg.act, cfg.gate, cfg.dtype, cfg.router_bias, 88)
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    desc = moe.desc_of(cfg0)
    out = moe.backward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"], dev["W2"],
                       dev["b2"], torch.empty((0, cfg.d), dtype=torch.bfloat16, device="cuda"), 0.5)
    torch.cuda.synchronize()
    for k, v in out.items():
        if v is not None and k != "dh":
            assert not v.any(), k
