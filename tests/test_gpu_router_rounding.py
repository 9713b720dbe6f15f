"""Router logits on inputs where any other rounding shows: bit for bit against the oracle.

The logits are four float32 fmaf chains per (token, expert) over the groups of four
consecutive k dealt round-robin to the chains, then (c0 + c1) + (c2 + c3). For 17..64
experts the chains run on the float32 matrix cores, whose 32x32x2 MFMA applies its two
k as two correctly rounded fmas in k order; up to 16 experts they run as VALU fmaf. The
inputs below are built so that a product rounded before its add, a fused two-term sum,
another k order, or flushed denormals would change logit bits:

* "cancel": h near +-1 (values 1 + m 2^-7, exact in bfloat16) against weights 1 + m 2^-20
  of alternating sign, so every chain sums to a small remainder of large terms;
* "tiny": bfloat16 denormal h (m 2^-133) against weights of magnitude 1..2, so every
  product and partial sum is a float32 denormal;
* "wide": h ~ N(0, 1) against weights whose magnitudes span 2^-20 .. 2^20.

The whole layer's expert choice and counts must agree too (the oracle runs the layer).
"""
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
SHAPES = {
    "e64_bf16": L("rr_e64", 96, 200, 64, 2, 64, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 121),
    "e24_bf16_k1": L("rr_e24", 70, 256, 24, 1, 64, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16, "none", 122),
    "e64_f32": L("rr_e64f", 64, 136, 64, 2, 64, W.ACT_GELU, W.GATE_RENORM, W.DT_F32, "none", 123),
    "e12_bf16": L("rr_e12", 300, 200, 12, 2, 64, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16, "none", 124),
}


def _adversarial(cfg, family, seed):
    rng = np.random.default_rng(seed)
    T, d, E = cfg.T, cfg.d, cfg.E
    if family == "cancel":
        h = (1.0 + rng.integers(0, 16, (T, d)) * 2.0 ** -7) * rng.choice([-1.0, 1.0], (T, d))
        sign = np.where(np.arange(d)[:, None] % 2 == 0, 1.0, -1.0)
        w = sign * (1.0 + rng.integers(0, 4096, (d, E)) * 2.0 ** -20)
    elif family == "tiny":
        h = rng.integers(1, 128, (T, d)) * 2.0 ** -133 * rng.choice([-1.0, 1.0], (T, d))
        w = rng.uniform(1.0, 2.0, (d, E)) * rng.choice([-1.0, 1.0], (d, E))
    else:
        h = rng.standard_normal((T, d))
        w = rng.standard_normal((d, E)) * 2.0 ** rng.integers(-20, 21, (d, E))
    h32 = torch.from_numpy(h.astype(np.float32))
    hin = h32.to(torch.bfloat16) if cfg.dtype == W.DT_BF16 else h32
    if cfg.dtype == W.DT_BF16:  # the constructions above are exact in bfloat16 (except "wide", rounded here)
        assert family == "wide" or torch.equal(hin.float(), h32)
    return hin.contiguous(), torch.from_numpy(w.astype(np.float32)).contiguous()


@pytest.mark.parametrize("family", ["cancel", "tiny", "wide"])
@pytest.mark.parametrize("name", sorted(SHAPES))
def test_router_logits_bitwise(name, family):
    cfg = SHAPES[name]
    H.say("[gpu] router rounding %s %s %s" % (name, family, cfg))
    inp = W.make_inputs(cfg)
    inp["h"], inp["W_r"] = _adversarial(cfg, family, cfg.seed)
    inp["b_r"] = None
    r = H.run_oracle(cfg, inp)
    dev = H.to_dev(inp)
    desc = moe.desc_of(cfg)
    g = moe.route(desc, dev["h"], dev["W_r"], None, want_logits=True)
    torch.cuda.synchronize()
    H.check_logits_bits(H.to_np(g["logits"]), r["logits"])
    H.check_bits_equal("topk_idx", H.to_np(g["topk_idx"]), r["topk_idx"])
    H.check_bits_equal("expert_counts", H.to_np(g["counts"]), r["counts"])
