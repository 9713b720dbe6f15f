"""Parity of the HIP path (through the C-ABI) against the CPU oracle.

Bars: bit-exact expert choice, router logits, counts, offsets, grouping and
gathered rows; gates within 1e-6; P and aux within 1e-5 relative; the float32
expert outputs within max|d|/rms <= 1e-5 (float32 layers) or 2e-2 (bfloat16
layers); y within the same bars once each element's own output rounding (half
an ulp of the output dtype) is discounted; the combine stage within one
rounding of its float32 sum.

Small cases run the whole oracle and span several tiles with ragged tails;
the five full-size workloads compare every routing output, every grouped
expert row and every y row, element by element, in the same launch
configuration as the benchmark. Only the largest-operand test samples y rows
(its oracle would take minutes).
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
SMALL = {
    # name: shape (T, d, E, K, width, act, gate, dtype, router_bias, seed)
    "f32_gelu_ragged": L("f32_gelu_ragged", 300, 128, 8, 2, 512, W.ACT_GELU, W.GATE_RENORM, W.DT_F32, "none", 11),
    "f32_swiglu_k1_fused": L("f32_swiglu_k1_fused", 201, 64, 4, 1, 200, W.ACT_SWIGLU, W.GATE_RAW, W.DT_F32,
                             "normal2", 12),
    "f32_swiglu_k2": L("f32_swiglu_k2", 97, 72, 6, 2, 136, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_F32, "none", 24),
    "bf16_gelu_skewed_e64": L("bf16_gelu_skewed_e64", 700, 128, 64, 2, 512, W.ACT_GELU, W.GATE_RENORM,
                              W.DT_BF16, "normal2", 13),
    "bf16_swiglu_tails": L("bf16_swiglu_tails", 333, 256, 8, 2, 680, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16,
                           "none", 14),
    "bf16_switch_k1": L("bf16_switch_k1", 517, 512, 16, 1, 344, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                        "zipf1.1", 15),
    "bf16_k3_e12": L("bf16_k3_e12", 150, 192, 12, 3, 256, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16, "normal2", 16),
    "bf16_k_equals_e": L("bf16_k_equals_e", 100, 128, 4, 4, 128, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16,
                         "none", 17),
    "bf16_e1_k1": L("bf16_e1_k1", 64, 128, 1, 1, 256, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16, "none", 18),
    "bf16_raw_k2_e40": L("bf16_raw_k2_e40", 260, 136, 40, 2, 264, W.ACT_GELU, W.GATE_RAW, W.DT_BF16,
                         "normal2", 19),
    "bf16_many_tiles": L("bf16_many_tiles", 2048, 256, 8, 2, 384, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16,
                         "none", 25),
    "stream_T16": L("stream_T16", 16, 512, 8, 2, 1376, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 20),
    "stream_T32_tails": L("stream_T32_tails", 32, 264, 8, 2, 520, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16,
                          "none", 21),
    "stream_T5_k1_e64": L("stream_T5_k1_e64", 5, 256, 64, 1, 128, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                          "zipf1.1", 22),
    "stream_gelu_T24": L("stream_gelu_T24", 24, 128, 8, 2, 512, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16,
                         "normal2", 23),
    # both reductions shorter than one 64-k stage of the tiled kernel
    "bf16_short_k": L("bf16_short_k", 300, 40, 4, 2, 48, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16, "normal2", 28),
    "T1": L("T1", 1, 128, 8, 2, 256, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 26),
    "f32_T1": L("f32_T1", 1, 64, 8, 2, 64, W.ACT_GELU, W.GATE_RENORM, W.DT_F32, "normal2", 27),
    # router layouts over 17..64 experts with float32 h, expert counts that are
    # not a multiple of 4 (W_r rows then start off 16-byte boundaries) and d = 8
    # mod 16 (a last round of k that only two of the four chains reach)
    "f32_e37_k2_d136": L("f32_e37_k2_d136", 300, 136, 37, 2, 200, W.ACT_GELU, W.GATE_RENORM, W.DT_F32,
                         "normal2", 34),
    "f32_e20_k1_d72": L("f32_e20_k1_d72", 150, 72, 20, 1, 64, W.ACT_SWIGLU, W.GATE_RAW, W.DT_F32, "zipf1.1", 35),
    "bf16_e57_k2_d200": L("bf16_e57_k2_d200", 260, 200, 57, 2, 128, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16,
                          "normal2", 36),
    # ragged groups of small mean size with long reductions: many one-tile
    # experts beside a few many-tile ones
    "ragged_switch_k1": L("ragged_switch_k1", 600, 1024, 16, 1, 1024, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                         "zipf1.1", 41),
    "ragged_gelu_k2": L("ragged_gelu_k2", 300, 1024, 32, 2, 1032, W.ACT_GELU, W.GATE_RENORM, W.DT_BF16,
                       "zipf1.1", 42),
    # K = 1 over 64 experts, 13 of them hit, on 128 x 256 tiles: the gated
    # scatter into y from a grid far smaller than the chip
    "ragged_fused_k1": L("ragged_fused_k1", 400, 2048, 64, 1, 520, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                         "zipf1.1", 60),
    # many experts with large matrices and Zipf-ragged groups (17 or 21 with
    # 1..32 rows beside 6 or 8 with hundreds): one tiled launch, in which the
    # weight-bound tiles of the small experts run beside the large experts'
    # compute-bound tiles; top-1 with the gated scatter, and top-2 GELU with biases
    "ragged_large_k1": L("ragged_large_k1", 2048, 2048, 32, 1, 1024, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                         "zipf1.1", 61),
    "ragged_large_gelu_k2": L("ragged_large_gelu_k2", 1024, 2048, 32, 2, 1024, W.ACT_GELU, W.GATE_RENORM,
                              W.DT_BF16, "zipf1.1", 62),
}


def _case(cfg, zero_router=False):
    inp = W.make_inputs(cfg)
    if zero_router:  # every logit ties: experts 0..K-1 take every token
        inp["W_r"] = torch.zeros_like(inp["W_r"])
        inp["b_r"] = None
    return inp


def _check_route(cfg, dev, r):
    desc = moe.desc_of(cfg)
    g = moe.route(desc, dev["h"], dev["W_r"], dev["b_r"], want_logits=True)
    torch.cuda.synchronize()
    H.check_logits_bits(H.to_np(g["logits"]), r["logits"])
    H.check_bits_equal("topk_idx", H.to_np(g["topk_idx"]), r["topk_idx"])
    H.check_bits_equal("expert_counts", H.to_np(g["counts"]), r["counts"])
    gate_err = float(np.max(np.abs(H.to_np(g["topk_gate"]) - r["topk_gate"]))) if cfg.T else 0.0
    assert gate_err <= H.GATE_ATOL, gate_err
    P = r["probs"].mean(axis=0) if cfg.T else np.zeros(cfg.E)
    assert np.max(np.abs(H.to_np(g["prob_mean"]) - P)) <= H.PROB_RTOL * max(P.max(), 1e-30) + 1e-7
    aux = float(H.to_np(g["aux"])[0])
    assert abs(aux - r["aux"]) <= H.AUX_RTOL * max(abs(r["aux"]), 1.0), (aux, r["aux"])


def _check_permute(cfg, dev, r):
    desc = moe.desc_of(cfg)
    idx = torch.from_numpy(r["topk_idx"]).cuda()
    g = moe.permute(desc, idx, dev["h"])
    torch.cuda.synchronize()
    H.check_bits_equal("expert_offsets", H.to_np(g["offsets"]), r["offsets"])
    H.check_bits_equal("slot_token", H.to_np(g["slot_token"]), r["slot_token"])
    H.check_bits_equal("token_slot", H.to_np(g["token_slot"]), r["token_slot"])
    want = dev["h"][torch.from_numpy(r["slot_token"].astype(np.int64)).cuda()]
    assert torch.equal(g["h_perm"].view(torch.int16) if want.dtype == torch.bfloat16 else g["h_perm"],
                       want.view(torch.int16) if want.dtype == torch.bfloat16 else want), "h_perm rows differ"


def _check_expert_ffn(cfg, inp, dev, r, slots=None, full=False):
    desc = moe.desc_of(cfg)
    h_perm = dev["h"][torch.from_numpy(r["slot_token"].astype(np.int64)).cuda()].contiguous()
    offs = torch.from_numpy(r["offsets"]).cuda()
    o = moe.expert_ffn(desc, h_perm, offs, dev["W1"], dev["b1"], dev["W3"], dev["W2"], dev["b2"])
    torch.cuda.synchronize()
    o = H.to_np(o)
    p = H.oracle_params(inp)
    slots = np.arange(cfg.S) if slots is None else np.asarray(slots)
    ref = np.zeros((len(slots), cfg.d))
    got = o[slots]
    expert_of_slot = np.searchsorted(r["offsets"], slots, side="right") - 1
    for e in np.unique(expert_of_slot):
        sel = np.nonzero(expert_of_slot == e)[0]
        x = p["h"][r["slot_token"][slots[sel]]]
        ref[sel] = O.expert_ffn(x, int(e), p, cfg.act)
    err = H.rel_err(got, ref)
    H.record("o", cfg.name, full=full, slots=len(slots), err=err, bar=H.Y_TOL[cfg.dtype])
    assert err <= H.Y_TOL[cfg.dtype], err


def _check_combine(cfg, r):
    desc = moe.desc_of(cfg)
    # feed float32-rounded oracle expert outputs and gates; compare against the
    # oracle combine of exactly those float32 values
    rng = np.random.default_rng(cfg.seed)
    o32 = rng.standard_normal((cfg.S, cfg.d)).astype(np.float32)
    g32 = r["topk_gate"].astype(np.float32)
    y = moe.combine(desc, torch.from_numpy(o32).cuda(), torch.from_numpy(r["token_slot"]).cuda(),
                    torch.from_numpy(g32).cuda(), cfg.torch_dtype)
    torch.cuda.synchronize()
    ref = O.combine(o32.astype(np.float64), r["token_slot"], g32.astype(np.float64))
    # elementwise bound: K float32 fmas (each within 2^-24 of the running sum
    # of |g o|), then for bfloat16 one round-to-nearest (2^-8 relative)
    mag = O.combine(np.abs(o32.astype(np.float64)), r["token_slot"], np.abs(g32.astype(np.float64)))
    bound = (cfg.K + 1) * 2.0 ** -24 * mag
    if cfg.dtype == W.DT_BF16:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    diff = np.abs(H.to_np(y).astype(np.float64) - ref)
    worst = np.unravel_index(np.argmax(diff - bound), diff.shape)
    assert np.all(diff <= bound), ("combine outside one-rounding bound", worst, diff[worst], bound[worst])


def _check_forward(cfg, dev, r, rows=None, repeats=3, full=False):
    layer_desc = moe.desc_of(cfg)
    ws = moe.workspace(layer_desc)
    outs = []
    for _ in range(repeats):
        y, aux, counts = moe.forward(layer_desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"],
                                     dev["W3"], dev["W2"], dev["b2"], ws=ws)
        torch.cuda.synchronize()
        outs.append((y.clone(), aux.clone(), counts.clone()))
    for y2, a2, c2 in outs[1:]:  # bitwise run-to-run determinism
        assert torch.equal(y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2,
                           outs[0][0].view(torch.int16) if y2.dtype == torch.bfloat16 else outs[0][0])
        assert torch.equal(a2, outs[0][1]) and torch.equal(c2, outs[0][2])
    y, aux, counts = outs[0]
    H.check_bits_equal("expert_counts", H.to_np(counts), r["counts"])
    assert abs(float(H.to_np(aux)[0]) - r["aux"]) <= H.AUX_RTOL * max(abs(r["aux"]), 1.0)
    yg = H.to_np(y)
    if rows is not None:
        yg = yg[rows]
    raw, net = H.layer_err(yg, r["y"], cfg.dtype)
    H.say("[gpu] %s y: max|d|/rms = %.4f (raw), %.4f (net of output rounding)" % (cfg.name, raw, net))
    raw_bar = H.Y_TOL[cfg.dtype]
    if cfg.dtype == W.DT_BF16 and r["y"].size:
        raw_bar += (2.0 ** -8) * np.abs(r["y"]).max() / np.sqrt(np.mean(r["y"] ** 2))
    H.record("y", cfg.name, full=full, rows=len(yg), raw=raw, net=net, bar=H.Y_TOL[cfg.dtype], raw_bar=raw_bar)
    assert net <= H.Y_TOL[cfg.dtype], (raw, net)
    assert raw <= raw_bar, (raw, raw_bar)
    return raw


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_all_stages(name):
    cfg = SMALL[name]
    H.say("[gpu] small case %s %s" % (name, cfg))
    inp = _case(cfg)
    r = H.run_oracle(cfg, inp)
    dev = H.to_dev(inp)
    _check_route(cfg, dev, r)
    _check_permute(cfg, dev, r)
    _check_expert_ffn(cfg, inp, dev, r)
    _check_combine(cfg, r)
    _check_forward(cfg, dev, r)


@pytest.mark.parametrize("dtype,act", [(W.DT_BF16, W.ACT_SWIGLU), (W.DT_F32, W.ACT_GELU), (W.DT_BF16, W.ACT_GELU)])
def test_all_slots_on_first_experts(dtype, act):
    """W_r = 0: all logits tie, so experts 0..K-1 each take all T tokens (huge groups, idle rest)."""
    cfg = L("ties", 600, 128, 8, 2, 256, act, W.GATE_RENORM, dtype, "none", 31)
    H.say("[gpu] tie case %s" % (cfg,))
    inp = _case(cfg, zero_router=True)
    r = H.run_oracle(cfg, inp)
    assert r["counts"].tolist() == [600, 600, 0, 0, 0, 0, 0, 0]
    dev = H.to_dev(inp)
    _check_route(cfg, dev, r)
    _check_forward(cfg, dev, r)


@pytest.mark.parametrize("name,runs", [("ragged_large_k1", 3000), ("tiles_128x256", 3000)])
def test_forward_bitwise_repeatable_many(name, runs):
    """Thousands of forward calls give the same bits. Both shapes run 128-row
    tiles (128 x 128 and 128 x 256), whose last 16-k step of every stage is
    multiplied after the next stage's barrier: the wait before that barrier
    must also drain the LDS reads of those fragments, or another wave's refill
    of the slot can land first (before that wait was added, about 1 call in
    250 to 1000 of the first shape differed in one row)."""
    shapes = {"ragged_large_k1": SMALL["ragged_large_k1"],
              "tiles_128x256": L("tiles_128x256", 1600, 128, 16, 1, 4608, W.ACT_SWIGLU, W.GATE_RAW, W.DT_BF16,
                                 "zipf1.1", 37)}
    cfg = shapes[name]
    H.say("[gpu] repeatability %s x %d %s" % (name, runs, cfg))
    dev = H.to_dev(_case(cfg))
    desc = moe.desc_of(cfg)
    ws = moe.workspace(desc)
    ref = None
    differing = 0
    for _ in range(runs):
        y, aux, counts = moe.forward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"],
                                     dev["W2"], dev["b2"], ws=ws)
        yb = y.view(torch.int16).clone()
        if ref is None:
            ref = (yb, aux.clone(), counts.clone())
        elif not (torch.equal(yb, ref[0]) and torch.equal(aux, ref[1]) and torch.equal(counts, ref[2])):
            differing += 1
    torch.cuda.synchronize()
    assert differing == 0, "%d of %d calls differ from the first" % (differing, runs)


def test_empty_batch():
    cfg = L("empty", 0, 128, 8, 2, 256, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 32)
    H.say("[gpu] T=0")
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    desc = moe.desc_of(cfg)
    aux = torch.full((1,), 7.0, device="cuda")
    counts = torch.full((8,), 7, dtype=torch.int32, device="cuda")
    moe.forward(desc, dev["h"], dev["W_r"], None, dev["W1"], None, dev["W3"], dev["W2"], None, aux=aux,
                counts=counts)
    g = moe.route(desc, dev["h"], dev["W_r"], None)
    p = moe.permute(desc, g["topk_idx"], dev["h"])
    torch.cuda.synchronize()
    assert float(aux[0]) == 0.0 and counts.sum().item() == 0
    assert float(g["aux"][0]) == 0.0 and g["counts"].sum().item() == 0
    assert p["offsets"].tolist() == [0] * 9


def test_permute_skips_out_of_range_ids():
    """Slot ids outside [0, E) (only a caller of moe_permute can pass them):
    token_slot -1, no grouped row, not counted; every other slot is grouped as
    the stable sort by (expert, token) of the valid slots."""
    cfg = SMALL["bf16_raw_k2_e40"]
    H.say("[gpu] permute with out-of-range ids %s" % (cfg,))
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    r = H.run_oracle(cfg, inp)
    idx = r["topk_idx"].copy()
    rng = np.random.default_rng(5)
    bad = rng.random(idx.shape) < 0.1
    idx[bad] = rng.choice([-1, -7, cfg.E, cfg.E + 3], size=int(bad.sum()))
    desc = moe.desc_of(cfg)
    g = moe.permute(desc, torch.from_numpy(idx).cuda(), dev["h"])
    torch.cuda.synchronize()
    valid = ~bad
    tt, jj = np.nonzero(valid)
    ee = idx[tt, jj]
    order = np.lexsort((tt, ee))  # by expert, then token
    want_slot = np.full(idx.shape, -1, np.int64)
    want_slot[tt[order], jj[order]] = np.arange(len(order))
    counts = np.bincount(ee, minlength=cfg.E)
    H.check_bits_equal("expert_offsets", H.to_np(g["offsets"]), np.concatenate([[0], np.cumsum(counts)]))
    H.check_bits_equal("token_slot", H.to_np(g["token_slot"]), want_slot)
    n = len(order)
    H.check_bits_equal("slot_token", H.to_np(g["slot_token"])[:n], tt[order])
    rows = torch.from_numpy(tt[order].astype(np.int64)).cuda()
    assert torch.equal(g["h_perm"][:n].view(torch.int16), dev["h"][rows].view(torch.int16))


@pytest.mark.parametrize("act", [W.ACT_SWIGLU, W.ACT_GELU])
def test_group_size_boundaries(act):
    """Group sizes on both sides of the 16-, 32-, 64- and 128-row tile and
    fragment edges, with empty groups between, given to moe_expert_ffn
    directly as offsets over rows in token order (the tiled kernels enumerate
    their tiles from these offsets on the device)."""
    sizes = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 128, 129, 200, 0, 5]
    T = int(sum(sizes))
    cfg = L("group_bounds", T, 1024, len(sizes), 1, 1032, act, W.GATE_RAW, W.DT_BF16, "none", 43)
    H.say("[gpu] group size boundaries %s" % (cfg,))
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    o = moe.expert_ffn(moe.desc_of(cfg), dev["h"], torch.from_numpy(offs).cuda(), dev["W1"], dev["b1"],
                       dev["W3"], dev["W2"], dev["b2"])
    torch.cuda.synchronize()
    o = H.to_np(o)
    p = H.oracle_params(inp)
    ref = np.zeros((T, cfg.d))
    for e, n in enumerate(sizes):
        if n:
            ref[offs[e]:offs[e + 1]] = O.expert_ffn(p["h"][offs[e]:offs[e + 1]], e, p, act)
    for e, n in enumerate(sizes):
        if n:
            err = H.rel_err(o[offs[e]:offs[e + 1]], ref[offs[e]:offs[e + 1]])
            assert err <= H.Y_TOL[cfg.dtype], (e, n, err)


def _tiles_256(S, E, N, nmat):
    """The library's choice of 256 x 256 tiles for a grouped GEMM: about 1k rows
    per expert and at least two tiles per CU."""
    bn = 256 // nmat
    return S // E >= 512 and ((S + 255) // 256 + min(E, S)) * ((N + bn - 1) // bn) >= 2 * 256


@pytest.mark.parametrize("act", [W.ACT_SWIGLU, W.ACT_GELU])
def test_split_tails_256(act):
    """Second GEMM on 256 x 256 tiles with experts whose last m-tile holds at
    most 64 rows: those tails run as four tiles over quarters of the reduction
    and are summed into o_perm afterwards. Tails of 1, 63 and 64 rows, an
    expert of 40 rows (its only tile split), a tail of 65 rows and a whole
    number of tiles (not split). Every tail row and the first and last rows of
    every whole tile are compared with the oracle (GELU: the bias b2 enters
    once); o_perm is bitwise the same on a second call."""
    sizes = [2049, 1087, 1344, 1089, 1024, 40]
    T, d, width = int(sum(sizes)), 4096, 1024
    assert _tiles_256(T, len(sizes), d, 1) and (width + 63) // 64 >= 16
    cfg = L("split_tails", T, d, len(sizes), 1, width, act, W.GATE_RAW, W.DT_BF16, "none", 61)
    H.say("[gpu] split tails %s" % (cfg,))
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    offs_d = torch.from_numpy(offs).cuda()
    desc = moe.desc_of(cfg)
    o1 = moe.expert_ffn(desc, dev["h"], offs_d, dev["W1"], dev["b1"], dev["W3"], dev["W2"], dev["b2"])
    o2 = moe.expert_ffn(desc, dev["h"], offs_d, dev["W1"], dev["b1"], dev["W3"], dev["W2"], dev["b2"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "o_perm differs between two calls"
    o = H.to_np(o1)
    p = H.oracle_params(inp)
    for e, n in enumerate(sizes):
        full, rem = divmod(n, 256)
        rows = set()
        for m in range(full):
            rows.update((m * 256, m * 256 + 255))
        rows.update(range(full * 256, n))
        rows = np.array(sorted(rows), dtype=np.int64) + offs[e]
        ref = O.expert_ffn(p["h"][rows], e, p, act)
        err = H.rel_err(o[rows], ref)
        H.record("o", "split_tails_%s_e%d" % ("swiglu" if act == W.ACT_SWIGLU else "gelu", e), rows=len(rows),
                 tail=rem, err=err, bar=H.Y_TOL[cfg.dtype])
        assert err <= H.Y_TOL[cfg.dtype], (e, n, err)


@pytest.mark.parametrize("capacity", [0, 1])
def test_forward_equals_composition(capacity):
    """moe_forward against the four entry points in a row (moe_route,
    moe_permute, moe_expert_ffn, moe_combine) on the Mixtral-shaped prefill
    layer, whose second GEMM splits four experts' short tails: the fused path
    (h read through the grouping, workspace-resident o_perm) and the composition
    (gathered h_perm, caller's o_perm) must give y bit for bit the same
    (dropless, and with a capacity of T*K/E slots per expert)."""
    cfg = W.WORKLOADS["mixtral_prefill"]
    cap = moe.capacity_slots(1.0, cfg.T, cfg.K, cfg.E) if capacity else 0
    H.say("[gpu] forward vs composition %s capacity=%d" % (cfg.name, cap))
    inp = W.make_inputs(cfg)
    dev = H.to_dev(inp)
    desc = moe.desc_of(cfg, capacity=cap)
    y, _, _ = moe.forward(desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"], dev["W2"],
                          dev["b2"])
    g = moe.route(desc, dev["h"], dev["W_r"], dev["b_r"])
    pm = moe.permute(desc, g["topk_idx"], dev["h"])
    o = moe.expert_ffn(desc, pm["h_perm"], pm["offsets"], dev["W1"], dev["b1"], dev["W3"], dev["W2"], dev["b2"])
    y2 = moe.combine(desc, o, pm["token_slot"], g["topk_gate"], y.dtype)
    torch.cuda.synchronize()
    counts = np.diff(H.to_np(pm["offsets"]).astype(np.int64))
    kept = np.minimum(counts, cap) if cap else counts
    assert ((kept % 256 > 0) & (kept % 256 <= 64)).any() or cap, "no split tail in this layer"
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "moe_forward differs from the composition"
    del dev
    torch.cuda.empty_cache()


def test_max_operand_size():
    """The largest layer the 32-bit offsets allow: T*K*d = 2^31 - 2^22 elements
    of h rows read through the grouping (T = 261632 tokens, d = 4096, top-2),
    so the byte offsets of the last rows' loads sit at the limit. Routing of
    every token bit-exact; y on the first and last tokens and a seeded sample.
    (About 35 s of host time for the inputs and the oracle.)"""
    cfg = L("max_offsets", 261632, 4096, 8, 2, 512, W.ACT_SWIGLU, W.GATE_RENORM, W.DT_BF16, "none", 51)
    assert cfg.T * cfg.K * cfg.d == 2 ** 31 - 2 ** 22
    H.say("[gpu] max operand size %s" % (cfg,))
    inp = W.make_inputs(cfg)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(cfg.T - 8, cfg.T),
                                     rng.choice(cfg.T, size=24, replace=False)])).astype(np.int64)
    r = H.run_oracle(cfg, inp, tokens=rows)
    dev = H.to_dev(inp)
    del inp
    _check_route(cfg, dev, r)
    layer_desc = moe.desc_of(cfg)
    y, aux, counts = moe.forward(layer_desc, dev["h"], dev["W_r"], dev["b_r"], dev["W1"], dev["b1"], dev["W3"],
                                 dev["W2"], dev["b2"])
    torch.cuda.synchronize()
    H.check_bits_equal("expert_counts", H.to_np(counts), r["counts"])
    assert abs(float(H.to_np(aux)[0]) - r["aux"]) <= H.AUX_RTOL * max(abs(r["aux"]), 1.0)
    yg = H.to_np(y[torch.from_numpy(rows).cuda()])
    raw, net = H.layer_err(yg, r["y"], cfg.dtype)
    H.say("[gpu] max operand size y: max|d|/rms = %.4f (raw), %.4f (net)" % (raw, net))
    assert net <= H.Y_TOL[cfg.dtype], (raw, net)
    del dev, y
    torch.cuda.empty_cache()


FULL = ["micro", "skewed", "mixtral_prefill", "mixtral_decode", "switch_top1"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload(name):
    """Every token and every grouped row of the workload against the oracle."""
    cfg = W.WORKLOADS[name]
    H.say("[gpu] full workload %s %s" % (name, cfg))
    inp = W.make_inputs(cfg)
    r = H.run_oracle(cfg, inp)
    dev = H.to_dev(inp)
    _check_route(cfg, dev, r)
    _check_permute(cfg, dev, r)
    _check_expert_ffn(cfg, inp, dev, r, full=True)
    _check_combine(cfg, r)
    err = _check_forward(cfg, dev, r, full=True)
    H.say("[gpu] %s y max|d|/rms = %.3e, aux = %.6f, idle experts = %d, max share = %.3f" % (
        name, err, r["aux"], int((r["counts"] == 0).sum()), r["counts"].max() / cfg.S))
    del dev
    torch.cuda.empty_cache()
