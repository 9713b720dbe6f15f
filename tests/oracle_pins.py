"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Each check_* function raises AssertionError when the oracle disagrees with a
printed value, a closed form, an invariant, a textbook routine or brute force.
tests/test_oracle_pins.py runs them; tests/test_oracle_mutations.py plants
plausible mistakes in the oracle and requires that at least one check fails.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- exact fp32 fma

def _round_f32(x: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) float32 of an exact rational."""
    c = np.float32(float(x))
    cands = {np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))}
    best = None
    for v in cands:
        err = abs(Fraction(float(v)) - x)
        key = (err, int(np.array(v, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def _fma_f32(a: np.float32, b: np.float32, c: np.float32) -> np.float32:
    exact = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    if exact == 0:
        neg = (math.copysign(1.0, float(a) * float(b)) < 0) and (math.copysign(1.0, float(c)) < 0)
        return np.float32(-0.0 if neg else 0.0)
    return _round_f32(exact)


def check_router_logits_exact(seed=0):
    """Bit-exact: the C router equals four rational-arithmetic fma chains (groups
    of four k dealt round-robin) summed pairwise, with and without bias. d = 40
    wraps the round-robin twice and ends part-way through it."""
    rng = np.random.default_rng(seed)
    T, d, E = 5, 40, 6
    h = rng.standard_normal((T, d)).astype(np.float32)
    W = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    # cancellation-heavy token: exercises rounding of small results
    h[3] = np.float32(1e3) * np.sign(h[3])
    W[:, 2] = np.float32(1e-3) * (np.arange(d) % 2 * 2 - 1)
    b = rng.standard_normal(E).astype(np.float32)
    for bias in (None, b):
        got = O.router_logits_f32(h, W, bias)
        for t in range(T):
            for e in range(E):
                c = [np.float32(0.0)] * 4
                for k in range(d):
                    j = (k // 4) % 4
                    c[j] = _fma_f32(h[t, k], W[k, e], c[j])
                s01 = _round_f32(Fraction(float(c[0])) + Fraction(float(c[1])))
                s23 = _round_f32(Fraction(float(c[2])) + Fraction(float(c[3])))
                acc = _round_f32(Fraction(float(s01)) + Fraction(float(s23)))
                if bias is not None:
                    acc = _round_f32(Fraction(float(acc)) + Fraction(float(bias[e])))
                assert np.array(got[t, e]).view(np.uint32) == np.array(acc).view(np.uint32), \
                    (t, e, got[t, e], acc, bias is not None)


def check_router_logits_bound(seed=1):
    """|l32 - l| <= gamma_(d+1) (sum_k |h_k W_k| + |b|) for d = 4096 (float32 error bound)."""
    rng = np.random.default_rng(seed)
    T, d, E = 32, 4096, 8
    h = rng.standard_normal((T, d)).astype(np.float32)
    W = (rng.standard_normal((d, E)) * 0.02).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    l32 = O.router_logits_f32(h, W, b).astype(np.float64)
    h64, W64, b64 = h.astype(np.float64), W.astype(np.float64), b.astype(np.float64)
    exact = h64 @ W64 + b64
    u = 2.0 ** -24
    gamma = (d + 1) * u / (1 - (d + 1) * u)
    mag = np.abs(h64) @ np.abs(W64) + np.abs(b64)
    bound = gamma * mag + 1e-12 * mag  # float64 reference error is far below this margin
    assert np.all(np.abs(l32 - exact) <= bound)
    assert np.any(l32 != exact)  # genuinely float32


def check_topk_bruteforce(seed=2):
    """Top-K set and order vs brute force over all K-subsets, including forced ties."""
    rng = np.random.default_rng(seed)
    for E in range(1, 9):
        for K in range(1, min(4, E) + 1):
            for tie in (False, True):
                T = 24
                l = rng.standard_normal((T, E)).astype(np.float32)
                if tie:
                    l = np.round(l * 2) / 2  # many equal logits
                    l[0] = 0.0
                idx = O.select_topk(l, K)
                assert idx.shape == (T, K) and idx.dtype == np.int32
                for t in range(T):
                    best = None
                    for sub in itertools.combinations(range(E), K):
                        s = sum(Fraction(float(l[t, i])) for i in sub)
                        if best is None or s > best[0]:
                            best = (s, sub)
                    assert tuple(sorted(idx[t].tolist())) == best[1], (E, K, t, l[t], idx[t])
                    order = sorted(best[1], key=lambda i: (-float(l[t, i]), i))
                    assert idx[t].tolist() == order


def check_probs(seed=3):
    """Full softmax: rows sum to 1; matches scipy's softmax; shift invariance."""
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(seed)
    l = (rng.standard_normal((50, 8)) * 3).astype(np.float32)
    p = O.router_probs(l)
    assert np.allclose(p.sum(1), 1.0, atol=1e-15, rtol=0)
    assert np.allclose(p, sp_softmax(l.astype(np.float64), axis=1), atol=1e-15, rtol=0)
    assert np.allclose(O.router_probs(l.astype(np.float64) + 7.0), p, atol=1e-15, rtol=0)  # exact shift


def check_gates_worked_example():
    """Lensa ML Step 3: unchosen p's as printed, chosen gates 0.61 / 0.39, chosen mass 56%."""
    g = _golden("lensa_step3_topk_combine.json")
    mass = g["chosen_mass_percent"] / 100.0
    p = np.zeros(8)
    for k, v in g["unchosen_p"].items():
        p[int(k[1:]) - 1] = v
    p[2] = mass * g["chosen_gates"]["E3"]
    p[3] = mass * g["chosen_gates"]["E4"]
    assert abs(p.sum() - 1.0) < 1e-12  # the printed numbers are consistent
    logits = np.log(p).astype(np.float32)[None, :]
    idx = O.select_topk(logits, 2)
    assert idx[0].tolist() == [2, 3]
    gr = O.gates(logits, idx, O.GATE_RENORM)[0]
    assert round(gr[0], 2) == 0.61 and round(gr[1], 2) == 0.39
    pr = O.router_probs(logits)[0]
    for k, v in g["unchosen_p"].items():
        assert round(pr[int(k[1:]) - 1], 2) == v
    assert round(100 * (pr[2] + pr[3])) == g["chosen_mass_percent"]
    graw = O.gates(logits, idx, O.GATE_RAW)[0]
    assert np.allclose(graw, pr[[2, 3]], rtol=0, atol=1e-15)


def check_gates_invariants(seed=4):
    """RENORM gates sum to 1, K=1 RENORM is exactly 1, K=E gives the full softmax."""
    rng = np.random.default_rng(seed)
    E = 8
    l = (rng.standard_normal((40, E)) * 2).astype(np.float32)
    for K in (1, 2, 3, 8):
        idx = O.select_topk(l, K)
        g = O.gates(l, idx, O.GATE_RENORM)
        assert np.all(np.abs(g.sum(1) - 1.0) < 1e-15)
        assert np.all(np.diff(g, axis=1) <= 0)  # largest logit first -> largest gate first
        if K == 1:
            assert np.all(g == 1.0)
        if K == E:
            p = O.router_probs(l)
            assert np.allclose(g, np.take_along_axis(p, idx.astype(np.int64), 1), rtol=0, atol=1e-15)
            assert np.allclose(O.gates(l, idx, O.GATE_RAW), g, rtol=0, atol=1e-15)


def check_combine_worked_example():
    """Lensa ML Step 3: 0.61 E3(h) + 0.39 E4(h) printed as [0.27, 0.30, -0.53, -0.52]."""
    g = _golden("lensa_step3_topk_combine.json")
    o = np.array([g["E3_h"], g["E4_h"]], dtype=np.float64)
    gates = np.array([[g["chosen_gates"]["E3"], g["chosen_gates"]["E4"]]])
    y = O.combine(o, np.array([[0, 1]], dtype=np.int32), gates)[0]
    assert [round(v, g["printed_decimals"]) for v in y] == g["y_printed"], y


def check_permutation_sorted(seed=5):
    """Grouping equals Python's stable sorted() of the slots by (expert, token)."""
    rng = np.random.default_rng(seed)
    for T, E, K in ((1, 1, 1), (37, 5, 2), (64, 8, 3), (200, 64, 1), (0, 4, 2)):
        l = rng.standard_normal((T, E)).astype(np.float32)
        idx = O.select_topk(l, K)
        offsets, slot_token, token_slot = O.stable_permutation(idx, E)
        slots = sorted(((int(idx[t, j]), t, j) for t in range(T) for j in range(K)),
                       key=lambda s: (s[0], s[1]))
        assert slot_token.tolist() == [s[1] for s in slots]
        for s, (e, t, j) in enumerate(slots):
            assert token_slot[t, j] == s
        cnt = [sum(1 for s in slots if s[0] == e) for e in range(E)]
        assert offsets.tolist() == [sum(cnt[:e]) for e in range(E + 1)]
        assert O.expert_counts(idx, E).tolist() == cnt


def check_load_stats_page():
    """Lensa ML Step 4: 512 slots, balanced 64, busiest 44.7%, top two 77%, two idle."""
    g = _golden("lensa_step4_load.json")
    s = O.load_stats(g["counts"], g["T"], g["K"])
    assert s["slots"] == g["T"] * g["K"]
    assert s["balanced"] == g["balanced_printed"]
    assert round(100 * s["busiest_share"], 1) == g["busiest_share_percent_printed"]
    assert round(100 * s["top2_share"]) == g["top2_share_percent_printed"]
    assert s["idle"] == g["idle_printed"]


def check_aux_uniform_probs():
    """W_r = 0, no bias: every p = 1/E exactly, so E * sum f P = sum f = 1 exactly, for any K."""
    rng = np.random.default_rng(6)
    for E, K, T in ((8, 2, 40), (4, 1, 9), (64, 2, 33), (2, 2, 5), (1, 1, 7)):
        d = 16
        inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
               "W_r": np.zeros((d, E), np.float32), "b_r": None}
        l = O.router_logits_f32(inp["h"], inp["W_r"], None)
        idx = O.select_topk(l, K)
        assert idx[:, :].tolist() == [list(range(K))] * T  # all ties: lowest indices win
        aux = O.aux_loss(O.expert_counts(idx, E), O.router_probs(l), K)
        assert aux == 1.0, (E, K, aux)


def check_aux_uniform_load():
    """Every expert gets exactly T*K/E slots: E * sum f P = sum P = 1 whatever p is."""
    E, K, T, d = 4, 1, 12, 4
    h = np.zeros((T, d), np.float32)
    for t in range(T):
        h[t, t % E] = 1.0 + 0.1 * t  # token t points at expert t % E
    W = np.eye(d, E, dtype=np.float32) * 3.0
    l = O.router_logits_f32(h, W, None)
    idx = O.select_topk(l, K)
    counts = O.expert_counts(idx, E)
    assert counts.tolist() == [T * K // E] * E
    aux = O.aux_loss(counts, O.router_probs(l), K)
    assert abs(aux - 1.0) < 1e-14
    # sharply peaked router with one-hot routing: P -> f, so aux -> E * sum f^2
    W2 = np.eye(d, E, dtype=np.float32) * 200.0
    h2 = np.zeros((T, d), np.float32)
    h2[:, 0] = 1.0
    h2[: T // 2, 1] = 2.0
    l2 = O.router_logits_f32(h2, W2, None)
    idx2 = O.select_topk(l2, 1)
    c2 = O.expert_counts(idx2, E)
    f = c2 / T
    assert abs(O.aux_loss(c2, O.router_probs(l2), 1) - E * np.sum(f * f)) < 1e-12


def _torch_dense_ffn(x, W1, b1, W3, W2, b2, act):
    xt = torch.from_numpy(x)
    z = xt @ torch.from_numpy(W1).T
    if act == O.ACT_GELU:
        if b1 is not None:
            z = z + torch.from_numpy(b1)
        o = torch.nn.functional.gelu(z, approximate="none") @ torch.from_numpy(W2).T
        if b2 is not None:
            o = o + torch.from_numpy(b2)
        return o.numpy()
    z3 = xt @ torch.from_numpy(W3).T
    return ((torch.nn.functional.silu(z) * z3) @ torch.from_numpy(W2).T).numpy()


def check_dense_reduction(seed=7):
    """E = 1, K = 1: the layer is exactly the dense FFN (gate 1.0), checked against torch."""
    rng = np.random.default_rng(seed)
    T, d, w = 19, 24, 40
    for act in (O.ACT_GELU, O.ACT_SWIGLU):
        for gate in (O.GATE_RENORM, O.GATE_RAW):
            inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
                   "W_r": rng.standard_normal((d, 1)).astype(np.float32),
                   "b_r": rng.standard_normal(1).astype(np.float32),
                   "W1": rng.standard_normal((1, w, d)) * d ** -0.5,
                   "W2": rng.standard_normal((1, d, w)) * w ** -0.5}
            if act == O.ACT_GELU:
                inp.update(b1=rng.standard_normal((1, w)) * 0.3, b2=rng.standard_normal((1, d)) * 0.3, W3=None)
            else:
                inp.update(W3=rng.standard_normal((1, w, d)) * d ** -0.5, b1=None, b2=None)
            r = O.moe_forward(inp, T, d, 1, 1, act, gate)
            assert np.all(r["topk_gate"] == 1.0) and np.all(r["topk_idx"] == 0)
            ref = _torch_dense_ffn(inp["h"].astype(np.float64), inp["W1"][0],
                                   None if inp["b1"] is None else inp["b1"][0],
                                   None if inp["W3"] is None else inp["W3"][0], inp["W2"][0],
                                   None if inp["b2"] is None else inp["b2"][0], act)
            assert np.max(np.abs(r["y"] - ref)) < 1e-12
            assert r["aux"] == 1.0


def check_soft_mixture_K_equals_E(seed=8):
    """K = E: top-K keeps every expert and y = sum_e p_e E_e(h) (the dense soft mixture)."""
    rng = np.random.default_rng(seed)
    T, d, w, E = 7, 12, 20, 4
    inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
           "W_r": rng.standard_normal((d, E)).astype(np.float32), "b_r": None,
           "W1": rng.standard_normal((E, w, d)) * d ** -0.5,
           "W3": rng.standard_normal((E, w, d)) * d ** -0.5,
           "W2": rng.standard_normal((E, d, w)) * w ** -0.5, "b1": None, "b2": None}
    r = O.moe_forward(inp, T, d, E, E, O.ACT_SWIGLU, O.GATE_RENORM)
    p = r["probs"]
    x = inp["h"].astype(np.float64)
    ref = np.zeros((T, d))
    for e in range(E):
        ref += p[:, e:e + 1] * _torch_dense_ffn(x, inp["W1"][e], None, inp["W3"][e], inp["W2"][e],
                                                None, O.ACT_SWIGLU)
    assert np.max(np.abs(r["y"] - ref)) < 1e-12


def check_forward_subset_consistency(seed=9):
    """Computing only some rows of y gives the same rows as the full layer."""
    rng = np.random.default_rng(seed)
    T, d, w, E, K = 30, 16, 24, 5, 2
    inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
           "W_r": rng.standard_normal((d, E)).astype(np.float32),
           "b_r": rng.standard_normal(E).astype(np.float32),
           "W1": rng.standard_normal((E, w, d)), "W2": rng.standard_normal((E, d, w)),
           "b1": rng.standard_normal((E, w)), "b2": rng.standard_normal((E, d)), "W3": None}
    full = O.moe_forward(inp, T, d, E, K, O.ACT_GELU, O.GATE_RENORM)
    rows = [29, 0, 13, 13, 7]
    part = O.moe_forward(inp, T, d, E, K, O.ACT_GELU, O.GATE_RENORM, tokens=rows)
    # the library float64 matmul may round the last bit differently for a
    # different number of rows, so equal up to a few ulps, not bit for bit
    assert np.allclose(part["y"], full["y"][rows], rtol=1e-13, atol=1e-13)
    # the grouped formulation (permute -> per-expert FFN -> combine) gives the same y
    o = np.zeros((T * K, d))
    for e in range(E):
        s0, s1 = full["offsets"][e], full["offsets"][e + 1]
        if s1 > s0:
            o[s0:s1] = O.expert_ffn(inp["h"][full["slot_token"][s0:s1]], e, inp, O.ACT_GELU)
    y2 = O.combine(o, full["token_slot"], full["topk_gate"])
    assert np.max(np.abs(y2 - full["y"])) < 1e-12


def check_param_counts():
    """Printed parameter counts of the micro model, the 7B shape and Mixtral."""
    g = _golden("param_counts.json")
    m = g["micro"]
    c = O.param_counts_micro(m["d"], m["layers"], m["E"], m["K"], m["width"])
    assert round(c["total"] / 1e6, 2) == m["total_millions_printed"]
    assert round(c["active"] / 1e6, 2) == m["active_millions_printed"]
    assert round(c["total"] / c["active"], 2) == m["ratio_printed"]
    c64 = O.param_counts_micro(m["d"], m["layers"], 64, m["K"], m["width"])
    assert round(c64["total"] / c64["active"], 1) == m["ratio_E64_printed"]
    assert round(c["attention_plus_active_experts"] / 1e6, 2) == m["text_active_millions_printed"]

    s = g["seven_b_shape"]
    c7 = O.param_counts_swiglu_model(s["d"], s["layers"], s["E"], s["K"], s["width"])
    assert round(c7["expert"] / 1e6) == s["expert_millions_printed"]
    assert round(c7["total"] / 1e9, 1) == s["total_billions_printed"]
    assert round(c7["active"] / 1e9, 1) == s["active_billions_printed"]
    assert round(c7["total"] / c7["active"], 1) == s["ratio_printed"]
    # convention-free: the difference is exactly L (E - K) experts
    assert c7["total"] - c7["active"] == s["layers"] * (s["E"] - s["K"]) * c7["expert"]
    assert abs((c7["total"] - c7["active"]) / 1e9
               - (s["total_billions_printed"] - s["active_billions_printed"])) <= 0.1

    x = g["mixtral"]
    cm = O.param_counts_swiglu_model(x["d"], x["layers"], x["E"], x["K"], x["width"])
    assert round(cm["expert"] / 1e6) == x["expert_millions_printed"]
    assert round(cm["routed_total"] / 1e9, 1) == x["routed_billions_printed"]
    assert round(100 * cm["routed_total"] / (x["total_billions_printed"] * 1e9)) == \
        x["routed_share_percent_printed"]
    # active = shared + routed * K / E with shared = printed total - routed
    shared = x["total_billions_printed"] * 1e9 - cm["routed_total"]
    active = shared + cm["routed_total"] * x["K"] / x["E"]
    assert round(active / 1e9, 1) == x["active_billions_printed"]
    assert round(x["total_billions_printed"] * 2) == x["held_GB_fp16_printed"]
    assert round(x["active_billions_printed"] * 2) == x["read_per_token_GB_fp16_printed"]


# ----------------------------------------------------------------------------- capacity

def _routing_with_counts(counts, T, K, seed):
    """A T x K routing (distinct experts per token) whose per-expert counts are `counts`."""
    slots = [e for e, c in enumerate(counts) for _ in range(c)]
    assert len(slots) == T * K
    idx = np.array([[slots[t + j * T] for j in range(K)] for t in range(T)], np.int32)
    assert all(len(set(r)) == K for r in idx.tolist())
    return idx[np.random.default_rng(seed).permutation(T)]  # any token order


def check_capacity_widget():
    """Lensa ML Step 5: C = 1.00 x 256 x 2 / 8 = 64; 94 slots dropped (18.4 %)."""
    g = _golden("lensa_step5_capacity.json")
    C = O.capacity_slots(g["factor"], g["T"], g["K"], g["E"])
    assert C == g["capacity_printed"]
    st = O.drop_stats(g["counts"], C)
    assert st["dropped"] == g["dropped_printed"]
    assert round(st["percent"], 1) == g["percent_dropped_printed"]
    # the same through the slot-level rule, on a routing with the page's counts
    idx = _routing_with_counts(g["counts"], g["T"], g["K"], seed=11)
    keep = O.capacity_keep(idx, g["E"], C)
    assert int((~keep).sum()) == g["dropped_printed"]
    kept_per_expert = np.bincount(idx[keep].astype(np.int64), minlength=g["E"])
    assert kept_per_expert.tolist() == [min(c, C) for c in g["counts"]]


def check_capacity_order(seed=12):
    """'First C slots in token order', restated by sorting: for each expert, the C
    smallest token indices among the tokens that chose it are kept."""
    rng = np.random.default_rng(seed)
    for _ in range(200):
        T, E = int(rng.integers(1, 13)), int(rng.integers(1, 6))
        K = int(rng.integers(1, E + 1))
        idx = np.array([rng.permutation(E)[:K] for _ in range(T)], np.int32)
        for C in range(0, T + 2):
            keep = O.capacity_keep(idx, E, C)
            ref = np.zeros_like(keep)
            for e in range(E):
                toks = sorted({t for t in range(T) for j in range(K) if idx[t, j] == e})
                for t in toks[:C]:
                    ref[t, list(idx[t]).index(e)] = True
            assert np.array_equal(keep, ref), (T, E, K, C)
            if C >= T:
                assert keep.all()


def check_capacity_slots_rounding():
    """C is the smallest integer with C * E >= factor * T * K (exact for the page's integer case)."""
    for factor in ("0.5", "0.75", "1.0", "1.1", "1.25", "2.0", "0.3"):
        for T, K, E in ((256, 2, 8), (80, 1, 8), (7, 2, 3), (4096, 2, 8), (8192, 1, 64)):
            C = O.capacity_slots(factor, T, K, E)
            need = Fraction(factor) * T * K
            assert C * E >= need and (C - 1) * E < need, (factor, T, K, E, C)


def check_capacity_layer(seed=13):
    """C >= T is the dropless layer; C = 0 gives y = 0; tokens that keep every slot
    match the dropless rows and tokens that keep none are 0; routing outputs
    (counts, aux) describe the router's choices and do not change."""
    rng = np.random.default_rng(seed)
    T, d, w, E, K = 40, 12, 16, 4, 2
    inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
           "W_r": rng.standard_normal((d, E)).astype(np.float32),
           "b_r": (rng.standard_normal(E) * 2).astype(np.float32),
           "W1": rng.standard_normal((E, w, d)) * d ** -0.5, "W3": rng.standard_normal((E, w, d)) * d ** -0.5,
           "W2": rng.standard_normal((E, d, w)) * w ** -0.5, "b1": None, "b2": None}
    free = O.moe_forward(inp, T, d, E, K, O.ACT_SWIGLU, O.GATE_RENORM)
    big = O.moe_forward(inp, T, d, E, K, O.ACT_SWIGLU, O.GATE_RENORM, capacity=T)
    assert np.array_equal(big["y"], free["y"]) and big["keep"].all()
    zero = O.moe_forward(inp, T, d, E, K, O.ACT_SWIGLU, O.GATE_RENORM, capacity=0)
    assert not zero["y"].any() and not zero["keep"].any()
    assert np.all(zero["token_slot_kept"] == -1)
    C = O.capacity_slots("0.75", T, K, E)
    cap = O.moe_forward(inp, T, d, E, K, O.ACT_SWIGLU, O.GATE_RENORM, capacity=C)
    keep = cap["keep"]
    assert 0 < (~keep).sum() < T * K  # some, not all, slots dropped
    full_rows, none_rows = keep.all(axis=1), ~keep.any(axis=1)
    assert np.array_equal(cap["y"][full_rows], free["y"][full_rows])
    assert not cap["y"][none_rows].any()
    assert np.array_equal(cap["counts"], free["counts"]) and cap["aux"] == free["aux"]
    assert np.array_equal(cap["token_slot_kept"][keep], free["token_slot"][keep])


def _bias_case(seed):
    rng = np.random.default_rng(seed)
    T, d, E, K, w = 40, 24, 6, 2, 8
    inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
           "W_r": rng.standard_normal((d, E)).astype(np.float32), "b_r": None,
           "W1": rng.standard_normal((E, w, d)) * 0.3, "W3": rng.standard_normal((E, w, d)) * 0.3,
           "W2": rng.standard_normal((E, d, w)) * 0.3, "b1": None, "b2": None}
    return rng, inp, (T, d, E, K)


def check_bias_select_only(seed=21):
    """Selection-only routing bias ([LENSA] Step 4, DeepSeek-V3's per-expert
    routing bias): zero bias is the default path; the choice is the brute-force
    top-K of logits + bias; gates and P are those of the unbiased logits, so a
    bias that keeps the choice keeps them, and a forcing bias keeps the
    unbiased gate ratio of the chosen pair."""
    rng, inp, (T, d, E, K) = _bias_case(seed)
    fwd = lambda b, sel: O.moe_forward({**inp, "b_r": b}, T, d, E, K, O.ACT_SWIGLU, O.GATE_RENORM,
                                       bias_select_only=sel)
    base = fwd(None, False)
    r0 = fwd(np.zeros(E, np.float32), True)
    for k in ("topk_idx", "topk_gate", "probs", "y", "counts"):
        assert np.array_equal(r0[k], base[k]), k
    assert r0["aux"] == base["aux"]
    b = (rng.standard_normal(E) * 1.5).astype(np.float32)
    r = fwd(b, True)
    scores = base["logits"] + b[None, :]  # float32 addition, as the router does
    for t in range(T):
        best = max(itertools.combinations(range(E), K), key=lambda c: float(sum(scores[t, list(c)])))
        assert sorted(best) == sorted(r["topk_idx"][t].tolist()), t
        assert scores[t, r["topk_idx"][t, 0]] >= scores[t, r["topk_idx"][t, 1]]
    # gates from the unbiased logits of the chosen pair; P unbiased
    l = base["logits"].astype(np.float64)
    i0, i1 = r["topk_idx"][:, 0], r["topk_idx"][:, 1]
    ratio = r["topk_gate"][:, 0] / r["topk_gate"][:, 1]
    assert np.allclose(ratio, np.exp(l[np.arange(T), i0] - l[np.arange(T), i1]), rtol=1e-12)
    assert np.allclose(r["topk_gate"].sum(axis=1), 1.0, atol=1e-14)
    assert np.array_equal(r["probs"], base["probs"])
    f = r["counts"] / float(T * K)
    assert abs(r["aux"] - E * float(np.sum(f * base["probs"].mean(axis=0)))) < 1e-12
    # the same bias in the default mode moves the gates (the check above is not vacuous)
    rd = fwd(b, False)
    assert np.array_equal(rd["topk_idx"], r["topk_idx"])
    assert not np.allclose(rd["topk_gate"], r["topk_gate"])
    # a forcing bias: every token takes expert 3 first, gates still unbiased
    bf = np.zeros(E, np.float32)
    bf[3] = 1e4
    rf = fwd(bf, True)
    assert np.all(rf["topk_idx"][:, 0] == 3)
    j1 = rf["topk_idx"][:, 1]
    assert np.allclose(rf["topk_gate"][:, 0] / rf["topk_gate"][:, 1], np.exp(l[:, 3] - l[np.arange(T), j1]),
                       rtol=1e-12)


def _bw_case(seed, T, d, E, K, w, act, bias=True, ffn_bias=False):
    rng = np.random.default_rng(seed)
    inp = {"h": rng.standard_normal((T, d)), "W_r": rng.standard_normal((d, E)),
           "b_r": rng.standard_normal(E) if bias else None,
           "W1": rng.standard_normal((E, w, d)) * 0.4, "W2": rng.standard_normal((E, d, w)) * 0.4,
           "W3": rng.standard_normal((E, w, d)) * 0.4 if act == O.ACT_SWIGLU else None,
           "b1": rng.standard_normal((E, w)) * 0.3 if ffn_bias else None,
           "b2": rng.standard_normal((E, d)) * 0.3 if ffn_bias else None}
    return rng, inp


def _fd_backward(seed, T, d, E, K, w, act, gate, daux, n_probe=5, eps=1e-6, bias=True, ffn_bias=False, dz=0.0,
                 noise_scale=0.0, **kw):
    rng, inp = _bw_case(seed, T, d, E, K, w, act, bias, ffn_bias)
    dy = rng.standard_normal((T, d))
    noise = rng.standard_normal((T, E)) * noise_scale if noise_scale else None

    def loss(x):
        r = O.moe_forward(x, T, d, E, K, act, gate, logits_f64=True, noise=noise, **kw)
        return float(np.sum(dy * r["y"]) + daux * r["aux"] + dz * r["z_loss"])

    # the expert choice must not flip inside +-eps: keep clear top-K margins
    l = O.router_logits_f64(inp["h"], inp["W_r"], inp["b_r"])
    if noise is not None:
        l = l + noise
    srt = np.sort(l, axis=1)[:, ::-1]
    assert K == E or np.min(srt[:, K - 1] - srt[:, K]) > 1e-3
    g = O.moe_backward(inp, T, d, E, K, act, gate, dy, daux=daux, logits_f64=True, noise=noise, dz_loss=dz, **kw)
    for pname, gname in (("h", "dh"), ("W_r", "dW_r"), ("b_r", "db_r"), ("W1", "dW1"), ("W3", "dW3"),
                         ("W2", "dW2"), ("b1", "db1"), ("b2", "db2")):
        if inp[pname] is None:
            assert g[gname] is None, gname
            continue
        base = np.asarray(inp[pname], np.float64)
        for _ in range(n_probe):
            i = tuple(int(rng.integers(0, n)) for n in base.shape)
            up, dn = base.copy(), base.copy()
            up[i] += eps
            dn[i] -= eps
            fd = (loss({**inp, pname: up}) - loss({**inp, pname: dn})) / (2 * eps)
            an = float(g[gname][i])
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gname, i, fd, an)
    return g


def check_backward_fd_swiglu_renorm(seed=31):
    """Backward (reading: choice held fixed; gradient through the gates and
    through P of the aux loss) against central differences of the float64
    layer: SwiGLU, renormalised top-2, router bias, aux weight 0.7."""
    _fd_backward(seed, T=12, d=10, E=4, K=2, w=6, act=O.ACT_SWIGLU, gate=O.GATE_RENORM, daux=0.7)


def check_backward_fd_gelu_raw_capacity(seed=32):
    """GELU with biases, raw top-2 gates, a capacity that drops slots and a
    selection-only bias (whose gradient is 0)."""
    g = _fd_backward(seed, T=14, d=8, E=5, K=2, w=7, act=O.ACT_GELU, gate=O.GATE_RAW, daux=0.3, ffn_bias=True,
                     capacity=3, bias_select_only=True)
    assert not g["db_r"].any()


def check_backward_fd_switch_top1(seed=33):
    """Switch top-1 (raw p_i gate) with the aux loss, no router bias."""
    _fd_backward(seed, T=16, d=8, E=3, K=1, w=6, act=O.ACT_SWIGLU, gate=O.GATE_RAW, daux=1.0, bias=False)


def check_backward_dense_reduction(seed=34):
    """E = K = 1: the gate is 1 and aux is constant, so the layer is one dense
    FFN; its gradients equal torch autograd of that FFN in float64, and the
    router gets none."""
    T, d, w = 9, 6, 5
    for act in (O.ACT_SWIGLU, O.ACT_GELU):
        rng, inp = _bw_case(seed, T, d, 1, 1, w, act, bias=True, ffn_bias=(act == O.ACT_GELU))
        dy = rng.standard_normal((T, d))
        g = O.moe_backward(inp, T, d, 1, 1, act, O.GATE_RENORM, dy, daux=0.5)
        x = torch.tensor(inp["h"], requires_grad=True)
        W1 = torch.tensor(inp["W1"][0], requires_grad=True)
        W2 = torch.tensor(inp["W2"][0], requires_grad=True)
        if act == O.ACT_SWIGLU:
            W3 = torch.tensor(inp["W3"][0], requires_grad=True)
            y = (torch.nn.functional.silu(x @ W1.T) * (x @ W3.T)) @ W2.T
            ref_params = {"dW1": W1, "dW2": W2, "dW3": W3}
        else:
            b1 = torch.tensor(inp["b1"][0], requires_grad=True)
            b2 = torch.tensor(inp["b2"][0], requires_grad=True)
            y = torch.nn.functional.gelu(x @ W1.T + b1) @ W2.T + b2
            ref_params = {"dW1": W1, "dW2": W2, "db1": b1, "db2": b2}
        (y * torch.tensor(dy)).sum().backward()
        assert np.allclose(g["dh"], x.grad.numpy(), rtol=1e-12, atol=1e-12)
        for k, t in ref_params.items():
            assert np.allclose(g[k][0], t.grad.numpy(), rtol=1e-12, atol=1e-12), k
        assert not g["dW_r"].any() and not g["db_r"].any()


def check_noise_zero_and_bias_equivalence(seed=41):
    """Zero noise is the default path bit for bit; a noise that is the same
    per-expert vector for every token equals that router bias bit for bit
    (both are one float32 add after the logits), so choice, gates, P and the
    z-loss agree exactly."""
    T, d, E, K = 37, 24, 7, 2
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, d)).astype(np.float32)
    Wr = (rng.standard_normal((d, E)) * 0.3).astype(np.float32)
    b = (rng.standard_normal(E) * 0.5).astype(np.float32)
    base = {"h": h, "W_r": Wr, "b_r": None, "W1": rng.standard_normal((E, 8, d)), "W2": rng.standard_normal((E, d, 8)),
            "W3": rng.standard_normal((E, 8, d)), "b1": None, "b2": None}
    for gate in (O.GATE_RENORM, O.GATE_RAW):
        r0 = O.moe_forward(base, T, d, E, K, O.ACT_SWIGLU, gate)
        rz = O.moe_forward(base, T, d, E, K, O.ACT_SWIGLU, gate, noise=np.zeros((T, E), np.float32))
        assert np.array_equal(r0["logits"].view(np.uint32), rz["logits"].view(np.uint32))
        assert np.array_equal(r0["topk_gate"], rz["topk_gate"]) and r0["z_loss"] == rz["z_loss"]
        rb = O.moe_forward({**base, "b_r": b}, T, d, E, K, O.ACT_SWIGLU, gate)
        rn = O.moe_forward(base, T, d, E, K, O.ACT_SWIGLU, gate, noise=np.tile(b, (T, 1)))
        assert np.array_equal(rb["logits"].view(np.uint32), rn["logits"].view(np.uint32))
        assert np.array_equal(rb["topk_idx"], rn["topk_idx"])
        assert np.array_equal(rb["topk_gate"], rn["topk_gate"]) and np.array_equal(rb["probs"], rn["probs"])
        assert rb["z_loss"] == rn["z_loss"] and np.allclose(rb["y"], rn["y"], rtol=0, atol=0)


def check_noise_forcing(seed=42):
    """A noise of +1e4 on one expert per token picks that expert as the first
    choice of every token; with top-1 renormalised gates the gate is 1, with
    raw gates p of that expert is 1 to float64 rounding. With a
    selection-only bias the noise still reaches the gates (only the bias is
    choice-only)."""
    T, d, E = 29, 16, 5
    rng = np.random.default_rng(seed)
    inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
           "W_r": rng.standard_normal((d, E)).astype(np.float32), "b_r": rng.standard_normal(E).astype(np.float32),
           "W1": rng.standard_normal((E, 4, d)), "W2": rng.standard_normal((E, d, 4)),
           "W3": rng.standard_normal((E, 4, d)), "b1": None, "b2": None}
    want = rng.integers(0, E, T)
    noise = np.zeros((T, E), np.float32)
    noise[np.arange(T), want] = 1e4
    for gate, sel in ((O.GATE_RENORM, False), (O.GATE_RAW, False), (O.GATE_RAW, True)):
        r = O.moe_forward(inp, T, d, E, 1, O.ACT_SWIGLU, gate, noise=noise, bias_select_only=sel)
        assert np.array_equal(r["topk_idx"][:, 0], want)
        assert np.allclose(r["topk_gate"][:, 0], 1.0, rtol=0, atol=1e-12)
        assert np.allclose(r["probs"][np.arange(T), want], 1.0, rtol=0, atol=1e-12)


def check_z_loss_closed_forms(seed=43):
    """W_r = 0 and no bias: every logit is 0, log-sum-exp is ln E and the
    z-loss (ln E)^2; a per-token constant c_t (as noise) gives the mean of
    (ln E + c_t)^2; with E = 2 and bias (0, x) every token's log-sum-exp is
    log(1 + e^x), so the z-loss is log1p(exp(x))^2."""
    rng = np.random.default_rng(seed)
    T, d = 23, 12
    for E in (1, 2, 3, 8, 64):
        inp = {"h": rng.standard_normal((T, d)).astype(np.float32), "W_r": np.zeros((d, E), np.float32),
               "b_r": None, "W1": np.zeros((E, 4, d)), "W2": np.zeros((E, d, 4)), "W3": np.zeros((E, 4, d)),
               "b1": None, "b2": None}
        r = O.moe_forward(inp, T, d, E, 1, O.ACT_SWIGLU, O.GATE_RENORM)
        assert abs(r["z_loss"] - math.log(E) ** 2) <= 1e-13 * max(1.0, math.log(E) ** 2), (E, r["z_loss"])
        c = rng.integers(-8, 9, T).astype(np.float32) / 4  # exact in float32
        r = O.moe_forward(inp, T, d, E, 1, O.ACT_SWIGLU, O.GATE_RENORM, noise=np.repeat(c[:, None], E, axis=1))
        want = float(np.mean((math.log(E) + c.astype(np.float64)) ** 2))
        assert abs(r["z_loss"] - want) <= 1e-12 * max(1.0, want), (E, r["z_loss"], want)
    for x in (-3.0, 0.0, 0.75, 5.5):
        inp = {"h": rng.standard_normal((T, d)).astype(np.float32), "W_r": np.zeros((d, 2), np.float32),
               "b_r": np.array([0.0, x], np.float32), "W1": np.zeros((2, 4, d)), "W2": np.zeros((2, d, 4)),
               "W3": np.zeros((2, 4, d)), "b1": None, "b2": None}
        r = O.moe_forward(inp, T, d, 2, 1, O.ACT_SWIGLU, O.GATE_RENORM)
        assert abs(r["z_loss"] - math.log1p(math.exp(x)) ** 2) <= 1e-13 * max(1.0, r["z_loss"]), (x, r["z_loss"])


def check_z_loss_ignores_selection_bias(seed=45):
    """A bias that only steers the choice never reaches the softmax, so the
    z-loss is the same bits as without that bias (any bias vector, chosen to
    change the choice), while the same bias added to the logits changes it: the
    z-loss is taken on the logits the softmax sees, not on the choice scores."""
    rng = np.random.default_rng(seed)
    T, d, E = 31, 16, 6
    inp = {"h": rng.standard_normal((T, d)).astype(np.float32),
           "W_r": (rng.standard_normal((d, E)) * 0.3).astype(np.float32), "b_r": None,
           "W1": np.zeros((E, 4, d)), "W2": np.zeros((E, d, 4)), "W3": np.zeros((E, 4, d)), "b1": None, "b2": None}
    r0 = O.moe_forward(inp, T, d, E, 2, O.ACT_SWIGLU, O.GATE_RENORM)
    b = (rng.standard_normal(E) * 3).astype(np.float32)
    sel = O.moe_forward(dict(inp, b_r=b), T, d, E, 2, O.ACT_SWIGLU, O.GATE_RENORM, bias_select_only=True)
    lgt = O.moe_forward(dict(inp, b_r=b), T, d, E, 2, O.ACT_SWIGLU, O.GATE_RENORM)
    assert not np.array_equal(sel["topk_idx"], r0["topk_idx"]), "the bias should change the choice"
    assert sel["z_loss"] == r0["z_loss"], (sel["z_loss"], r0["z_loss"])
    assert lgt["z_loss"] != r0["z_loss"]


def check_backward_fd_zloss_noise(seed=44):
    """The z-loss gradient and a noisy router: central differences of
    sum(dy y) + daux aux + dz z_loss, with noise on the logits (held fixed:
    an input, not a parameter) — SwiGLU, renormalised top-2, router bias."""
    _fd_backward(seed, T=12, d=10, E=4, K=2, w=6, act=O.ACT_SWIGLU, gate=O.GATE_RENORM, daux=0.4, dz=0.8,
                 noise_scale=0.3)
    _fd_backward(seed + 1, T=10, d=8, E=5, K=1, w=6, act=O.ACT_GELU, gate=O.GATE_RAW, daux=0.0, dz=1.5,
                 noise_scale=0.5, ffn_bias=True, bias_select_only=True)


ALL_CHECKS = [check_router_logits_exact, check_router_logits_bound, check_topk_bruteforce,
              check_probs, check_gates_worked_example, check_gates_invariants,
              check_combine_worked_example, check_permutation_sorted, check_load_stats_page,
              check_aux_uniform_probs, check_aux_uniform_load, check_dense_reduction,
              check_soft_mixture_K_equals_E, check_forward_subset_consistency, check_param_counts,
              check_capacity_widget, check_capacity_order, check_capacity_slots_rounding,
              check_capacity_layer, check_bias_select_only, check_backward_fd_swiglu_renorm,
              check_backward_fd_gelu_raw_capacity, check_backward_fd_switch_top1, check_backward_dense_reduction,
              check_noise_zero_and_bias_equivalence, check_noise_forcing, check_z_loss_closed_forms,
              check_z_loss_ignores_selection_bias,
              check_backward_fd_zloss_noise]
