"""Plant plausible mistakes in the oracle and require that the pins catch each one.

Every mutation is applied to the oracle module on the CPU only (monkeypatch);
the pins of tests/oracle_pins.py must then fail at least once.
"""
import numpy as np
import pytest

import oracle_pins
from oracle import moe_oracle as O

_orig = {name: getattr(O, name) for name in
         ("moe_forward", "gelu_grad", "silu_grad", "gate_logit_grad", "router_logits_f32", "select_topk", "router_probs", "gates", "stable_permutation",
          "aux_loss", "gelu", "silu", "expert_ffn", "combine", "param_counts_micro",
          "param_counts_swiglu_model", "expert_counts", "capacity_keep", "capacity_slots", "drop_stats",
          "z_loss", "z_loss_logit_grad")}


def _logits_no_bias(h, W, b):
    return _orig["router_logits_f32"](h, W, None)


def _logits_reverse_k(h, W, b):
    h = np.ascontiguousarray(np.asarray(h, np.float32)[:, ::-1])
    W = np.ascontiguousarray(np.asarray(W, np.float32)[::-1, :])
    return _orig["router_logits_f32"](h, W, b)


def _logits_bias_first(h, W, b):
    # bias folded in at the start of the chain instead of added at the end
    if b is None:
        return _orig["router_logits_f32"](h, W, None)
    h = np.asarray(h, np.float32)
    h1 = np.concatenate([np.ones((h.shape[0], 1), np.float32), h], axis=1)
    W1 = np.concatenate([np.asarray(b, np.float32)[None, :], np.asarray(W, np.float32)], axis=0)
    return _orig["router_logits_f32"](h1, W1, None)


def _logits_single_chain(h, W, b):
    # one sequential chain per logit instead of four interleaved chains
    h = np.asarray(h, np.float32).astype(np.float64)
    W = np.asarray(W, np.float32).astype(np.float64)
    acc = np.zeros((h.shape[0], W.shape[1]), np.float32)
    for k in range(h.shape[1]):
        acc = (acc.astype(np.float64) + np.outer(h[:, k], W[k])).astype(np.float32)
    if b is not None:
        acc = acc + np.asarray(b, np.float32)[None, :]
    return acc


def _logits_pairs_swapped(h, W, b):
    # (c0 + c2) + (c1 + c3): relabel the groups of chains 1 and 2
    h = np.asarray(h, np.float32)
    d = h.shape[1]
    k = np.arange(d)
    g, j = k // 4, (k // 4) % 4
    partner = g - j + np.where(j == 1, 2, np.where(j == 2, 1, j))
    src = np.where(4 * partner < d, 4 * partner + k % 4, k)  # a group without partner stays
    return _orig["router_logits_f32"](np.ascontiguousarray(h[:, src]),
                                      np.ascontiguousarray(np.asarray(W, np.float32)[src, :]), b)


def _forward_bias_everywhere(*a, bias_select_only=False, **kw):
    # the selection-only flag ignored: gates and P see the bias too
    return _orig["moe_forward"](*a, **kw)


def _forward_bias_ignored(inp, *a, bias_select_only=False, **kw):
    # the selection-only flag drops the bias altogether
    if bias_select_only:
        inp = {**inp, "b_r": None}
    return _orig["moe_forward"](inp, *a, **kw)


def _silu_grad_sigmoid_only(z):
    return 1.0 / (1.0 + np.exp(-z))


def _gelu_grad_cdf_only(z):
    return 0.5 * (1.0 + O._erf(z / np.sqrt(2.0)))


def _gate_grad_no_centering(gl, idx, g, p, dg, gate, daux, f):
    # renormalised gates: g * dg instead of g * (dg - sum g dg)
    out = _orig["gate_logit_grad"](gl, idx, g, p, dg, gate, daux, f)
    if gate == O.GATE_RENORM:
        T = gl.shape[0]
        fix = np.zeros_like(out)
        sdot = np.sum(g * dg, axis=1, keepdims=True)
        np.add.at(fix, (np.broadcast_to(np.arange(T)[:, None], idx.shape), idx), g * sdot)
        out = out + fix
    return out


def _gate_grad_aux_without_E(gl, idx, g, p, dg, gate, daux, f):
    return _orig["gate_logit_grad"](gl, idx, g, p, dg, gate, daux / gl.shape[1], f)


def _topk_high_index_wins(l, K):
    E = l.shape[1]
    idx = _orig["select_topk"](l[:, ::-1], K)
    return (E - 1 - idx).astype(np.int32)


def _topk_smallest(l, K):
    return _orig["select_topk"](-np.asarray(l), K)


def _gates_no_renorm(l, idx, mode):
    return np.take_along_axis(_orig["router_probs"](l), idx.astype(np.int64), axis=1)


def _probs_wrong_sign(l):
    l = np.asarray(l, np.float64)
    ex = np.exp(l.min(axis=1, keepdims=True) - l)
    return ex / ex.sum(axis=1, keepdims=True)


def _perm_token_descending(idx, E):
    T, K = idx.shape
    off, st, ts = _orig["stable_permutation"](idx[::-1].copy(), E)
    st = (T - 1 - st).astype(np.int32)
    ts = ts[::-1].copy()
    return off, st, ts


def _aux_missing_K(counts, p, K):
    return _orig["aux_loss"](counts, p, 1)


def _aux_missing_E(counts, p, K):
    return _orig["aux_loss"](counts, p, K) / p.shape[1]


def _aux_sum_not_mean(counts, p, K):
    return _orig["aux_loss"](counts, p, K) * p.shape[0]


def _gelu_tanh(z):
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def _ffn_silu_on_w3(x, e, params, act):
    if act != O.ACT_SWIGLU:
        return _orig["expert_ffn"](x, e, params, act)
    x = np.asarray(x, np.float64)
    W1, W3, W2 = (np.asarray(params[k][e], np.float64) for k in ("W1", "W3", "W2"))
    return ((x @ W1.T) * O.silu(x @ W3.T)) @ W2.T


def _ffn_no_b2(x, e, params, act):
    p = dict(params)
    p["b2"] = None
    return _orig["expert_ffn"](x, e, p, act)


def _combine_swapped(o, ts, g):
    return _orig["combine"](o, ts, g[:, ::-1])


def _micro_three_matrices(d, layers, E, K, width):
    c = _orig["param_counts_micro"](d, layers, E, K, width)
    extra = layers * d * width
    return {"total": c["total"] + E * extra, "active": c["active"] + K * extra,
            "attention_plus_active_experts": c["attention_plus_active_experts"] + K * extra}


def _swiglu_two_matrices(d, layers, E, K, width, vocab=32000):
    c = _orig["param_counts_swiglu_model"](d, layers, E, K, width, vocab)
    e2 = 2 * d * width
    shared = c["total"] - c["routed_total"]
    return {"expert": e2, "total": shared + layers * E * e2, "active": shared + layers * K * e2,
            "routed_total": layers * E * e2}


def _counts_off_by_one(idx, E):
    c = _orig["expert_counts"](idx, E).copy()
    if len(c):
        c[0] += 1
    return c


def _keep_later_tokens_win(idx, E, C):
    # slots taken from the last token backwards
    return _orig["capacity_keep"](idx[::-1].copy(), E, C)[::-1].copy()


def _keep_off_by_one(idx, E, C):
    return _orig["capacity_keep"](idx, E, C + 1)


def _capacity_floor(factor, T, K, E):
    from fractions import Fraction
    return int(Fraction(str(factor)) * T * K / E)


def _drop_stats_over_T(counts, C):
    st = _orig["drop_stats"](counts, C)
    return {"dropped": st["dropped"], "percent": 100.0 * st["dropped"] / max(int(sum(counts)) // 2, 1)}


def _zloss_not_squared(gl):
    return float(np.mean(O.logsumexp_rows(gl))) if gl.shape[0] else 0.0


def _zloss_sum_not_mean(gl):
    return float(np.sum(O.logsumexp_rows(gl) ** 2))


def _zloss_grad_factor_one(gl, p):
    return 0.5 * _orig["z_loss_logit_grad"](gl, p)


def _forward_noise_ignored(*a, noise=None, **kw):
    return _orig["moe_forward"](*a, **kw)


def _forward_noise_selection_only(inp, T, d, E, K, act, gate, *a, noise=None, **kw):
    # the noise steers the choice but the gates and P come from noise-free logits
    r = _orig["moe_forward"](inp, T, d, E, K, act, gate, *a, noise=noise, **kw)
    if noise is None:
        return r
    r0 = _orig["moe_forward"](inp, T, d, E, K, act, gate, *a, **kw)
    r["topk_gate"] = O.gates(r0["gate_logits"], r["topk_idx"], gate)
    r["probs"] = O.router_probs(r0["gate_logits"])
    return r


def _forward_zloss_on_choice_scores(*a, **kw):
    # the z-loss taken on the scores the choice is made on (bias included even
    # when it only steers the choice) instead of the softmax's logits
    r = _orig["moe_forward"](*a, **kw)
    r["z_loss"] = _orig["z_loss"](np.asarray(r["logits"], np.float64))
    return r


MUTATIONS = {
    "zloss_on_choice_scores": ("moe_forward", _forward_zloss_on_choice_scores),
    "zloss_not_squared": ("z_loss", _zloss_not_squared),
    "zloss_sum_not_mean": ("z_loss", _zloss_sum_not_mean),
    "zloss_grad_factor_one": ("z_loss_logit_grad", _zloss_grad_factor_one),
    "noise_ignored": ("moe_forward", _forward_noise_ignored),
    "noise_selection_only": ("moe_forward", _forward_noise_selection_only),
    "capacity_later_tokens_win": ("capacity_keep", _keep_later_tokens_win),
    "capacity_off_by_one": ("capacity_keep", _keep_off_by_one),
    "capacity_rounded_down": ("capacity_slots", _capacity_floor),
    "drop_percent_of_tokens": ("drop_stats", _drop_stats_over_T),
    "router_drops_bias": ("router_logits_f32", _logits_no_bias),
    "router_reverse_k_order": ("router_logits_f32", _logits_reverse_k),
    "router_bias_first": ("router_logits_f32", _logits_bias_first),
    "select_bias_reaches_gates": ("moe_forward", _forward_bias_everywhere),
    "select_bias_ignored": ("moe_forward", _forward_bias_ignored),
    "backward_silu_grad_sigmoid_only": ("silu_grad", _silu_grad_sigmoid_only),
    "backward_gelu_grad_cdf_only": ("gelu_grad", _gelu_grad_cdf_only),
    "backward_renorm_not_centred": ("gate_logit_grad", _gate_grad_no_centering),
    "backward_aux_without_E": ("gate_logit_grad", _gate_grad_aux_without_E),
    "router_single_chain": ("router_logits_f32", _logits_single_chain),
    "router_pairs_swapped": ("router_logits_f32", _logits_pairs_swapped),
    "topk_high_index_wins_ties": ("select_topk", _topk_high_index_wins),
    "topk_smallest": ("select_topk", _topk_smallest),
    "gates_not_renormalised": ("gates", _gates_no_renorm),
    "softmax_wrong_sign": ("router_probs", _probs_wrong_sign),
    "permutation_tokens_descending": ("stable_permutation", _perm_token_descending),
    "aux_f_over_T": ("aux_loss", _aux_missing_K),
    "aux_missing_E": ("aux_loss", _aux_missing_E),
    "aux_sum_not_mean": ("aux_loss", _aux_sum_not_mean),
    "gelu_tanh_approx": ("gelu", _gelu_tanh),
    "swiglu_silu_on_w3": ("expert_ffn", _ffn_silu_on_w3),
    "expert_drops_b2": ("expert_ffn", _ffn_no_b2),
    "combine_swaps_gates": ("combine", _combine_swapped),
    "micro_counts_three_matrices": ("param_counts_micro", _micro_three_matrices),
    "swiglu_counts_two_matrices": ("param_counts_swiglu_model", _swiglu_two_matrices),
    "counts_off_by_one": ("expert_counts", _counts_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # an assertion, or a crash caused by the planted mistake
            failed.append((check.__name__, type(exc).__name__))
    assert failed, "mutation %s slipped past every pin" % name
