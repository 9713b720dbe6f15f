"""CPU oracle for the forward pass of one top-K routed mixture-of-experts FFN layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product library never calls it and
shares no code with it: the HIP path and this oracle have only the seeded input
generator in common.

Plain, slow, obviously correct. Everything after the router logits is float64
(numpy matmul serves as the library primitive). The router logits are float32
in the canonical order of four interleaved fmaf chains (router_fp32.c), because the router is
kept in float32 (Arjun Jaggi, "Mixture of Experts in LLMs: How Sparse Models
Scale", section "Switch Transformers") and the expert choice must agree bit
for bit with any implementation that follows the same order.

Page references (title, site, section):
  [MTA]   "Mixture of Experts", maptheai.com tutorial
  [GLO]   "Mixture of Experts (MoE)", ai-and-cloud.com glossary
  [CUR]   "Mixture of Experts.", llm.curionode.com, Vol. VII Plate 4
  [LENSA] "Mixture of Experts", Lensa ML explainer (Steps 1-6, FAQ)
  [AJ]    "Mixture of Experts in LLMs: How Sparse Models Scale", arjunjaggi.com

Function -> passage it follows -> what pins it (tests/test_oracle_pins.py):
  router_logits_f32   [LENSA] Step 2; [CUR] "Parameters you hold..." (linear
                      router + softmax); [AJ] "Switch Transformers" (float32)
                      -> exact correctly-rounded fma chains and sums
                         recomputed with rational arithmetic; float64
                         error bound.
  select_topk         [MTA] "The mechanism"; [LENSA] Step 3 (top-k)
                      -> brute force over all K-subsets, with ties.
  router_probs        [LENSA] Step 2 (softmax over experts)
                      -> sums to 1; the page's illustrative distribution.
  gates               [LENSA] Step 3 (softmax over the chosen logits; the
                      Mixtral formula; Switch scales by p_i)
                      -> the page's worked gates 0.61 / 0.39; sum to 1.
  expert_counts,
  stable_permutation  [LENSA] Step 4 (T*K routing slots counted per expert);
                      Step 5 (experts that take any number of tokens)
                      -> Python's stable sorted(); the page's histogram stats.
  expert_ffn          [LENSA] Step 1 (each expert is a full FFN, 3 x d x w);
                      [CUR] intro (E separate MLPs)
                      -> E=1, K=1 equals a dense FFN built from torch's own
                         gelu/silu and matmul.
  combine             [MTA] "The mechanism"; [LENSA] Step 3 (y = sum g E(h))
                      -> the page's worked 4-dim example.
  aux_loss            [LENSA] Step 4 (E * sum f * P; equals 1 when routing is
                      uniform) -> uniform-P and uniform-f closed forms.
  capacity_slots,
  capacity_keep,
  drop_stats          [LENSA] Step 5 (C = factor x tokens x k / E slots per
                      expert; slots past C are skipped; a token with no
                      expert keeps its residual)
                      -> the page's C = 64 and 94 dropped slots (18.4 %);
                         a sort-based restatement of "first C in token order"
                         on small random routings; C >= T equals the dropless
                         layer; C = 0 gives y = 0.
  moe_forward(bias_select_only=True)
                      [LENSA] Step 4 (DeepSeek-V3 steers the load with a
                      per-expert routing bias instead of the aux loss) and
                      the summary (a routing bias keeps the load even): the
                      bias enters the top-K choice only; softmax, gates and
                      P use the unbiased logits (reading: the pages do not
                      say what the gates see)
                      -> zero bias equals the default path; the choice is the
                         brute-force top-K of logits + bias; gates and P do
                         not move with a bias that leaves the choice alone; a
                         forcing bias picks its expert for every token with
                         the unbiased gate ratio.
  moe_forward(noise=...)
                      [AJ] "Load Balancing" (Shazeer's noisy top-K: tuned
                      Gaussian noise on the router logits; the pages give no
                      scale or form). Reading: the caller draws the noise and
                      passes it, already scaled, as a [T][E] float32 input;
                      it is added to the logits after the bias (a separate
                      float32 add) and enters the choice, the gates and P
                      -> zero noise equals the default path bit for bit; a
                         per-expert constant noise equals that router bias
                         bit for bit; a forcing noise picks its expert.
  z_loss              [AJ] "Mixtral and the Open MoE Era" (ST-MoE's router
                      z-loss, a penalty on large router logits; the formula
                      is not on the pages). Reading: the ST-MoE form, the mean
                      over tokens of the squared log-sum-exp of the logits
                      the softmax sees
                      -> uniform logits give (ln E)^2 exactly; a per-token
                         shift c moves each term to (lse + c)^2; the gradient
                         2 lse p / T by central differences.
  param_counts        [CUR] "Parameters you hold..."; [LENSA] Steps 1 and 6
                      -> the printed 4.46M / 1.32M / 3.39x / 25.2x,
                         37.0B / 11.1B / 3.3x and 176M / 45.1B.
"""
from __future__ import annotations

import ctypes
import math
import os
from fractions import Fraction
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

ACT_GELU = 0
ACT_SWIGLU = 1
GATE_RENORM = 0
GATE_RAW = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_router.so")
_SRC_PATH = os.path.join(_HERE, "router_fp32.c")
_lib = None


def build(force: bool = False) -> str:
    """Compile router_fp32.c with gcc (no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-shared", "-fPIC", _SRC_PATH, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_router_logits_f32.restype = None
        lib.oracle_router_logits_f32.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------- router

def router_logits_f32(h32: np.ndarray, W_r: np.ndarray, b_r: Optional[np.ndarray]) -> np.ndarray:
    """logit[t,e] = (h . W_r)[t,e] (+ b_r[e]) in float32, canonical fmaf order ([LENSA] Step 2)."""
    h32 = np.ascontiguousarray(h32, dtype=np.float32)
    W_r = np.ascontiguousarray(W_r, dtype=np.float32)
    T, d = h32.shape
    d2, E = W_r.shape
    assert d == d2
    out = np.empty((T, E), dtype=np.float32)
    if b_r is not None:
        b_r = np.ascontiguousarray(b_r, dtype=np.float32)
        assert b_r.shape == (E,)
    if T > 0:
        _load().oracle_router_logits_f32(h32.ctypes.data, W_r.ctypes.data,
                                         None if b_r is None else b_r.ctypes.data,
                                         T, d, E, out.ctypes.data)
    return out


def router_logits_f64(h: np.ndarray, W_r: np.ndarray, b_r: Optional[np.ndarray]) -> np.ndarray:
    """The same logits in float64 (used only to bound the float32 rounding)."""
    l = np.asarray(h, np.float64) @ np.asarray(W_r, np.float64)
    if b_r is not None:
        l = l + np.asarray(b_r, np.float64)[None, :]
    return l


def select_topk(logits: np.ndarray, K: int) -> np.ndarray:
    """The K chosen experts per token, largest logit first; equal logits: lower index first.

    Selecting on the logits is the same as selecting on the softmax
    probabilities, since the softmax is increasing ([LENSA] Step 3).
    """
    T, E = logits.shape
    idx = np.empty((T, K), dtype=np.int32)
    experts = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> logit descending, then expert ascending
        order = np.lexsort((experts, -logits[t].astype(np.float64)))
        idx[t] = order[:K]
    return idx


def router_probs(logits: np.ndarray) -> np.ndarray:
    """p[t,e] = softmax over all E experts of the logits, in float64 ([LENSA] Step 2)."""
    l = np.asarray(logits, np.float64)
    m = l.max(axis=1, keepdims=True)
    ex = np.exp(l - m)
    return ex / ex.sum(axis=1, keepdims=True)


def gates(logits: np.ndarray, idx: np.ndarray, mode: int) -> np.ndarray:
    """Gate weight of each chosen expert ([LENSA] Step 3).

    RENORM: a softmax over the K chosen logits only (the Mixtral form
            softmax(TopK(h W_g))), so the K gates sum to 1.
    RAW:    the full-softmax probability p_i of the chosen expert, not
            renormalised (Switch top-1).
    """
    l = np.asarray(logits, np.float64)
    chosen = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    if mode == GATE_RENORM:
        ex = np.exp(chosen - chosen[:, :1])
        return ex / ex.sum(axis=1, keepdims=True)
    if mode == GATE_RAW:
        return np.take_along_axis(router_probs(logits), idx.astype(np.int64), axis=1)
    raise ValueError(mode)


# ----------------------------------------------------------------------------- grouping

def expert_counts(idx: np.ndarray, E: int) -> np.ndarray:
    """Routing slots per expert: T*K slots in all ([LENSA] Step 4)."""
    return np.bincount(idx.reshape(-1).astype(np.int64), minlength=E).astype(np.int32)


def stable_permutation(idx: np.ndarray, E: int):
    """Group the T*K slots by expert, keeping token order inside each group.

    Returns (offsets[E+1], slot_token[S], token_slot[T,K]): group e occupies
    rows offsets[e] .. offsets[e+1]-1; row s holds token slot_token[s]; the
    j-th choice of token t sits in row token_slot[t, j].
    """
    T, K = idx.shape
    counts = expert_counts(idx, E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    tok = np.repeat(np.arange(T, dtype=np.int64), K)
    ch = np.tile(np.arange(K, dtype=np.int64), T)
    ex = idx.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, ex))  # primary: expert, then token (stable)
    slot_token = tok[order].astype(np.int32)
    token_slot = np.empty((T, K), dtype=np.int32)
    token_slot[tok[order], ch[order]] = np.arange(T * K, dtype=np.int32)
    return offsets, slot_token, token_slot


# ----------------------------------------------------------------------------- experts

def gelu(z: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU."""
    return 0.5 * z * (1.0 + _erf(z / np.sqrt(2.0)))


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, e: int, params: Dict[str, Optional[np.ndarray]], act: int) -> np.ndarray:
    """Expert e's feed-forward block on rows x, float64 ([LENSA] Step 1; [CUR] intro).

    Stored weights are output-major: params["W1"][e] is width x d, i.e. the
    transpose of the d x width matrix of the math, so x . W1 = x @ W1[e].T.
      GELU:   o = GELU(x W1 + b1) W2 + b2
      SwiGLU: o = (SiLU(x W1) * (x W3)) W2     (three d x width matrices, no bias)
    """
    x = np.asarray(x, np.float64)
    W1 = np.asarray(params["W1"][e], np.float64)
    W2 = np.asarray(params["W2"][e], np.float64)
    if act == ACT_GELU:
        z = x @ W1.T
        if params.get("b1") is not None:
            z = z + np.asarray(params["b1"][e], np.float64)
        o = gelu(z) @ W2.T
        if params.get("b2") is not None:
            o = o + np.asarray(params["b2"][e], np.float64)
        return o
    if act == ACT_SWIGLU:
        W3 = np.asarray(params["W3"][e], np.float64)
        return (silu(x @ W1.T) * (x @ W3.T)) @ W2.T
    raise ValueError(act)


def combine(o: np.ndarray, token_slot: np.ndarray, g: np.ndarray) -> np.ndarray:
    """y[t] = sum_j g[t,j] * o[token_slot[t,j]] ([MTA] "The mechanism"; [LENSA] Step 3)."""
    T, K = token_slot.shape
    y = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(K):
        y += g[:, j:j + 1] * o[token_slot[:, j]]
    return y


def aux_loss(counts: np.ndarray, p: np.ndarray, K: int) -> float:
    """E * sum_e f_e * P_e ([LENSA] Step 4).

    f_e = share of the T*K routing slots that go to expert e;
    P_e = mean over tokens of the full-softmax probability of expert e.
    """
    T, E = p.shape
    if T == 0:
        return 0.0
    f = np.asarray(counts, np.float64) / float(T * K)
    P = p.mean(axis=0)
    return float(E * np.sum(f * P))


# ----------------------------------------------------------------------------- capacity

def capacity_slots(factor, T: int, K: int, E: int) -> int:
    """Slots per expert, C = factor * T * K / E ([LENSA] Step 5), rounded up
    when fractional (the page prints only integer cases; rounding up keeps
    C * E >= factor * T * K). The factor is read as the decimal it is written as."""
    return int(math.ceil(Fraction(str(factor)) * T * K / E))


def capacity_keep(idx: np.ndarray, E: int, C: int) -> np.ndarray:
    """Which routing slots are processed when every expert has C slots ([LENSA] Step 5).

    Tokens are taken in order; each of a token's choices fills a free slot of
    its expert or is dropped. (A token never picks one expert twice, so the
    order of its K choices does not matter.)
    """
    T, K = idx.shape
    keep = np.zeros((T, K), dtype=bool)
    used = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(K):
            e = int(idx[t, j])
            if used[e] < C:
                keep[t, j] = True
                used[e] += 1
    return keep


def drop_stats(counts: Sequence[int], C: int) -> Dict[str, float]:
    """Dropped slots and their share when every expert has C slots ([LENSA] Step 5)."""
    c = np.asarray(counts, np.int64)
    dropped = int(np.maximum(c - C, 0).sum())
    return {"dropped": dropped, "percent": 100.0 * dropped / max(int(c.sum()), 1)}


# ----------------------------------------------------------------------------- layer

def moe_forward(inp: Dict[str, Optional[np.ndarray]], T: int, d: int, E: int, K: int,
                act: int, gate: int, tokens: Optional[Sequence[int]] = None,
                capacity: Optional[int] = None, bias_select_only: bool = False,
                logits_f64: bool = False, noise: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The whole layer. `inp` holds float32 arrays of the exact input values.

    Routing, grouping and the aux loss cover all T tokens. The expert FFNs and
    y are computed for all tokens, or only for the rows listed in `tokens`
    (y then has len(tokens) rows, in that order).

    capacity: slots per expert ([LENSA] Step 5), or None for dropless. Dropped
    slots contribute nothing; kept slots keep their gates; a token with every
    slot dropped has y = 0 (the layer adds nothing to its residual). Counts and
    the aux loss describe the router's choices, before any drop.

    bias_select_only: the router bias b_r steers only which experts are chosen
    ([LENSA] Step 4: a per-expert routing bias in place of the aux loss); the
    probabilities, the gates and P come from the unbiased logits h W_r.
    Otherwise b_r is part of the logits everywhere.

    logits_f64: router logits in float64 instead of the float32 contract (a
    smooth function of the inputs, for finite-difference checks of the
    backward pass).

    noise: [T][E] values added to the logits after the bias (noisy top-K;
    drawn and scaled by the caller), in the logits' precision; they enter the
    choice, the gates and P (with bias_select_only too: only the bias is
    choice-only).

    Also returns z_loss: mean over tokens of (log sum_e exp gate_logits)^2.
    """
    h32 = np.asarray(inp["h"], np.float32).reshape(T, d)
    router = router_logits_f64 if logits_f64 else router_logits_f32
    hin = np.asarray(inp["h"], np.float64).reshape(T, d) if logits_f64 else h32
    logits = router(hin, inp["W_r"], inp.get("b_r"))  # the scores the choice is made on
    if bias_select_only and inp.get("b_r") is not None:
        gate_logits = router(hin, inp["W_r"], None)
    else:
        gate_logits = logits
    if noise is not None:
        nz = np.asarray(noise, logits.dtype).reshape(T, E)
        same = gate_logits is logits
        logits = logits + nz           # one rounding in the logits' precision, after the bias
        gate_logits = logits if same else gate_logits + nz
    idx = select_topk(logits, K)
    p = router_probs(gate_logits)
    g = gates(gate_logits, idx, gate)
    counts = expert_counts(idx, E)
    offsets, slot_token, token_slot = stable_permutation(idx, E)
    aux = aux_loss(counts, p, K)
    zl = z_loss(gate_logits)
    keep = np.ones((T, K), dtype=bool) if capacity is None else capacity_keep(idx, E, capacity)
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = np.zeros((len(rows), d), dtype=np.float64)
    h64 = np.asarray(inp["h"], np.float64).reshape(T, d) if logits_f64 else h32.astype(np.float64)
    for e in range(E):
        sel_r, sel_j = np.nonzero((idx[rows] == e) & keep[rows])
        if len(sel_r) == 0:
            continue
        o = expert_ffn(h64[rows[sel_r]], e, inp, act)
        # y[t] += g[t,j] * E_e(h[t]); each token meets each expert at most once
        y[sel_r] += g[rows[sel_r], sel_j][:, None] * o
    return {"logits": logits, "gate_logits": gate_logits, "topk_idx": idx, "topk_gate": g, "probs": p,
            "counts": counts,
            "offsets": offsets, "slot_token": slot_token, "token_slot": token_slot,
            "token_slot_kept": np.where(keep, token_slot, -1).astype(np.int32), "keep": keep,
            "aux": aux, "z_loss": zl, "y": y, "rows": rows}


def logsumexp_rows(l: np.ndarray) -> np.ndarray:
    """log sum_e exp l[t, e] per row, float64, shifted by the row maximum."""
    l = np.asarray(l, np.float64)
    m = l.max(axis=1)
    return m + np.log(np.exp(l - m[:, None]).sum(axis=1))


def z_loss(gate_logits: np.ndarray) -> float:
    """Router z-loss (ST-MoE form): the mean over tokens of the squared
    log-sum-exp of the logits the softmax sees."""
    if gate_logits.shape[0] == 0:
        return 0.0
    return float(np.mean(logsumexp_rows(gate_logits) ** 2))


# ----------------------------------------------------------------------------- backward

def z_loss_logit_grad(gate_logits: np.ndarray, p: np.ndarray) -> np.ndarray:
    """d z_loss / d gate_logits: the derivative of lse_t^2 is 2 lse_t times
    the softmax of row t; the mean over T tokens divides by T."""
    T = gate_logits.shape[0]
    return (2.0 / T) * logsumexp_rows(gate_logits)[:, None] * p


def gelu_grad(z: np.ndarray) -> np.ndarray:
    """d GELU / dz = Phi(z) + z phi(z) (exact GELU; Phi, phi: normal cdf and density)."""
    return 0.5 * (1.0 + _erf(z / np.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d SiLU / dz = s (1 + z (1 - s)), s = sigmoid(z)."""
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def gate_logit_grad(gl: np.ndarray, idx: np.ndarray, g: np.ndarray, p: np.ndarray, dg: np.ndarray,
                    gate: int, daux: float, f: np.ndarray) -> np.ndarray:
    """d loss / d gate logits, given d loss / d gates (dg) and the aux weight.

    The choice itself passes no gradient ([MTA] "The difficulties": top-k is
    not differentiable, the router learns through the weights of the chosen
    experts). RENORM: g = softmax over the chosen logits, so
    dl[c_j] = g_j (dg_j - sum_i g_i dg_i). RAW: g_j = p[c_j] of the full
    softmax ([LENSA] Step 3: the gradient reaches the router through p_i).
    aux = E sum_e f_e P_e with P_e = mean_t p[t, e]; only P is differentiable
    ([LENSA] Step 4), d aux / d p[t, e] = E f_e / T.
    """
    T, E = gl.shape
    dl = np.zeros((T, E))
    dp = np.zeros((T, E))
    rows = np.arange(T)[:, None]
    if gate == GATE_RENORM:
        sdot = np.sum(g * dg, axis=1, keepdims=True)
        np.add.at(dl, (np.broadcast_to(rows, idx.shape), idx), g * (dg - sdot))
    elif gate == GATE_RAW:
        np.add.at(dp, (np.broadcast_to(rows, idx.shape), idx), dg)
    else:
        raise ValueError(gate)
    if daux != 0.0 and T > 0:
        dp = dp + daux * E * np.asarray(f, np.float64)[None, :] / T
    return dl + p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def moe_backward(inp: Dict[str, Optional[np.ndarray]], T: int, d: int, E: int, K: int, act: int, gate: int,
                 dy: np.ndarray, daux: float = 0.0, capacity: Optional[int] = None,
                 bias_select_only: bool = False, logits_f64: bool = False,
                 with_scales: bool = False, noise: Optional[np.ndarray] = None,
                 dz_loss: float = 0.0) -> Dict[str, Optional[np.ndarray]]:
    """Gradients of loss = sum(dy * y) + daux * aux + dz_loss * z_loss with respect
    to every input of the layer, float64 (reading: the expert choice and the
    capacity drops are held fixed; see gate_logit_grad for the router; the
    noise is an input, not differentiated).

    Returns dh [T][d], dW_r [d][E], db_r [E] (zero when the bias only steers
    the choice; None without a bias), and per expert dW1, dW3 (SwiGLU), dW2 in
    the stored layouts and db1, db2 (GELU with biases; else None).

    with_scales: also "scale", the same sums taken over the absolute values of
    their terms (|do|^T |a| for dW2, and so on): the size against which the
    rounding error of an implementation's sum is judged.
    """
    fwd = moe_forward(inp, T, d, E, K, act, gate, capacity=capacity, bias_select_only=bias_select_only,
                      logits_f64=logits_f64, noise=noise)
    idx, g, p, keep = fwd["topk_idx"], fwd["topk_gate"], fwd["probs"], fwd["keep"]
    h = np.asarray(inp["h"], np.float64).reshape(T, d)
    dy = np.asarray(dy, np.float64).reshape(T, d)
    W1 = [np.asarray(inp["W1"][e], np.float64) for e in range(E)]
    W2 = [np.asarray(inp["W2"][e], np.float64) for e in range(E)]
    W3 = [np.asarray(inp["W3"][e], np.float64) for e in range(E)] if act == ACT_SWIGLU else None
    b1 = inp.get("b1") if act == ACT_GELU else None
    b2 = inp.get("b2") if act == ACT_GELU else None
    out = {"dh": np.zeros((T, d)), "dW1": np.zeros((E,) + W1[0].shape), "dW2": np.zeros((E,) + W2[0].shape),
           "dW3": None if W3 is None else np.zeros((E,) + W3[0].shape),
           "db1": None if b1 is None else np.zeros((E, W1[0].shape[0])),
           "db2": None if b2 is None else np.zeros((E, d))}
    dg = np.zeros((T, K))
    sc = {k: (None if v is None else np.zeros_like(v)) for k, v in out.items()}
    for e in range(E):
        st, sj = np.nonzero((idx == e) & keep)
        if len(st) == 0:
            continue
        x = h[st]
        if act == ACT_GELU:
            z = x @ W1[e].T
            if b1 is not None:
                z = z + np.asarray(b1[e], np.float64)
            a = gelu(z)
        else:
            z1, z3 = x @ W1[e].T, x @ W3[e].T
            a = silu(z1) * z3
        o = a @ W2[e].T
        if b2 is not None:
            o = o + np.asarray(b2[e], np.float64)
        do = g[st, sj][:, None] * dy[st]           # y[t] = sum_j g[t, j] o_j
        dg[st, sj] = np.sum(dy[st] * o, axis=1)
        out["dW2"][e] = do.T @ a
        if b2 is not None:
            out["db2"][e] = do.sum(axis=0)
        da = do @ W2[e]
        if act == ACT_GELU:
            dz = da * gelu_grad(z)
            out["dW1"][e] = dz.T @ x
            if b1 is not None:
                out["db1"][e] = dz.sum(axis=0)
            dx = dz @ W1[e]
        else:
            dz1 = da * z3 * silu_grad(z1)
            dz3 = da * silu(z1)
            out["dW1"][e] = dz1.T @ x
            out["dW3"][e] = dz3.T @ x
            dx = dz1 @ W1[e] + dz3 @ W3[e]
        out["dh"][st] += dx                          # a token meets an expert at most once
        if with_scales:
            sc["dW2"][e] = np.abs(do).T @ np.abs(a)
            if b2 is not None:
                sc["db2"][e] = np.abs(do).sum(axis=0)
            if act == ACT_GELU:
                sc["dW1"][e] = np.abs(dz).T @ np.abs(x)
                if b1 is not None:
                    sc["db1"][e] = np.abs(dz).sum(axis=0)
                sc["dh"][st] += np.abs(dz) @ np.abs(W1[e])
            else:
                sc["dW1"][e] = np.abs(dz1).T @ np.abs(x)
                sc["dW3"][e] = np.abs(dz3).T @ np.abs(x)
                sc["dh"][st] += np.abs(dz1) @ np.abs(W1[e]) + np.abs(dz3) @ np.abs(W3[e])
    f = fwd["counts"] / float(max(T * K, 1))
    dl = gate_logit_grad(fwd["gate_logits"].astype(np.float64), idx, g, p, dg, gate, daux, f)
    if dz_loss != 0.0 and T > 0:
        dl = dl + dz_loss * z_loss_logit_grad(fwd["gate_logits"], p)
    W_r = np.asarray(inp["W_r"], np.float64)
    out["dh"] += dl @ W_r.T                          # gate logits = h W_r (+ b_r)
    out["dW_r"] = h.T @ dl
    if inp.get("b_r") is None:
        out["db_r"] = None
    else:
        out["db_r"] = np.zeros(E) if bias_select_only else dl.sum(axis=0)
    out["dgates"] = dg
    out["dlogits"] = dl
    if with_scales:
        sc["dh"] += np.abs(dl) @ np.abs(W_r).T
        sc["dW_r"] = np.abs(h).T @ np.abs(dl)
        sc["db_r"] = None if out["db_r"] is None else np.abs(dl).sum(axis=0)
        out["scale"] = sc
    return out


# ----------------------------------------------------------------------------- closed forms

def param_counts_micro(d: int, layers: int, E: int, K: int, width: int) -> Dict[str, int]:
    """Non-embedding parameters of the micro model ([CUR] Workshop and "Parameters you hold").

    Per layer: attention 4 d^2, two LayerNorms (gain + bias: 4 d), the router
    d E, and E experts of two bias-free d x width matrices; plus a final
    LayerNorm (2 d). Active counts K experts instead of E.
    """
    shared = layers * (4 * d * d + 4 * d + d * E) + 2 * d
    expert = 2 * d * width
    return {"total": shared + layers * E * expert, "active": shared + layers * K * expert,
            "attention_plus_active_experts": layers * (4 * d * d + K * expert)}


def param_counts_swiglu_model(d: int, layers: int, E: int, K: int, width: int,
                              vocab: int = 32000) -> Dict[str, int]:
    """A 7B-style model with SwiGLU experts ([LENSA] Step 1).

    Per layer: attention 4 d^2, two RMSNorm gains (2 d), the router d E, and E
    experts of 3 d width parameters; plus a final norm (d) and untied input and
    output embeddings (2 vocab d). Active counts K experts instead of E.
    """
    shared = layers * (4 * d * d + 2 * d + d * E) + d + 2 * vocab * d
    expert = 3 * d * width
    return {"expert": expert, "total": shared + layers * E * expert,
            "active": shared + layers * K * expert, "routed_total": layers * E * expert}


def load_stats(counts: Sequence[int], T: int, K: int) -> Dict[str, float]:
    """Histogram statistics of the Step 4 widget ([LENSA] Step 4)."""
    c = np.asarray(counts, np.int64)
    S = T * K
    top2 = np.sort(c)[::-1][:2].sum()
    return {"slots": int(c.sum()), "balanced": S / len(c), "busiest_share": float(c.max() / S),
            "top2_share": float(top2 / S), "idle": int((c == 0).sum())}

