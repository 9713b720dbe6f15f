"""Seeded synthetic inputs for the top-K routed MoE FFN layer.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle. It draws numbers and lays them out; it holds none of the layer's
arithmetic (no routing, no softmax, no expert MLP).

Shapes follow the workloads the pages talk about:
  * the micro model of the Curionode plate "Mixture of Experts." (Vol. VII,
    Plate 4), section "Workshop": d = 128, experts of width 512, E = 8, K = 2;
  * many small experts with a skewed router, after the Lensa ML explainer
    "Mixture of Experts", Step 1 (many small experts) and Step 4 (a router with
    a built-in per-expert bias that favours a few experts);
  * the Mixtral shape of the same explainer, Step 6 (8 experts of
    3 x 4096 x 14336 parameters, top-2), at a prefill batch and at a decode
    batch (FAQ "Does MoE make inference faster?": small batches are bound by
    weight reads);
  * Switch-style top-1 with many experts (Step 3: Switch scales by p_i).

Value distributions (every reading is listed in the design notes):
  * h ~ N(0, 1);
  * router weight W_r ~ N(0, std 0.02), always float32 (the router is kept in
    float32, Arjun Jaggi, "Mixture of Experts in LLMs: How Sparse Models
    Scale", section "Switch Transformers");
  * expert weights ~ N(0, variance 1/fan_in); expert biases ~ N(0, variance
    1/fan_in of the layer they follow);
  * router bias: N(0, std 2) for the skewed workload; -1.1 * ln(r_e) with r a
    seeded permutation of 1..E (log of a Zipf(1.1) law) for the Switch one.

Storage layout (what the C-ABI expects):
  h      [T][d]            dtype
  W_r    [d][E]            float32
  b_r    [E]               float32 (or None)
  W1,W3  [E][width][d]     dtype   (row n of expert e = column n of the d x width matrix)
  b1     [E][width]        dtype   (GELU experts only)
  W2     [E][d][width]     dtype   (row j of expert e = column j of the width x d matrix)
  b2     [E][d]            dtype   (GELU experts only)

Every tensor is drawn in float32 in storage order from
numpy.random.default_rng([seed, tensor_id, chunk]) and, for bfloat16 workloads,
rounded to bfloat16 (round to nearest even) by torch on the CPU.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Optional

import numpy as np
import torch

ACT_GELU = 0
ACT_SWIGLU = 1
GATE_RENORM = 0
GATE_RAW = 1
DT_F32 = 0
DT_BF16 = 1

_TENSOR_IDS = {"h": 1, "W_r": 2, "b_r": 3, "W1": 4, "b1": 5, "W3": 6, "W2": 7, "b2": 8}


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE FFN layer: T tokens of width d, E experts of width `width`, top-K."""
    name: str
    T: int
    d: int
    E: int
    K: int
    width: int
    act: int          # ACT_GELU (exact erf GELU MLP with biases) or ACT_SWIGLU (no biases)
    gate: int         # GATE_RENORM (softmax over the chosen K) or GATE_RAW (p_i of the full softmax)
    dtype: int        # DT_F32 or DT_BF16 for h, expert weights, expert biases and y
    router_bias: str  # "none" | "normal2" | "zipf1.1"
    seed: int

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)

    @property
    def S(self) -> int:
        return self.T * self.K

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == DT_F32 else torch.bfloat16


WORKLOADS: Dict[str, LayerShape] = {
    "micro": LayerShape("micro", T=256, d=128, E=8, K=2, width=512, act=ACT_GELU,
                        gate=GATE_RENORM, dtype=DT_F32, router_bias="none", seed=1),
    "skewed": LayerShape("skewed", T=4096, d=128, E=64, K=2, width=512, act=ACT_GELU,
                         gate=GATE_RENORM, dtype=DT_BF16, router_bias="normal2", seed=2),
    "mixtral_prefill": LayerShape("mixtral_prefill", T=4096, d=4096, E=8, K=2, width=14336,
                                  act=ACT_SWIGLU, gate=GATE_RENORM, dtype=DT_BF16,
                                  router_bias="none", seed=3),
    "mixtral_decode": LayerShape("mixtral_decode", T=16, d=4096, E=8, K=2, width=14336,
                                 act=ACT_SWIGLU, gate=GATE_RENORM, dtype=DT_BF16,
                                 router_bias="none", seed=4),
    "switch_top1": LayerShape("switch_top1", T=8192, d=4096, E=64, K=1, width=1376,
                              act=ACT_SWIGLU, gate=GATE_RAW, dtype=DT_BF16,
                              router_bias="zipf1.1", seed=5),
}
WORKLOAD_ORDER = ["micro", "skewed", "mixtral_prefill", "mixtral_decode", "switch_top1"]

_POOL_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _normal(seed: int, tid: int, shape, std: float, chunk_axis0: bool = False) -> np.ndarray:
    """float32 N(0, std^2) draws in storage order; axis 0 drawn per chunk (in parallel)."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    if out.size == 0:
        return out
    if chunk_axis0 and shape[0] > 1:
        def fill(i):
            np.random.default_rng([seed, tid, i]).standard_normal(dtype=np.float32, out=out[i])
            out[i] *= np.float32(std)
        with _cf.ThreadPoolExecutor(_POOL_THREADS) as ex:
            list(ex.map(fill, range(shape[0])))
    else:
        np.random.default_rng([seed, tid, 0]).standard_normal(dtype=np.float32, out=out)
        out *= np.float32(std)
    return out


def _to_dtype(a: np.ndarray, cfg: LayerShape) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t if cfg.dtype == DT_F32 else t.to(torch.bfloat16)


def make_inputs(cfg: LayerShape, seed: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """All layer inputs as contiguous CPU torch tensors (see module doc for layout)."""
    s = cfg.seed if seed is None else seed
    T, d, E, w = cfg.T, cfg.d, cfg.E, cfg.width
    ids = _TENSOR_IDS
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["h"] = _to_dtype(_normal(s, ids["h"], (T, d), 1.0), cfg)
    out["W_r"] = torch.from_numpy(_normal(s, ids["W_r"], (d, E), 0.02))
    if cfg.router_bias == "none":
        out["b_r"] = None
    elif cfg.router_bias == "normal2":
        out["b_r"] = torch.from_numpy(_normal(s, ids["b_r"], (E,), 2.0))
    elif cfg.router_bias == "zipf1.1":
        r = np.random.default_rng([s, ids["b_r"], 0]).permutation(E) + 1
        out["b_r"] = torch.from_numpy((-1.1 * np.log(r.astype(np.float64))).astype(np.float32))
    else:
        raise ValueError(cfg.router_bias)
    out["W1"] = _to_dtype(_normal(s, ids["W1"], (E, w, d), d ** -0.5, chunk_axis0=True), cfg)
    out["W2"] = _to_dtype(_normal(s, ids["W2"], (E, d, w), w ** -0.5, chunk_axis0=True), cfg)
    if cfg.act == ACT_SWIGLU:
        out["W3"] = _to_dtype(_normal(s, ids["W3"], (E, w, d), d ** -0.5, chunk_axis0=True), cfg)
        out["b1"] = None
        out["b2"] = None
    else:
        out["W3"] = None
        out["b1"] = _to_dtype(_normal(s, ids["b1"], (E, w), d ** -0.5), cfg)
        out["b2"] = _to_dtype(_normal(s, ids["b2"], (E, d), w ** -0.5), cfg)
    return out


def as_float64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact upcast of a float32/bfloat16 CPU tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def as_float32(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact upcast of a float32/bfloat16 CPU tensor to a float32 numpy array."""
    if t is None:
        return None
    return np.ascontiguousarray(t.detach().to("cpu").to(torch.float32).numpy())
