"""ctypes binding of libmoe_mi355x.so (the C-ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch supplies device memory and the current stream. There is no
fallback: if the library is missing, or a tensor is not on a GPU, the call
raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, List, Optional, Tuple

import torch

from . import workloads as W

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
                4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP"}
KERNEL_IDS = {0: "route", 1: "finalize", 2: "hist", 3: "permute", 4: "gemm1", 5: "gemm2",
              6: "combine", 7: "zero", 8: "backward", 9: "wgrad"}


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("E", ctypes.c_int64),
                ("K", ctypes.c_int64), ("width", ctypes.c_int64), ("act", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("bias_mode", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s" % (fn, lib().moe_status_string(status).decode()))


_vp = ctypes.c_void_p
_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_workspace_size": (ctypes.c_int, [ctypes.POINTER(MoeDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 11 + [_vp, ctypes.c_size_t, _vp]),
    "moe_permute": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 6 + [_vp, ctypes.c_size_t, _vp]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 4 + [_vp]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 13 + [_vp, ctypes.c_size_t, _vp]),
    "moe_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 13 + [_vp]),
    "moe_capacity_slots": (ctypes.c_int, [ctypes.c_double, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int32)]),
    "moe_backward_workspace_size": (ctypes.c_int, [ctypes.POINTER(MoeDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_backward": (ctypes.c_int, [ctypes.POINTER(MoeDesc)] + [_vp] * 9 + [ctypes.c_float, _vp, ctypes.c_float]
                     + [_vp] * 8 + [_vp, ctypes.c_size_t, _vp]),
    "moe_trace_enable": (ctypes.c_int, [ctypes.c_int]),
    "moe_trace_read": (ctypes.c_int, [_vp, _vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    "moe_trace_disable": (ctypes.c_int, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("HIP library %s is missing: run __graft_entry__.build() or "
                               "python sparse_mixture_experts_48_amd/build.py" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> List[str]:
    """Every function name that include/moe.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


BIAS_LOGITS, BIAS_SELECT = 0, 1


def desc_of(cfg: W.LayerShape, T: Optional[int] = None, capacity: int = 0, bias_mode: int = BIAS_LOGITS) -> MoeDesc:
    """Descriptor of a layer shape; capacity = slots per expert (0: dropless);
    bias_mode = what the router bias acts on (moe_bias_mode)."""
    return MoeDesc(cfg.T if T is None else T, cfg.d, cfg.E, cfg.K, cfg.width, cfg.act, cfg.gate, cfg.dtype,
                   capacity, bias_mode)


def capacity_slots(factor: float, T: int, K: int, E: int) -> int:
    """Slots per expert for a capacity factor (moe_capacity_slots)."""
    c = ctypes.c_int32(0)
    _check("moe_capacity_slots", lib().moe_capacity_slots(float(factor), T, K, E, ctypes.byref(c)))
    return c.value


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() or None


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def workspace_size(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def workspace(desc: MoeDesc, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(desc), 256), dtype=torch.uint8, device=device)


def route(desc: MoeDesc, h, W_r, b_r=None, ws=None, want_logits=False, noise=None) -> Dict[str, torch.Tensor]:
    """moe_route; noise: [T][E] float32 added to the logits (or None). Also returns z_loss."""
    dev = h.device
    T, E, K = desc.T, desc.E, desc.K
    out = {"topk_idx": torch.empty((T, K), dtype=torch.int32, device=dev),
           "topk_gate": torch.empty((T, K), dtype=torch.float32, device=dev),
           "counts": torch.empty(E, dtype=torch.int32, device=dev),
           "prob_mean": torch.empty(E, dtype=torch.float32, device=dev),
           "aux": torch.empty(1, dtype=torch.float32, device=dev),
           "z_loss": torch.empty(1, dtype=torch.float32, device=dev)}
    if want_logits:
        out["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    ws = workspace(desc, dev) if ws is None else ws
    _check("moe_route", lib().moe_route(
        ctypes.byref(desc), _ptr(h), _ptr(W_r), _ptr(b_r), _ptr(out["topk_idx"]), _ptr(out["topk_gate"]),
        _ptr(out["counts"]), _ptr(out["prob_mean"]), _ptr(out["aux"]), _ptr(out.get("logits")), _ptr(noise),
        _ptr(out["z_loss"]), _ptr(ws), ws.numel(), _stream()))
    return out


def permute(desc: MoeDesc, topk_idx, h, ws=None) -> Dict[str, torch.Tensor]:
    dev = h.device
    T, E, K = desc.T, desc.E, desc.K
    out = {"offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
           "slot_token": torch.empty(T * K, dtype=torch.int32, device=dev),
           "token_slot": torch.empty((T, K), dtype=torch.int32, device=dev),
           "h_perm": torch.empty((T * K, desc.d), dtype=h.dtype, device=dev)}
    ws = workspace(desc, dev) if ws is None else ws
    _check("moe_permute", lib().moe_permute(
        ctypes.byref(desc), _ptr(topk_idx), _ptr(h), _ptr(out["offsets"]), _ptr(out["slot_token"]),
        _ptr(out["token_slot"]), _ptr(out["h_perm"]), _ptr(ws), ws.numel(), _stream()))
    return out


def expert_ffn(desc: MoeDesc, h_perm, offsets, W1, b1, W3, W2, b2, ws=None) -> torch.Tensor:
    dev = h_perm.device
    o_perm = torch.empty((desc.T * desc.K, desc.d), dtype=torch.float32, device=dev)
    ws = workspace(desc, dev) if ws is None else ws
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        ctypes.byref(desc), _ptr(h_perm), _ptr(offsets), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2), _ptr(b2),
        _ptr(o_perm), _ptr(ws), ws.numel(), _stream()))
    return o_perm


def combine(desc: MoeDesc, o_perm, token_slot, topk_gate, dtype) -> torch.Tensor:
    y = torch.empty((desc.T, desc.d), dtype=dtype, device=o_perm.device)
    _check("moe_combine", lib().moe_combine(ctypes.byref(desc), _ptr(o_perm), _ptr(token_slot),
                                            _ptr(topk_gate), _ptr(y), _stream()))
    return y


def forward(desc: MoeDesc, h, W_r, b_r, W1, b1, W3, W2, b2, ws=None, y=None, aux=None,
            counts=None, noise=None, z_loss=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """moe_forward: (y, aux, counts). noise: [T][E] float32 added to the logits
    (or None); z_loss: a float32 tensor of one element to receive the router
    z-loss (or None: not computed)."""
    dev = h.device
    y = torch.empty((desc.T, desc.d), dtype=h.dtype, device=dev) if y is None else y
    aux = torch.empty(1, dtype=torch.float32, device=dev) if aux is None else aux
    counts = torch.empty(desc.E, dtype=torch.int32, device=dev) if counts is None else counts
    ws = workspace(desc, dev) if ws is None else ws
    _check("moe_forward", lib().moe_forward(
        ctypes.byref(desc), _ptr(h), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2), _ptr(b2),
        _ptr(y), _ptr(aux), _ptr(counts), _ptr(noise), _ptr(z_loss), _ptr(ws), ws.numel(), _stream()))
    return y, aux, counts


# Bytes of the static device scratch of moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES in include/moe.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(desc: MoeDesc, h, W_r, b_r, W1, b1, W3, W2, b2, y, aux=None, counts=None, noise=None,
                    z_loss=None) -> None:
    """moe_forward_noalloc: the layer into the caller's y (and aux, counts,
    z_loss if given) with the library's static scratch; nothing is allocated
    here or in the library."""
    _check("moe_forward_noalloc", lib().moe_forward_noalloc(
        ctypes.byref(desc), _ptr(h), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2), _ptr(b2),
        _ptr(y), _ptr(aux), _ptr(counts), _ptr(noise), _ptr(z_loss), _stream()))


def backward_workspace(desc: MoeDesc, device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size", lib().moe_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)


def backward(desc: MoeDesc, h, W_r, b_r, W1, b1, W3, W2, b2, dy, daux: float = 0.0, ws=None,
             bias_grads: bool = True, noise=None, dz: float = 0.0) -> Dict[str, Optional[torch.Tensor]]:
    """Gradients of sum(dy * y) + daux * aux + dz * z_loss (moe_backward), with
    the router noise (or None) held fixed; float32 except dh."""
    dev = h.device
    E, d, w = desc.E, desc.d, desc.width
    f32 = dict(dtype=torch.float32, device=dev)
    swiglu = desc.act == W.ACT_SWIGLU
    out = {"dh": torch.empty((desc.T, d), dtype=h.dtype, device=dev),
           "dW_r": torch.empty((d, E), **f32),
           "db_r": torch.empty(E, **f32) if bias_grads and b_r is not None else None,
           "dW1": torch.empty((E, w, d), **f32),
           "db1": torch.empty((E, w), **f32) if bias_grads and not swiglu and b1 is not None else None,
           "dW3": torch.empty((E, w, d), **f32) if swiglu else None,
           "dW2": torch.empty((E, d, w), **f32),
           "db2": torch.empty((E, d), **f32) if bias_grads and not swiglu and b2 is not None else None}
    ws = backward_workspace(desc, dev) if ws is None else ws
    _check("moe_backward", lib().moe_backward(
        ctypes.byref(desc), _ptr(h), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2), _ptr(b2),
        _ptr(dy), float(daux), _ptr(noise), float(dz), _ptr(out["dh"]), _ptr(out["dW_r"]), _ptr(out["db_r"]), _ptr(out["dW1"]),
        _ptr(out["db1"]), _ptr(out["dW3"]), _ptr(out["dW2"]), _ptr(out["db2"]), _ptr(ws), ws.numel(), _stream()))
    return out


class MoELayer:
    """One layer's weights on the GPU plus its workspace, for repeated forward calls."""

    def __init__(self, cfg: W.LayerShape, inputs: Dict[str, Optional[torch.Tensor]], device="cuda"):
        self.cfg = cfg
        self.desc = desc_of(cfg)
        self.p = {k: (None if v is None else v.to(device).contiguous()) for k, v in inputs.items()}
        self.ws = workspace(self.desc, device)
        self.y = torch.empty((cfg.T, cfg.d), dtype=cfg.torch_dtype, device=device)
        self.aux = torch.empty(1, dtype=torch.float32, device=device)
        self.counts = torch.empty(cfg.E, dtype=torch.int32, device=device)

    def forward(self, h: Optional[torch.Tensor] = None):
        p = self.p
        return forward(self.desc, p["h"] if h is None else h, p["W_r"], p["b_r"], p["W1"], p["b1"], p["W3"],
                       p["W2"], p["b2"], ws=self.ws, y=self.y, aux=self.aux, counts=self.counts)


class Trace:
    """Context manager around moe_trace_enable / moe_trace_read / moe_trace_disable."""

    def __init__(self, capacity: int = 4096):
        self.capacity = capacity

    def __enter__(self):
        _check("moe_trace_enable", lib().moe_trace_enable(self.capacity))
        return self

    def read(self) -> List[Tuple[str, float]]:
        ids = (ctypes.c_int32 * self.capacity)()
        ms = (ctypes.c_float * self.capacity)()
        n = ctypes.c_int(0)
        _check("moe_trace_read", lib().moe_trace_read(ctypes.cast(ids, _vp), ctypes.cast(ms, _vp),
                                                      self.capacity, ctypes.byref(n)))
        return [(KERNEL_IDS.get(ids[i], str(ids[i])), float(ms[i])) for i in range(n.value)]

    def __exit__(self, *exc):
        lib().moe_trace_disable()
        return False
