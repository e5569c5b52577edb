"""Thin Python binding of libmoe.so (declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  Torch tensors serve as device memory and torch's current stream
as the HIP stream.  If the library is not built, every call raises; there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_WQ_NONE, MOE_WQ_INT8, MOE_WQ_INT4 = 0, 1, 2
_WQ = {"none": MOE_WQ_NONE, "int8": MOE_WQ_INT8, "int4": MOE_WQ_INT4}
MOE_ROUTER_AUTO, MOE_ROUTER_EXACT, MOE_ROUTER_CERTIFIED = 0, 1, 2
_ROUTER = {"auto": MOE_ROUTER_AUTO, "exact": MOE_ROUTER_EXACT, "certified": MOE_ROUTER_CERTIFIED}
STAGES = {"route": 0, "dispatch": 1, "expert_ffn": 2, "combine": 3, "aux": 4, "layer": 5,
          "expert_ffn_train": 6, "layer_train": 7, "expert_ffn_backward": 8,
          "route_backward": 9, "layer_backward": 10}
ENTRY_POINTS = ("moe_workspace_size", "moe_capacity_from_factor", "moe_route", "moe_dispatch",
                "moe_expert_ffn", "moe_combine", "moe_aux_loss", "moe_router_z_loss",
                "moe_routing_stats", "moe_quantize_int8", "moe_quantize_int4", "moe_layer_forward",
                "moe_route_partials_size", "moe_router_path", "moe_layer_forward_stats",
                "moe_expert_ffn_train", "moe_layer_forward_train", "moe_combine_backward",
                "moe_expert_ffn_backward", "moe_route_backward", "moe_dispatch_backward",
                "moe_layer_backward", "moe_layer_forward_noalloc", "moe_last_error")
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # MOE_NOALLOC_SCRATCH_BYTES


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("aux_alpha", ctypes.c_float),
                ("weight_quant", ctypes.c_int32), ("router", ctypes.c_int32)]


_WEIGHT_FIELDS = ("w_router", "b_router", "logit_offset", "sel_bias", "w1", "b1", "w2", "b2",
                  "ws1", "ws2", "w1_scale", "w2_scale")


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


SAVED_FIELDS = ("logits", "topk_idx", "topk_w", "counts", "expert_offsets", "slot_row",
                "row_token", "n_dropped", "x_perm", "z", "h", "y_perm", "zs", "hs")
GRAD_FIELDS = ("d_w_router", "d_b_router", "d_w1", "d_b1", "d_w2", "d_b2", "d_ws1", "d_ws2")


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in SAVED_FIELDS]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class MoeLayerStats(ctypes.Structure):
    _fields_ = [("aux_out", ctypes.c_void_p), ("zloss_beta", ctypes.c_float),
                ("zloss_out", ctypes.c_void_p), ("counts_out", ctypes.c_void_p),
                ("n_dropped_out", ctypes.c_void_p), ("weight_mean_out", ctypes.c_void_p)]


class MoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_layer_prefix_amd.csrc.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    cfgp, wp = ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeWeights)
    L.moe_workspace_size.argtypes = [cfgp, ctypes.c_int]
    L.moe_workspace_size.restype = sz
    L.moe_capacity_from_factor.argtypes = [i32, i32, ctypes.c_double]
    L.moe_capacity_from_factor.restype = i32
    L.moe_route_partials_size.argtypes = [cfgp]
    L.moe_route_partials_size.restype = sz
    L.moe_router_path.argtypes = [cfgp]
    L.moe_router_path.restype = ctypes.c_int
    L.moe_route.argtypes = [cfgp, vp, wp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn.argtypes = [cfgp, vp, vp, wp, vp, vp, vp, vp, sz, vp]
    L.moe_combine.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
    L.moe_aux_loss.argtypes = [cfgp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_router_z_loss.argtypes = [cfgp, vp, vp, ctypes.c_float, vp, vp, sz, vp]
    L.moe_routing_stats.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_quantize_int8.argtypes = [vp, i32, ctypes.c_int64, i32, vp, vp, vp]
    L.moe_quantize_int4.argtypes = [vp, i32, ctypes.c_int64, i32, vp, vp, vp]
    L.moe_layer_forward.argtypes = [cfgp, vp, wp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_layer_forward_noalloc.argtypes = [cfgp, vp, wp, vp, vp, vp, vp, vp]
    L.moe_layer_forward_stats.argtypes = [cfgp, vp, wp, vp, ctypes.POINTER(MoeLayerStats), vp, sz,
                                          vp]
    svp, gp, f32 = ctypes.POINTER(MoeSaved), ctypes.POINTER(MoeGrads), ctypes.c_float
    L.moe_expert_ffn_train.argtypes = [cfgp, vp, vp, wp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_layer_forward_train.argtypes = [cfgp, vp, wp, vp, vp, svp, vp, sz, vp]
    L.moe_combine_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_ffn_backward.argtypes = [cfgp, vp, vp, wp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          gp, vp, sz, vp]
    L.moe_route_backward.argtypes = [cfgp, vp, wp, vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, gp,
                                     vp, sz, vp]
    L.moe_dispatch_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
    L.moe_layer_backward.argtypes = [cfgp, vp, wp, svp, vp, f32, f32, f32, vp, gp, vp, sz, vp]
    for name in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_aux_loss",
                 "moe_router_z_loss", "moe_routing_stats", "moe_quantize_int8", "moe_quantize_int4",
                 "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_stats",
                 "moe_expert_ffn_train",
                 "moe_layer_forward_train",
                 "moe_combine_backward", "moe_expert_ffn_backward", "moe_route_backward",
                 "moe_dispatch_backward", "moe_layer_backward"):
        getattr(L, name).restype = ctypes.c_int
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code: int):
    if code != MOE_OK:
        raise MoEError(code, lib().moe_last_error().decode())


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (or None)."""
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------- config / weights
def capacity_from_factor(T: int, n_experts: int, capacity_factor: float) -> int:
    c = lib().moe_capacity_from_factor(T, n_experts, float(capacity_factor))
    if c < 0:
        raise ValueError("invalid capacity arguments")
    return c


def make_config(T, d_model, d_ff, n_experts, top_k, *, capacity=0, d_ff_shared=0, dtype="bf16",
                aux_alpha=0.0, weight_quant="none", router="auto") -> MoeConfig:
    return MoeConfig(T=T, d_model=d_model, d_ff=d_ff, n_experts=n_experts, top_k=top_k,
                     capacity=capacity or 0, d_ff_shared=d_ff_shared,
                     dtype=MOE_F32 if dtype in ("f32", MOE_F32) else MOE_BF16,
                     aux_alpha=float(aux_alpha),
                     weight_quant=_WQ.get(weight_quant, weight_quant),
                     router=_ROUTER.get(router, router))


def router_path(cfg: MoeConfig) -> str:
    """'exact' or 'certified': the router path cfg.router resolves to."""
    p = lib().moe_router_path(ctypes.byref(cfg))
    if p < 0:
        raise ValueError("invalid config")
    return "certified" if p == MOE_ROUTER_CERTIFIED else "exact"


def config_for(shape, T: Optional[int] = None, router="auto") -> MoeConfig:
    """MoeConfig of a workload shape (configs.MoEShape), optionally with another T
    and router path."""
    T = shape.T if T is None else T
    cap = 0
    if shape.capacity_factor is not None:
        cap = capacity_from_factor(T, shape.n_experts, shape.capacity_factor)
    return make_config(T, shape.d_model, shape.d_ff, shape.n_experts, shape.top_k, capacity=cap,
                       d_ff_shared=shape.d_ff_shared, dtype=shape.dtype, aux_alpha=shape.aux_alpha,
                       weight_quant=getattr(shape, "weight_quant", "none"), router=router)


def make_weights(t: Dict[str, object]) -> MoeWeights:
    """MoeWeights from a dict of device tensors (missing or None -> NULL)."""
    return MoeWeights(**{n: _p(t.get(n)) for n in _WEIGHT_FIELDS})


def workspace_size(cfg: MoeConfig, stage: str = "layer") -> int:
    n = lib().moe_workspace_size(ctypes.byref(cfg), STAGES[stage])
    if n == ctypes.c_size_t(-1).value:
        raise MoEError(MOE_ERR_INVALID_ARG, "invalid config")
    return n


def alloc_workspace(cfg: MoeConfig, stage: str = "layer", device="cuda"):
    import torch
    n = workspace_size(cfg, stage)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ws(ws):
    return (None, 0) if ws is None else (_p(ws), ws.numel() * ws.element_size())


# ---------------------------------------------------------------- entry points
def route_partials_size(cfg: MoeConfig) -> int:
    n = lib().moe_route_partials_size(ctypes.byref(cfg))
    if n == ctypes.c_size_t(-1).value:
        raise MoEError(MOE_ERR_INVALID_ARG, "invalid config")
    return n


def alloc_route_partials(cfg: MoeConfig, device="cuda"):
    """A device buffer for moe_route's routing partials (256-byte aligned)."""
    import torch
    return torch.empty(route_partials_size(cfg), dtype=torch.uint8, device=device)


def moe_route(cfg, x, w: MoeWeights, logits, topk_idx, topk_w, ws=None, stream=None,
              partials=None):
    p, n = _ws(ws)
    _check(lib().moe_route(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(logits), _p(topk_idx),
                           _p(topk_w), _p(partials), p, n, _stream(stream)))


def moe_dispatch(cfg, topk_idx, x, counts, expert_offsets, slot_row, row_token, x_perm,
                 n_dropped, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_dispatch(ctypes.byref(cfg), _p(topk_idx), _p(x), _p(counts),
                              _p(expert_offsets), _p(slot_row), _p(row_token), _p(x_perm),
                              _p(n_dropped), p, n, _stream(stream)))


def moe_expert_ffn(cfg, x_perm, expert_offsets, w: MoeWeights, x, y_perm, y_shared, ws,
                   stream=None):
    p, n = _ws(ws)
    _check(lib().moe_expert_ffn(ctypes.byref(cfg), _p(x_perm), _p(expert_offsets),
                                ctypes.byref(w), _p(x), _p(y_perm), _p(y_shared), p, n,
                                _stream(stream)))


def moe_combine(cfg, y_perm, slot_row, topk_w, y_shared, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(cfg), _p(y_perm), _p(slot_row), _p(topk_w),
                             _p(y_shared), _p(out), _stream(stream)))


def moe_aux_loss(cfg, logits, counts, loss_out, ws, stream=None, partials=None):
    """From the logits, or (logits=None) from moe_route's partials."""
    p, n = _ws(ws)
    _check(lib().moe_aux_loss(ctypes.byref(cfg), _p(logits), _p(partials), _p(counts),
                              _p(loss_out), p, n, _stream(stream)))


def moe_router_z_loss(cfg, logits, beta, loss_out, ws, stream=None, partials=None):
    """From the logits, or (logits=None) from moe_route's partials."""
    p, n = _ws(ws)
    _check(lib().moe_router_z_loss(ctypes.byref(cfg), _p(logits), _p(partials), float(beta),
                                   _p(loss_out), p, n, _stream(stream)))


def moe_routing_stats(cfg, topk_idx, topk_w, counts_out, weight_mean_out, ws, stream=None,
                      partials=None):
    """From the routing, or (topk_idx = topk_w = None) from moe_route's partials."""
    p, n = _ws(ws)
    _check(lib().moe_routing_stats(ctypes.byref(cfg), _p(topk_idx), _p(topk_w), _p(partials),
                                   _p(counts_out), _p(weight_mean_out), p, n, _stream(stream)))


def moe_quantize_int8(w, q_out, scale_out, stream=None):
    """Per-row INT8 codes and fp32 scales of a [rows, cols] bf16 or fp32 device
    tensor (any leading shape; the last dimension is the row)."""
    import torch
    dt = MOE_F32 if w.dtype == torch.float32 else MOE_BF16
    cols = int(w.shape[-1])
    rows = int(w.numel() // cols)
    _check(lib().moe_quantize_int8(_p(w), dt, rows, cols, _p(q_out), _p(scale_out),
                                   _stream(stream)))


def moe_quantize_int4(w, q_out, scale_out, stream=None):
    """Per-row INT4 codes (two per byte, [rows, cols/2] uint8) and fp32 scales
    of a [rows, cols] bf16 or fp32 device tensor (any leading shape)."""
    import torch
    dt = MOE_F32 if w.dtype == torch.float32 else MOE_BF16
    cols = int(w.shape[-1])
    rows = int(w.numel() // cols)
    _check(lib().moe_quantize_int4(_p(w), dt, rows, cols, _p(q_out), _p(scale_out),
                                   _stream(stream)))


def quantize_expert_weights(t: Dict[str, object], bits: int = 8) -> Dict[str, object]:
    """A copy of a weight dict whose routed w1 / w2 are INT8 (bits=8) or packed
    INT4 (bits=4) codes with their w1_scale / w2_scale, made on the device by
    moe_quantize_int8 / moe_quantize_int4."""
    import torch
    if bits not in (8, 4):
        raise ValueError("bits must be 8 or 4")
    out = dict(t)
    for name in ("w1", "w2"):
        w = t[name]
        sc = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
        if bits == 8:
            q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
            moe_quantize_int8(w, q, sc)
        else:
            q = torch.empty(tuple(w.shape[:-1]) + (w.shape[-1] // 2,), dtype=torch.uint8,
                            device=w.device)
            moe_quantize_int4(w, q, sc)
        out[name] = q
        out[name + "_scale"] = sc
    return out


def moe_layer_forward(cfg, x, w: MoeWeights, out, aux_out=None, counts_out=None,
                      n_dropped_out=None, ws=None, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_layer_forward(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(out),
                                   _p(aux_out), _p(counts_out), _p(n_dropped_out), p, n,
                                   _stream(stream)))


def moe_layer_forward_stats(cfg, x, w: MoeWeights, out, aux_out=None, zloss_beta=0.0,
                            zloss_out=None, counts_out=None, n_dropped_out=None,
                            weight_mean_out=None, ws=None, stream=None):
    st = MoeLayerStats(aux_out=_p(aux_out), zloss_beta=float(zloss_beta), zloss_out=_p(zloss_out),
                       counts_out=_p(counts_out), n_dropped_out=_p(n_dropped_out),
                       weight_mean_out=_p(weight_mean_out))
    p, n = _ws(ws)
    _check(lib().moe_layer_forward_stats(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(out),
                                         ctypes.byref(st), p, n, _stream(stream)))


def moe_layer_forward_noalloc(cfg, x, w: MoeWeights, out, aux_out=None, counts_out=None,
                              n_dropped_out=None, stream=None):
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(out),
                                           _p(aux_out), _p(counts_out), _p(n_dropped_out),
                                           _stream(stream)))


# ---------------------------------------------------------------- training entry points
def make_saved(t: Dict[str, object]) -> MoeSaved:
    return MoeSaved(**{n: _p(t.get(n)) for n in SAVED_FIELDS})


def make_grads(t: Dict[str, object]) -> MoeGrads:
    return MoeGrads(**{n: _p(t.get(n)) for n in GRAD_FIELDS})


def moe_expert_ffn_train(cfg, x_perm, expert_offsets, w: MoeWeights, x, z, h, y_perm, zs, hs,
                         y_shared, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_expert_ffn_train(ctypes.byref(cfg), _p(x_perm), _p(expert_offsets),
                                      ctypes.byref(w), _p(x), _p(z), _p(h), _p(y_perm), _p(zs),
                                      _p(hs), _p(y_shared), p, n, _stream(stream)))


def moe_layer_forward_train(cfg, x, w: MoeWeights, out, aux_out, saved: MoeSaved, ws,
                            stream=None):
    p, n = _ws(ws)
    _check(lib().moe_layer_forward_train(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(out),
                                         _p(aux_out), ctypes.byref(saved), p, n,
                                         _stream(stream)))


def moe_combine_backward(cfg, d_out, y_perm, slot_row, topk_w, d_y_perm, d_topk_w, stream=None):
    _check(lib().moe_combine_backward(ctypes.byref(cfg), _p(d_out), _p(y_perm), _p(slot_row),
                                      _p(topk_w), _p(d_y_perm), _p(d_topk_w), _stream(stream)))


def moe_expert_ffn_backward(cfg, x_perm, expert_offsets, w: MoeWeights, x, z, h, zs, hs,
                            d_y_perm, d_out, d_x_perm, d_x_shared, grads: MoeGrads, ws,
                            stream=None):
    p, n = _ws(ws)
    _check(lib().moe_expert_ffn_backward(ctypes.byref(cfg), _p(x_perm), _p(expert_offsets),
                                         ctypes.byref(w), _p(x), _p(z), _p(h), _p(zs), _p(hs),
                                         _p(d_y_perm), _p(d_out), _p(d_x_perm), _p(d_x_shared),
                                         ctypes.byref(grads), p, n, _stream(stream)))


def moe_route_backward(cfg, x, w: MoeWeights, logits, topk_idx, topk_w, d_topk_w, counts,
                       aux_grad, zloss_beta, zloss_grad, d_logits, d_x_router, grads: MoeGrads,
                       ws, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_route_backward(ctypes.byref(cfg), _p(x), ctypes.byref(w), _p(logits),
                                    _p(topk_idx), _p(topk_w), _p(d_topk_w), _p(counts),
                                    float(aux_grad), float(zloss_beta), float(zloss_grad),
                                    _p(d_logits), _p(d_x_router), ctypes.byref(grads), p, n,
                                    _stream(stream)))


def moe_dispatch_backward(cfg, d_x_perm, slot_row, d_x_shared, d_x_router, d_x, stream=None):
    _check(lib().moe_dispatch_backward(ctypes.byref(cfg), _p(d_x_perm), _p(slot_row),
                                       _p(d_x_shared), _p(d_x_router), _p(d_x), _stream(stream)))


def moe_layer_backward(cfg, x, w: MoeWeights, saved: MoeSaved, d_out, aux_grad, zloss_beta,
                       zloss_grad, d_x, grads: MoeGrads, ws, stream=None):
    p, n = _ws(ws)
    _check(lib().moe_layer_backward(ctypes.byref(cfg), _p(x), ctypes.byref(w),
                                    ctypes.byref(saved), _p(d_out), float(aux_grad),
                                    float(zloss_beta), float(zloss_grad), _p(d_x),
                                    ctypes.byref(grads), p, n, _stream(stream)))


def alloc_saved(cfg: MoeConfig, device="cuda") -> Dict[str, object]:
    """Device buffers for the tensors the training forward keeps."""
    import torch
    T, K, N, d, f, fs = cfg.T, cfg.top_k, cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    dt = torch.float32 if cfg.dtype == MOE_F32 else torch.bfloat16
    i32, f32 = torch.int32, torch.float32
    t = dict(logits=torch.empty(T, N, dtype=f32, device=device),
             topk_idx=torch.empty(T, K, dtype=i32, device=device),
             topk_w=torch.empty(T, K, dtype=f32, device=device),
             counts=torch.empty(N, dtype=i32, device=device),
             expert_offsets=torch.empty(N + 1, dtype=i32, device=device),
             slot_row=torch.empty(T, K, dtype=i32, device=device),
             row_token=torch.empty(T * K, dtype=i32, device=device),
             n_dropped=torch.empty(1, dtype=i32, device=device),
             x_perm=torch.empty(T * K, d, dtype=dt, device=device),
             z=torch.empty(T * K, f, dtype=dt, device=device),
             h=torch.empty(T * K, f, dtype=dt, device=device),
             y_perm=torch.empty(T * K, d, dtype=dt, device=device))
    if fs:
        t["zs"] = torch.empty(T, fs, dtype=dt, device=device)
        t["hs"] = torch.empty(T, fs, dtype=dt, device=device)
    return t


def alloc_grads(cfg: MoeConfig, biases: bool, router_bias: bool, device="cuda") -> Dict[str, object]:
    """Device buffers for the gradients (expert biases and router bias optional)."""
    import torch
    N, d, f, fs = cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    dt = torch.float32 if cfg.dtype == MOE_F32 else torch.bfloat16
    g = dict(d_w_router=torch.empty(N, d, dtype=torch.float32, device=device),
             d_w1=torch.empty(N, f, d, dtype=dt, device=device),
             d_w2=torch.empty(N, d, f, dtype=dt, device=device))
    if router_bias:
        g["d_b_router"] = torch.empty(N, dtype=torch.float32, device=device)
    if biases:
        g["d_b1"] = torch.empty(N, f, dtype=dt, device=device)
        g["d_b2"] = torch.empty(N, d, dtype=dt, device=device)
    if fs:
        g["d_ws1"] = torch.empty(fs, d, dtype=dt, device=device)
        g["d_ws2"] = torch.empty(d, fs, dtype=dt, device=device)
    return g


# ---------------------------------------------------------------- convenience
class MoELayer:
    """Holds a config, device weights and a workspace; ``forward`` enqueues
    moe_layer_forward on the current stream and returns device tensors."""

    def __init__(self, cfg: MoeConfig, tensors: Dict[str, object], device="cuda"):
        import torch
        self.cfg = cfg
        self.tensors = tensors
        self.w = make_weights(tensors)
        self.ws = alloc_workspace(cfg, "layer", device)
        self.dtype = torch.float32 if cfg.dtype == MOE_F32 else torch.bfloat16
        self.device = device
        N = cfg.n_experts
        wr = tensors["w_router"]
        if tuple(wr.shape) != (N, cfg.d_model):
            raise ValueError(f"router weight {tuple(wr.shape)} does not match N={N}, "
                             f"d_model={cfg.d_model}")
        # packed INT4 codes hold two elements per byte along the row
        div = 2 if cfg.weight_quant == MOE_WQ_INT4 else 1
        if tuple(tensors["w1"].shape) != (N, cfg.d_ff, cfg.d_model // div):
            raise ValueError("w1 must be [N, d_ff, d_model] and match the router's N")
        if tuple(tensors["w2"].shape) != (N, cfg.d_model, cfg.d_ff // div):
            raise ValueError("w2 must be [N, d_model, d_ff] and match the router's N")

    def forward(self, x, aux: bool = False, out=None, stream=None):
        import torch
        if tuple(x.shape) != (self.cfg.T, self.cfg.d_model) or x.dtype != self.dtype:
            raise ValueError("x must be [T, d_model] in the layer dtype")
        out = torch.empty_like(x) if out is None else out
        aux_t = torch.empty(1, dtype=torch.float32, device=x.device) if aux else None
        counts = torch.empty(self.cfg.n_experts, dtype=torch.int32, device=x.device)
        ndrop = torch.empty(1, dtype=torch.int32, device=x.device)
        moe_layer_forward(self.cfg, x, self.w, out, aux_t, counts, ndrop, self.ws, stream)
        return out, aux_t, counts, ndrop


class MoETrainLayer(MoELayer):
    """MoELayer with a training step: ``forward`` keeps the tensors the
    backward needs; ``backward`` fills the gradient buffers and returns d_x."""

    def __init__(self, cfg: MoeConfig, tensors: Dict[str, object], device="cuda"):
        super().__init__(cfg, tensors, device)
        self.ws = alloc_workspace(cfg, "layer_train", device)
        self.ws_bwd = alloc_workspace(cfg, "layer_backward", device)
        self.saved_t = alloc_saved(cfg, device)
        self.saved = make_saved(self.saved_t)
        biases = tensors.get("b1") is not None or tensors.get("b2") is not None
        self.grads_t = alloc_grads(cfg, biases, tensors.get("b_router") is not None, device)
        self.grads = make_grads(self.grads_t)

    def forward(self, x, aux: bool = False, out=None, stream=None):
        import torch
        if tuple(x.shape) != (self.cfg.T, self.cfg.d_model) or x.dtype != self.dtype:
            raise ValueError("x must be [T, d_model] in the layer dtype")
        out = torch.empty_like(x) if out is None else out
        aux_t = torch.empty(1, dtype=torch.float32, device=x.device) if aux else None
        moe_layer_forward_train(self.cfg, x, self.w, out, aux_t, self.saved, self.ws, stream)
        return out, aux_t

    def backward(self, x, d_out, aux_grad=0.0, zloss_beta=0.0, zloss_grad=0.0, d_x=None,
                 stream=None):
        import torch
        d_x = torch.empty_like(x) if d_x is None else d_x
        moe_layer_backward(self.cfg, x, self.w, self.saved, d_out, aux_grad, zloss_beta,
                           zloss_grad, d_x, self.grads, self.ws_bwd, stream)
        return d_x
