"""Seeded synthetic inputs for the MoE layer forward.

This module serves both the GPU path's callers and the CPU oracle's callers;
it holds none of the layer's arithmetic.  It only draws random tensors and
stores them in the layer's dtype.

Recipe (seed s, workload index c):
  * every tensor block has its own numpy PCG64 stream, keyed by
    SeedSequence(entropy=s, spawn_key=(c, tensor_code, block)), so blocks can
    be drawn in parallel and any single expert can be regenerated on its own;
  * x ~ N(0, 1), drawn in blocks of 1024 token rows;
  * a weight matrix with fan-in F ~ N(0, 1/F): fp32 standard normal draws
    times the fp32 constant F**-0.5; router W_r [N, d], expert W1[e] [f, d],
    W2[e] [d, f], shared Ws1 [f_s, d], Ws2 [d, f_s] (nn.Linear [out, in]
    layout, the reduction dimension contiguous);
  * biases (tiny fp32 layer only) ~ N(0, 0.01), i.e. sigma = 0.1;
  * logit offsets: "normal" -> N(0, 1) per expert; "zipf" -> pi(e) ** -1.1
    with pi a seeded random permutation of 1..N;
  * selection bias ~ U(-0.5, 0.5) per expert;
  * bf16 workloads round every x / weight value once, to nearest-even, to
    bfloat16; offsets, selection biases and router bias stay fp32.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

from .configs import MoEShape

# tensor codes for the stream keys
_ROUTER_W, _ROUTER_B, _OFFSET, _SEL_BIAS = 1, 2, 3, 4
_W1, _B1, _W2, _B2, _WS1, _WS2, _X, _PERM = 5, 6, 7, 8, 9, 10, 11, 12
_D_OUT = 13
_X_BLOCK = 1024


def _rng(seed: int, shape: MoEShape, code: int, block: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(shape.index, code, block))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite, so no NaN handling is needed."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_widen(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exact same values as fp32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_block(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return bf16_round(a) if dtype == "bf16" else a


def _threads() -> int:
    n = os.cpu_count() or 8
    return max(1, min(16, n))


@dataclasses.dataclass
class MoEInputs:
    """Host copies of every input of one workload.

    bf16 tensors are uint16 bit patterns; fp32 tensors are float32.  Use
    ``f32(name)`` for the exact values as float32."""
    shape: MoEShape
    seed: int
    x: np.ndarray
    w_router: np.ndarray
    b_router: Optional[np.ndarray]
    logit_offset: Optional[np.ndarray]
    sel_bias: Optional[np.ndarray]
    w1: Optional[np.ndarray]         # [N, f, d]  (None when generated lazily)
    b1: Optional[np.ndarray]         # [N, f]
    w2: Optional[np.ndarray]         # [N, d, f]
    b2: Optional[np.ndarray]         # [N, d]
    ws1: Optional[np.ndarray]        # [f_s, d]
    ws2: Optional[np.ndarray]        # [d, f_s]

    def f32(self, name: str) -> Optional[np.ndarray]:
        a = getattr(self, name)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return bf16_widen(a)
        return a

    def expert(self, e: int):
        """(W1[e], b1[e], W2[e], b2[e]) in storage form; regenerated from the
        expert's own streams when the full stacks were not materialised."""
        if self.w1 is not None:
            return (self.w1[e], None if self.b1 is None else self.b1[e],
                    self.w2[e], None if self.b2 is None else self.b2[e])
        return expert_weights(self.shape, e, self.seed)


def expert_weights(shape: MoEShape, e: int, seed: int = 0):
    """W1[e] [f, d], b1[e] [f] | None, W2[e] [d, f], b2[e] [d] | None."""
    d, f = shape.d_model, shape.d_ff
    w1 = _normal_block(_rng(seed, shape, _W1, e), (f, d), d ** -0.5, shape.dtype)
    w2 = _normal_block(_rng(seed, shape, _W2, e), (d, f), f ** -0.5, shape.dtype)
    b1 = b2 = None
    if shape.expert_bias:
        b1 = _normal_block(_rng(seed, shape, _B1, e), (f,), 0.1, shape.dtype)
        b2 = _normal_block(_rng(seed, shape, _B2, e), (d,), 0.1, shape.dtype)
    return w1, b1, w2, b2


def make_inputs(shape: MoEShape, seed: int = 0, materialize_experts: bool = True,
                threads: Optional[int] = None) -> MoEInputs:
    """Draw every input of ``shape`` from the seeded streams.

    With ``materialize_experts=False`` the expert stacks are left out and
    ``MoEInputs.expert(e)`` regenerates one expert on demand (same values)."""
    T, d, f, N = shape.T, shape.d_model, shape.d_ff, shape.n_experts
    dt = shape.dtype
    nthr = threads or _threads()
    store = np.uint16 if dt == "bf16" else np.float32

    x = np.empty((T, d), dtype=store)
    nxb = (T + _X_BLOCK - 1) // _X_BLOCK

    def fill_x(b):
        r0, r1 = b * _X_BLOCK, min(T, (b + 1) * _X_BLOCK)
        x[r0:r1] = _normal_block(_rng(seed, shape, _X, b), (r1 - r0, d), 1.0, dt)

    w_router = _normal_block(_rng(seed, shape, _ROUTER_W), (N, d), d ** -0.5, dt)
    b_router = None
    if shape.router_bias:
        b_router = _rng(seed, shape, _ROUTER_B).standard_normal(N, dtype=np.float32) * np.float32(0.1)
    logit_offset = None
    if shape.logit_offset == "normal":
        logit_offset = _rng(seed, shape, _OFFSET).standard_normal(N, dtype=np.float32)
    elif shape.logit_offset == "zipf":
        rank = _rng(seed, shape, _PERM).permutation(N) + 1
        logit_offset = (rank.astype(np.float64) ** -1.1).astype(np.float32)
    elif shape.logit_offset is not None:
        raise ValueError(f"unknown logit_offset kind {shape.logit_offset!r}")
    sel_bias = None
    if shape.sel_bias:
        sel_bias = _rng(seed, shape, _SEL_BIAS).uniform(-0.5, 0.5, N).astype(np.float32)

    w1 = b1 = w2 = b2 = None
    if materialize_experts:
        w1 = np.empty((N, f, d), dtype=store)
        w2 = np.empty((N, d, f), dtype=store)
        if shape.expert_bias:
            b1 = np.empty((N, f), dtype=store)
            b2 = np.empty((N, d), dtype=store)

    def fill_e(e):
        ew1, eb1, ew2, eb2 = expert_weights(shape, e, seed)
        w1[e] = ew1
        w2[e] = ew2
        if shape.expert_bias:
            b1[e] = eb1
            b2[e] = eb2

    ws1 = ws2 = None
    if shape.d_ff_shared:
        fs = shape.d_ff_shared
        ws1 = _normal_block(_rng(seed, shape, _WS1), (fs, d), d ** -0.5, dt)
        ws2 = _normal_block(_rng(seed, shape, _WS2), (d, fs), fs ** -0.5, dt)

    with ThreadPoolExecutor(nthr) as ex:
        jobs = [ex.submit(fill_x, b) for b in range(nxb)]
        if materialize_experts:
            jobs += [ex.submit(fill_e, e) for e in range(N)]
        for j in jobs:
            j.result()

    return MoEInputs(shape=shape, seed=seed, x=x, w_router=w_router, b_router=b_router,
                     logit_offset=logit_offset, sel_bias=sel_bias, w1=w1, b1=b1, w2=w2,
                     b2=b2, ws1=ws1, ws2=ws2)


def upstream_grad(shape: MoEShape, seed: int = 0) -> np.ndarray:
    """A seeded upstream gradient d_out [T, d_model] ~ N(0, 1) in the layer
    dtype (bf16 bit patterns or fp32), for the backward pass."""
    return _normal_block(_rng(seed, shape, _D_OUT), (shape.T, shape.d_model), 1.0, shape.dtype)


def to_torch(inp: MoEInputs, device) -> Dict[str, "object"]:
    """Copy the inputs to ``device`` as torch tensors (bf16 via a bit view)."""
    import torch

    def conv(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.to(device)

    out = {}
    for name in ("x", "w_router", "b_router", "logit_offset", "sel_bias",
                 "w1", "b1", "w2", "b2", "ws1", "ws2"):
        out[name] = conv(getattr(inp, name))
    return out
