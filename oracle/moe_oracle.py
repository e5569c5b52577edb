"""CPU oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or call this module.  The GPU library never routes through it, and it
shares no code, tables or constants with the GPU path.

Plain, slow, fp64 NumPy.  Each function cites the page passage it follows.
Pages (by site and title):
  [lmnt]   lmnt.cn MoE walkthrough (news/351908): §1.2 per-token flow,
           §2.1 gate scoring equation, §2.2 TopK, §3.1 dispatch, §3.2 combine
           equation, §3.3 capacity equation, §4.3 weight quantisation for
           inference (INT8 or INT4), §5.2 load-balance code, §5.3 router z-loss equation,
           §8.2 routing statistics.
  [csdn]   "MoE逐token路由与活跃参数率实战解析": §3.1 worked top-2 example,
           §4.2 MoELayer code.
  [yunthe] "MoE混合专家模型实战：专家路由与稀疏激活的推理成本优化方案":
           section "MoE架构的稀疏激活原理与Transformer实现" (output equation,
           reference forward), section "专家负载均衡与辅助损失函数设计"
           (Switch aux loss, per-expert bias b_i, capacity drop).
  [wiblog] "MoE 专家路由如何实现稀疏激活": section on fine-grained and shared
           experts.

Readings taken where the pages are silent or disagree (all in the design
notes as well):
  * logits are the fp32 rounding of the dot product computed in fp64, plus
    the router bias and logit offset added in fp64 before that one rounding;
  * top-K orders by (score descending, expert index ascending); NaN scores
    order as -inf; a per-expert selection bias changes only the choice, the
    weights use the unbiased logits;
  * capacity drops keep, per expert, the first C (token, slot) pairs in token
    order; a dropped pair contributes zero and the remaining weights are not
    renormalised;
  * GELU is the exact erf form; the shared expert enters with weight 1;
  * aux loss f_e is the mean over tokens of the pre-drop selection mask
    ([yunthe] form, sum f = K), P_e the mean full-N softmax of the logits;
  * INT8 weight-only experts: symmetric, one fp32 scale per output row,
    s = maxabs / 127 and q = round-half-even(w / s) clamped to +-127, both
    divisions in fp32; the expert then uses the weights s * q;
  * INT4 weight-only experts: the same with 7 for 127 (codes in [-7, 7]),
    stored two per byte (element 2i in the low nibble of byte i);
  * backward: the gradient of the forward above with the Top-K choice and the
    capacity drops held fixed, the logits' fp32 rounding taken as the
    identity, selection bias, logit offsets and the aux loss's f constant.

Pins: every function here is pinned by tests/test_oracle_pins.py (the
backward by tests/test_oracle_backward_pins.py: central finite differences of
the forward, torch.autograd of an independently written forward, and
invariants) against brute force, closed forms, the corrected worked example,
special cases and textbook routines.  Absolute output values at the large workload sizes are
"parity unpinned" beyond that: the pages print none, and the oracle runs the
same code at every size.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Callable, Optional, Sequence, Union

import numpy as np

try:  # exact erf, vectorised
    from scipy.special import erf as _erf
except Exception:  # pragma: no cover - scipy is present in this image
    _erf = np.vectorize(math.erf, otypes=[np.float64])


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# a1: router scoring.  [lmnt] §2.1: scores come from W_g . x, W_g being
# d_model x N; [yunthe] reference forward: the router is a Linear layer
# (with bias in nn.Linear's default form).
def router_logits(x, w_router, b_router=None, logit_offset=None,
                  round_fp32: bool = True) -> np.ndarray:
    """logits[t, e] = fp32( sum_j x[t, j] * W_r[e, j] + b_r[e] + off[e] ).

    x: [T, d]; w_router: [N, d] (nn.Linear [out, in]); b_router, logit_offset: [N]
    or None.  Products and sums in fp64; one rounding to fp32 at the end
    (round_fp32=False keeps the fp64 value: the gradient pins differentiate
    the unrounded function)."""
    z = _f64(x) @ _f64(w_router).T
    if b_router is not None:
        z = z + _f64(b_router)[None, :]
    if logit_offset is not None:
        z = z + _f64(logit_offset)[None, :]
    return z.astype(np.float32) if round_fp32 else z


# --------------------------------------------------------------------------
# a2: TopK first, then softmax over the K chosen logits.
# [lmnt] §2.1 (score = Softmax(TopK(W_g x)); the K logits are normalised within
# the candidate set); [yunthe] reference forward (topk then F.softmax over the
# K values); [yunthe] load-balancing section: a per-expert bias b_i adjusts the
# routing score.
def selection_scores(logits: np.ndarray, sel_bias=None) -> np.ndarray:
    """s = fp32(logits + b) (selection only); s = logits when b is None."""
    s = np.asarray(logits, dtype=np.float32)
    if sel_bias is not None:
        s = (s + np.asarray(sel_bias, dtype=np.float32)[None, :]).astype(np.float32)
    return s


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """idx[t, :] = the k experts with the largest score, ordered by
    (score descending, expert index ascending).  NaN orders as -inf."""
    s = np.asarray(scores, dtype=np.float64).copy()
    s[np.isnan(s)] = -np.inf
    T, N = s.shape
    if not (1 <= k <= N):
        raise ValueError("need 1 <= k <= N")
    expert = np.broadcast_to(np.arange(N), (T, N))
    # lexsort: last key is primary -> primary -s ascending, then expert ascending
    order = np.lexsort((expert, -s), axis=-1)
    return order[:, :k].astype(np.int32)


def topk_softmax(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t, k] = exp(l[t, idx_k]) / sum_k' exp(l[t, idx_k']) over the K chosen
    (unbiased) logits, in fp64."""
    sel = np.take_along_axis(_f64(logits), idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return e / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# a3: dispatch with an optional capacity.
# [lmnt] §3.1 (reorder from token order to contiguous per-expert blocks),
# §3.3 (capacity = ceil(T / N * capacity_factor); over-capacity tokens skip the
# expert and pass on through the residual).
def capacity_from_factor(T: int, n_experts: int, capacity_factor: float) -> int:
    """ceil(T / N * capacity_factor), in exact rational arithmetic."""
    return math.ceil(Fraction(T, n_experts) * Fraction(capacity_factor))


def dispatch(idx: np.ndarray, n_experts: int, capacity: Optional[int] = None) -> dict:
    """Enumerate (token, slot) pairs token-major; within each expert keep pairs
    in token order; a pair is kept iff fewer than ``capacity`` earlier pairs
    went to its expert.  Returns
      counts [N]          pre-drop pairs per expert,
      kept [N]            min(counts, C),
      expert_offsets [N+1] exclusive scan of kept,
      slot_row [T, K]     row of the pair in the permuted buffer, -1 if dropped,
      row_token [M]       token of each permuted row (M = kept total),
      n_dropped           T*K - M."""
    idx = np.asarray(idx)
    T, K = idx.shape
    N = n_experts
    counts = np.zeros(N, dtype=np.int64)
    pos = np.zeros((T, K), dtype=np.int64)
    for t in range(T):               # token order ...
        for k in range(K):           # ... then slot order within the token
            e = int(idx[t, k])
            pos[t, k] = counts[e]
            counts[e] += 1
    cap = np.iinfo(np.int64).max if capacity is None or capacity <= 0 else int(capacity)
    kept = np.minimum(counts, cap)
    offsets = np.zeros(N + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    M = int(offsets[-1])
    slot_row = np.full((T, K), -1, dtype=np.int64)
    row_token = np.full(M, -1, dtype=np.int64)
    for t in range(T):
        for k in range(K):
            if pos[t, k] < cap:
                r = offsets[idx[t, k]] + pos[t, k]
                slot_row[t, k] = r
                row_token[r] = t
    return dict(counts=counts.astype(np.int32), kept=kept.astype(np.int32),
                expert_offsets=offsets.astype(np.int32), slot_row=slot_row.astype(np.int32),
                row_token=row_token.astype(np.int32), n_dropped=int(T * K - M))


# --------------------------------------------------------------------------
# a4/a5: expert FFN = Linear -> GELU -> Linear.  [yunthe] reference forward
# (nn.Linear(d_model, d_ff), nn.GELU(), nn.Linear(d_ff, d_model)); [csdn] §4.2
# create_simple_moe_layer (same form).  nn.GELU's default is the erf form.
def gelu(z):
    """GELU(z) = z/2 * (1 + erf(z / sqrt(2)))."""
    z = _f64(z)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def expert_ffn(x_rows, w1, b1, w2, b2):
    """E(x) = W2 . GELU(W1 . x + b1) + b2 for each row; W1 [f, d], W2 [d, f]."""
    h = _f64(x_rows) @ _f64(w1).T
    if b1 is not None:
        h = h + _f64(b1)[None, :]
    y = gelu(h) @ _f64(w2).T
    if b2 is not None:
        y = y + _f64(b2)[None, :]
    return y


# --------------------------------------------------------------------------
# a7: Switch auxiliary loss.  [yunthe] "专家负载均衡与辅助损失函数设计":
# alpha * N * sum(f * P), f = mean over tokens of the 0/1 selection mask,
# P = mean over tokens of the softmax router probabilities; [lmnt] §5.1-5.2
# (same product, P from the full softmax of the router logits).
def aux_loss(logits: np.ndarray, idx: np.ndarray, n_experts: int, alpha: float) -> float:
    T, K = idx.shape
    N = n_experts
    mask = np.zeros((T, N), dtype=np.float64)
    for k in range(K):
        mask[np.arange(T), idx[:, k]] = 1.0
    f = mask.mean(axis=0)
    z = _f64(logits)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    return float(alpha * N * np.sum(f * P))


# [lmnt] §5.3 router z-loss: beta * mean_t (logsumexp_e logits[t, e])^2.
def router_z_loss(logits: np.ndarray, beta: float) -> float:
    z = _f64(logits)
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    return float(beta * np.mean(lse ** 2))


# [lmnt] §8.2 routing-distribution monitoring: tokens received per expert and
# their mean routing weight (the drop count is the dispatch's).
def routing_stats(idx: np.ndarray, w: np.ndarray, n_experts: int):
    T, K = idx.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    wsum = np.zeros(n_experts, dtype=np.float64)
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            counts[e] += 1
            wsum[e] += float(w[t, k])
    mean = np.where(counts > 0, wsum / np.maximum(counts, 1), 0.0)
    return counts, mean


# --------------------------------------------------------------------------
# [lmnt] §4.3 (inference: expert weights compressed from 16-bit to INT8 halve
# their memory and bandwidth); [yunthe] deployment section (weight-only
# quantisation of the experts).  The pages fix no scheme; the reading here is
# the plain symmetric per-output-channel one, decided in fp32 so the GPU can
# reproduce every code exactly:
#   s[r] = fp32(maxabs_k |w[r, k]| / 127),  q[r, k] = rint(fp32(w[r, k] / s[r]))
# clamped to [-127, 127]; a row of zeros gets s = 0 and q = 0.
def quantize_int8(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows = w.reshape(-1, w.shape[-1])
    m = np.abs(rows).max(axis=1)                           # exact in fp32
    s = (m / np.float32(127.0)).astype(np.float32)         # fp32 division
    div = np.where(s > 0, s, np.float32(1.0))
    v = np.rint(rows / div[:, None])                       # fp32 division, half to even
    v[s == 0] = 0                                          # a row of zeros: s = 0, q = 0
    q = np.clip(v, -127, 127).astype(np.int8)
    return q.reshape(w.shape), s.reshape(w.shape[:-1])


def dequantize_int8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return _f64(s)[..., None] * q.astype(np.float64)


# [lmnt] §4.3 names INT4 beside INT8 for the expert weights (a quarter of the
# 16-bit memory and bandwidth); [yunthe] deployment section cites 4-bit
# weight-only formats.  The pages fix no scheme; the reading here is the INT8
# one above with 4-bit codes, decided in fp32:
#   s[r] = fp32(maxabs_k |w[r, k]| / 7),  q[r, k] = rint(fp32(w[r, k] / s[r]))
# clamped to [-7, 7]; a row of zeros gets s = 0 and q = 0.  The expert uses
# the weights s * q.
def quantize_int4(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows = w.reshape(-1, w.shape[-1])
    m = np.abs(rows).max(axis=1)                           # exact in fp32
    s = (m / np.float32(7.0)).astype(np.float32)           # fp32 division
    div = np.where(s > 0, s, np.float32(1.0))
    v = np.rint(rows / div[:, None])                       # fp32 division, half to even
    v[s == 0] = 0
    q = np.clip(v, -7, 7).astype(np.int8)
    return q.reshape(w.shape), s.reshape(w.shape[:-1])


def dequantize_int4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return _f64(s)[..., None] * q.astype(np.float64)


# Storage of 4-bit codes: two per byte along the row, element 2i in the low
# nibble and element 2i+1 in the high nibble of byte i, each as a 4-bit two's
# complement number.
def pack_int4(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.int8)
    if q.shape[-1] % 2:
        raise ValueError("the row length must be even")
    lo = q[..., 0::2].astype(np.uint8) & np.uint8(0x0F)
    hi = q[..., 1::2].astype(np.uint8) & np.uint8(0x0F)
    return (lo | (hi << np.uint8(4))).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & np.uint8(0x0F)).astype(np.int8)
    hi = (p >> np.uint8(4)).astype(np.int8)
    lo = np.where(lo >= 8, lo - 16, lo).astype(np.int8)
    hi = np.where(hi >= 8, hi - 16, hi).astype(np.int8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# --------------------------------------------------------------------------
# The whole layer.  [lmnt] §3.2 combine equation: output[t] = sum over the
# experts e selected for t of weight[t, e] * E_e(x_t).  Each expert runs once
# on the batch of all tokens routed to it ([yunthe] reference forward: the
# rows that chose expert e are gathered with a boolean mask and passed
# through E_e together; the note after it: production code batches the tokens
# of one expert), and w * E_e(x) is added into those tokens' rows; the
# capacity mask of [lmnt] §3.3 removes dropped pairs; a shared expert
# ([wiblog], shared-expert isolation) is added for every token.  A token
# selects an expert at most once, so within one expert every token appears in
# at most one row.  The K terms of a token are added in expert order (in
# fp64; in exact arithmetic the sum does not depend on the order).
ExpertSource = Union[Sequence, Callable[[int], tuple]]


def moe_forward(x, w_router, experts: ExpertSource, top_k: int, *, n_experts: Optional[int] = None,
                b_router=None, logit_offset=None, sel_bias=None, shared=None,
                capacity: Optional[int] = None, aux_alpha: float = 0.0,
                out_tokens: Optional[np.ndarray] = None, round_logits: bool = True,
                return_y_perm: bool = False) -> dict:
    """experts: sequence of (W1 [f, d], b1 [f] | None, W2 [d, f], b2 [d] | None)
    or a callable e -> that tuple.  shared: None or (Ws1 [f_s, d], Ws2 [d, f_s]).
    capacity: None or <= 0 for dropless, else C.  out_tokens: compute ``out``
    only for these token indices (other rows stay 0); routing, dispatch and the
    aux loss always cover every token.  return_y_perm: also return
    ``y_perm`` [M, d], the expert output of every kept pair at its dispatch
    row (y_perm[slot_row[t, k]] = E_{idx[t, k]}(x_t); rows of tokens outside
    out_tokens stay 0)."""
    x64 = _f64(x)
    T = x64.shape[0]
    N = n_experts if n_experts is not None else np.asarray(w_router).shape[0]
    get = experts if callable(experts) else (lambda e: experts[e])

    logits = router_logits(x64, w_router, b_router, logit_offset, round_fp32=round_logits)
    scores = selection_scores(logits, sel_bias) if round_logits else (
        logits if sel_bias is None else logits + _f64(sel_bias)[None, :])
    idx = topk_select(scores, top_k)
    w = topk_softmax(logits, idx)
    disp = dispatch(idx, N, capacity)
    kept_pair = disp["slot_row"] >= 0

    active = np.zeros(T, dtype=bool)
    if out_tokens is None:
        active[:] = True
    else:
        active[np.asarray(out_tokens)] = True

    out = np.zeros_like(x64)
    y_perm = np.zeros((int(disp["expert_offsets"][-1]), x64.shape[1])) if return_y_perm else None
    for e in range(N):
        # the (token, slot) pairs routed to e, kept, and of an active token
        tok, slot = np.nonzero((idx == e) & kept_pair & active[:, None])
        if tok.size == 0:
            continue
        w1, b1, w2, b2 = get(e)
        y = expert_ffn(x64[tok], w1, b1, w2, b2)
        out[tok] += w[tok, slot][:, None] * y
        if y_perm is not None:
            y_perm[disp["slot_row"][tok, slot]] = y
    if shared is not None:
        ws1, ws2 = shared
        out[active] += expert_ffn(x64[active], ws1, None, ws2, None)

    res = dict(logits=logits, scores=scores, idx=idx, w=w, out=out, **disp)
    if y_perm is not None:
        res["y_perm"] = y_perm
    if aux_alpha:
        res["aux"] = aux_loss(logits, idx, N, aux_alpha)
    return res


# --------------------------------------------------------------------------
# Backward pass (training).  [lmnt] §2.2: in training the K routing weights
# take part in back-propagation, which is how the gate learns its scores;
# §5.1-5.2: the balance loss reaches the gate through the probabilities P;
# §5.3: the z-loss constrains only the router scores; §4.1: under mixed
# precision the gradients are kept in 16 bits like the weights; §6.2: an
# expert that receives no tokens gets no gradient.
#
# What is differentiated is the forward defined above, with the Top-K choice
# and the capacity drops held at their forward values (both are piecewise
# constant in the inputs), the fp32 rounding of the logits taken as the
# identity, the selection bias and logit offsets constants, and the aux
# loss's f_e (a count) constant.  The scalar differentiated is
#   L = <d_out, out> + g_aux * aux + g_z * zloss
# so d_out is the upstream gradient of the layer output and g_aux, g_z those
# of the two losses.
def gelu_grad(z):
    """d/dz GELU(z) = Phi(z) + z * phi(z) (erf form)."""
    z = _f64(z)
    return 0.5 * (1.0 + _erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def expert_ffn_backward(x_rows, w1, b1, w2, g_y):
    """Backward of E(x) = W2 . GELU(W1 . x + b1) + b2 for a block of rows.

    g_y: [R, d] gradient of the rows' outputs.  Returns (g_x [R, d], dW1 [f, d],
    db1 [f], dW2 [d, f], db2 [d]); every sum over rows in fp64."""
    x64, g_y = _f64(x_rows), _f64(g_y)
    z = x64 @ _f64(w1).T
    if b1 is not None:
        z = z + _f64(b1)[None, :]
    h = gelu(z)
    dW2 = g_y.T @ h
    db2 = g_y.sum(axis=0)
    g_h = g_y @ _f64(w2)
    g_z = g_h * gelu_grad(z)
    dW1 = g_z.T @ x64
    db1 = g_z.sum(axis=0)
    g_x = g_z @ _f64(w1)
    return g_x, dW1, db1, dW2, db2


def topk_softmax_backward(w: np.ndarray, d_w: np.ndarray) -> np.ndarray:
    """Gradient of the K selected logits from that of w = softmax(selected):
    d_l_j = w_j * (d_w_j - sum_k w_k d_w_k)."""
    w, d_w = _f64(w), _f64(d_w)
    return w * (d_w - (w * d_w).sum(axis=1, keepdims=True))


def aux_loss_logit_grad(logits: np.ndarray, counts, alpha: float) -> np.ndarray:
    """d aux / d logits[t, e] = alpha * N / T * p_te * (f_e - sum_e' f_e' p_te'),
    p_t = softmax_N(logits_t), f_e = counts_e / T held constant."""
    z = _f64(logits)
    T, N = z.shape
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    f = _f64(counts) / T
    return alpha * N / T * p * (f[None, :] - (p @ f)[:, None])


def router_z_loss_logit_grad(logits: np.ndarray, beta: float) -> np.ndarray:
    """d (beta * mean_t lse_t^2) / d logits[t, e] = 2 beta / T * lse_t * p_te."""
    z = _f64(logits)
    T = z.shape[0]
    m = z.max(axis=1, keepdims=True)
    s = np.exp(z - m).sum(axis=1, keepdims=True)
    lse = m + np.log(s)
    p = np.exp(z - m) / s
    return 2.0 * beta / T * lse * p


def moe_backward(x, w_router, experts: ExpertSource, top_k: int, d_out, *,
                 n_experts: Optional[int] = None, b_router=None, logit_offset=None,
                 sel_bias=None, shared=None, capacity: Optional[int] = None,
                 aux_alpha: float = 0.0, aux_grad: float = 1.0, zloss_beta: float = 0.0,
                 zloss_grad: float = 1.0, round_logits: bool = True,
                 expert_grad_sink: Optional[Callable] = None) -> dict:
    """Gradients of L = <d_out, out> + aux_grad * aux + zloss_grad * zloss.

    Same arguments as moe_forward plus d_out [T, d].  Returns d_x [T, d],
    d_w_router [N, d], d_b_router [N], d_w1 [N, f, d], d_b1 [N, f],
    d_w2 [N, d, f], d_b2 [N, d], d_ws1, d_ws2 (shared, or None), d_topk_w [T, K]
    (zero for dropped slots), d_logits [T, N] and the forward's routing.
    expert_grad_sink: when given, called as sink(e, dW1, db1, dW2, db2) with
    each routed expert's gradients (an expert without rows gets zeros), and
    d_w1, d_b1, d_w2, d_b2 are not returned (the large layers' [N, f, d]
    stacks need not be held at once)."""
    x64, g_out = _f64(x), _f64(d_out)
    T, d = x64.shape
    N = n_experts if n_experts is not None else np.asarray(w_router).shape[0]
    get = experts if callable(experts) else (lambda e: experts[e])
    logits = router_logits(x64, w_router, b_router, logit_offset, round_fp32=round_logits)
    scores = selection_scores(logits, sel_bias) if round_logits else (
        logits if sel_bias is None else logits + _f64(sel_bias)[None, :])
    idx = topk_select(scores, top_k)
    w = topk_softmax(logits, idx)
    disp = dispatch(idx, N, capacity)
    kept_pair = disp["slot_row"] >= 0

    d_x = np.zeros_like(x64)
    d_w = np.zeros((T, top_k))
    e0 = get(0)
    f = np.asarray(e0[0]).shape[0]
    if expert_grad_sink is None:
        d_w1 = np.zeros((N, f, d))
        d_b1 = np.zeros((N, f))
        d_w2 = np.zeros((N, d, f))
        d_b2 = np.zeros((N, d))
    # as in the forward, each expert takes the batch of all (kept) rows routed
    # to it; a token appears at most once per expert
    for e in range(N):
        tok, slot = np.nonzero((idx == e) & kept_pair)
        if tok.size == 0:
            if expert_grad_sink is not None:
                expert_grad_sink(e, np.zeros((f, d)), np.zeros(f), np.zeros((d, f)), np.zeros(d))
            continue
        w1, b1, w2, b2 = get(e)
        y = expert_ffn(x64[tok], w1, b1, w2, b2)
        d_w[tok, slot] = (g_out[tok] * y).sum(axis=1)
        g_y = w[tok, slot][:, None] * g_out[tok]
        g_x, dW1, db1, dW2, db2 = expert_ffn_backward(x64[tok], w1, b1, w2, g_y)
        d_x[tok] += g_x
        if expert_grad_sink is not None:
            expert_grad_sink(e, dW1, db1, dW2, db2)
        else:
            d_w1[e] = dW1
            d_b1[e] = db1
            d_w2[e] = dW2
            d_b2[e] = db2
    d_ws1 = d_ws2 = None
    if shared is not None:
        ws1, ws2 = shared
        g_x, d_ws1, _, d_ws2, _ = expert_ffn_backward(x64, ws1, None, ws2, g_out)
        d_x += g_x

    d_logits = np.zeros((T, N))
    np.put_along_axis(d_logits, idx.astype(np.int64), topk_softmax_backward(w, d_w), axis=1)
    if aux_alpha:
        d_logits += aux_grad * aux_loss_logit_grad(logits, disp["counts"], aux_alpha)
    if zloss_beta:
        d_logits += zloss_grad * router_z_loss_logit_grad(logits, zloss_beta)
    d_x += d_logits @ _f64(w_router)
    res = dict(d_x=d_x, d_w_router=d_logits.T @ x64, d_b_router=d_logits.sum(axis=0),
               d_ws1=d_ws1, d_ws2=d_ws2, d_topk_w=d_w, d_logits=d_logits, logits=logits,
               idx=idx, w=w, **disp)
    if expert_grad_sink is None:
        res.update(d_w1=d_w1, d_b1=d_b1, d_w2=d_w2, d_b2=d_b2)
    return res
