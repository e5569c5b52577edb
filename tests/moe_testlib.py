"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run
the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np

from mixture_experts_layer_prefix_amd import inputs, moe
from oracle import moe_oracle as O

BF16_TOL = 1e-2     # relative L2 of the layer output, bf16 storage / fp32 accumulation
F32_TOL = 1e-5      # relative L2 of the layer output, fp32 layer
W_TOL = 1e-6        # relative error of each routing weight
AUX_TOL = 1e-5      # relative error of the aux loss
# Certified bf16 router: each logit within CERT_C0 * |x_t| * |W_r[e]| of the
# exact one (the library's own coefficient is about 34 * 2^-23), routing
# weights within CERT_W_TOL (two logits' errors through the softmax).
CERT_C0 = 40 * 2.0 ** -23
CERT_W_TOL = 1e-5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_expert_source(inp):
    def get(e):
        return tuple(None if a is None else (inputs.bf16_widen(a) if a.dtype == np.uint16 else a)
                     for a in inp.expert(e))
    return get


def oracle_expert_source_int8(inp):
    """Experts as the oracle sees them with INT8 weights: its own quantisation
    of the seeded bf16 weights, dequantised (s * q)."""
    base = oracle_expert_source(inp)

    def get(e):
        w1, b1, w2, b2 = base(e)
        q1, s1 = O.quantize_int8(w1)
        q2, s2 = O.quantize_int8(w2)
        return O.dequantize_int8(q1, s1), b1, O.dequantize_int8(q2, s2), b2
    return get


def oracle_expert_source_int4(inp):
    """The same with INT4 weights (the oracle's 4-bit quantisation)."""
    base = oracle_expert_source(inp)

    def get(e):
        w1, b1, w2, b2 = base(e)
        q1, s1 = O.quantize_int4(w1)
        q2, s2 = O.quantize_int4(w2)
        return O.dequantize_int4(q1, s1), b1, O.dequantize_int4(q2, s2), b2
    return get


def oracle_expert_source_for(inp):
    wq = getattr(inp.shape, "weight_quant", "none")
    if wq == "int8":
        return oracle_expert_source_int8(inp)
    if wq == "int4":
        return oracle_expert_source_int4(inp)
    return oracle_expert_source(inp)


def prefetching_source(get, n, window=8, workers=8):
    """An expert source that prepares experts e+1 .. e+window (widened to
    fp64) in worker threads while the caller works on expert e.  The oracle
    walks the experts in increasing order, so the conversions of the large
    layers' weights overlap its products.  Serves the same values as get."""
    from concurrent.futures import ThreadPoolExecutor

    def prep(e):
        return tuple(None if a is None else np.asarray(a, dtype=np.float64) for a in get(e))

    ex = ThreadPoolExecutor(workers)
    futs = {}

    def fetch(e):
        for j in range(e, min(n, e + window + 1)):
            if j not in futs:
                futs[j] = ex.submit(prep, j)
        r = futs.pop(e).result()
        if e % 64 == 63:
            say(f"    oracle at expert {e + 1} of {n}")
        for j in [j for j in futs if j < e]:
            futs.pop(j).cancel()
        if e == n - 1:
            ex.shutdown(wait=False)
        return r
    return fetch


def oracle_run(inp, capacity, out_tokens=None, return_y_perm=False):
    s = inp.shape
    shared = None
    if s.d_ff_shared:
        shared = (inp.f32("ws1"), inp.f32("ws2"))
    src = oracle_expert_source_for(inp)
    if s.n_experts * s.d_model * s.d_ff >= (1 << 26):
        src = prefetching_source(src, s.n_experts)
    return O.moe_forward(inp.f32("x"), inp.f32("w_router"), src, s.top_k,
                         n_experts=s.n_experts, b_router=inp.b_router,
                         logit_offset=inp.logit_offset, sel_bias=inp.sel_bias, shared=shared,
                         capacity=capacity, aux_alpha=s.aux_alpha, out_tokens=out_tokens,
                         return_y_perm=return_y_perm)


def device_tensors(inp, device="cuda"):
    t = inputs.to_torch(inp, device)
    wq = getattr(inp.shape, "weight_quant", "none")
    if wq in ("int8", "int4"):
        t = moe.quantize_expert_weights(t, bits=8 if wq == "int8" else 4)
    return t


def run_stages(cfg, t, device="cuda"):
    """Every entry point in turn; returns host numpy copies of all outputs."""
    import torch
    T, N, K, d = cfg.T, cfg.n_experts, cfg.top_k, cfg.d_model
    dt = torch.float32 if cfg.dtype == moe.MOE_F32 else torch.bfloat16
    W = moe.make_weights(t)
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    logits = torch.empty(T, N, **f32)
    idx = torch.empty(T, K, **i32)
    w = torch.empty(T, K, **f32)
    moe.moe_route(cfg, t["x"], W, logits, idx, w, moe.alloc_workspace(cfg, "route", device))
    router_path = moe.router_path(cfg)
    counts = torch.empty(N, **i32)
    offsets = torch.empty(N + 1, **i32)
    slot_row = torch.empty(T, K, **i32)
    row_token = torch.full((T * K,), -7, **i32)
    x_perm = torch.empty(T * K, d, dtype=dt, device=device)
    ndrop = torch.empty(1, **i32)
    moe.moe_dispatch(cfg, idx, t["x"], counts, offsets, slot_row, row_token, x_perm, ndrop,
                     moe.alloc_workspace(cfg, "dispatch", device))
    y_perm = torch.empty(T * K, d, dtype=dt, device=device)
    y_shared = torch.empty(T, d, dtype=dt, device=device) if cfg.d_ff_shared else None
    moe.moe_expert_ffn(cfg, x_perm, offsets, W, t["x"] if cfg.d_ff_shared else None, y_perm,
                       y_shared, moe.alloc_workspace(cfg, "expert_ffn", device))
    out = torch.empty(T, d, dtype=dt, device=device)
    moe.moe_combine(cfg, y_perm, slot_row, w, y_shared, out)
    loss = torch.empty(1, **f32)
    moe.moe_aux_loss(cfg, logits, counts, loss, moe.alloc_workspace(cfg, "aux", device))
    torch.cuda.synchronize()
    M = int(offsets[-1].item())
    res = dict(logits=logits, idx=idx, w=w, counts=counts, expert_offsets=offsets,
               slot_row=slot_row, row_token=row_token[:M], n_dropped=ndrop, out=out.float(),
               aux=loss)
    res = {k: v.cpu().numpy() for k, v in res.items()}
    res["router_path"] = router_path
    res["n_dropped"] = int(res["n_dropped"][0])
    res["aux"] = float(res["aux"][0])
    res["x_perm_ok"] = bool(torch.equal(x_perm[:M], t["x"][row_token[:M].long()]))
    res["y_perm"] = y_perm
    return res


def run_layer(cfg, t, aux=True, device="cuda"):
    import torch
    layer = moe.MoELayer(cfg, t, device)
    out, aux_t, counts, nd = layer.forward(t["x"], aux=aux)
    torch.cuda.synchronize()
    r = dict(out=out, counts=counts.cpu().numpy(), n_dropped=int(nd.item()))
    if aux:
        r["aux"] = float(aux_t.item())
    return r


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def ulp_diff_f32(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ai - bi)


def report_decision_mismatch(g_logits, o_logits, sel_bias, g_idx, o_idx):
    bad = np.nonzero((g_idx != o_idx).any(axis=1))[0]
    for t in bad[:5]:
        s = O.selection_scores(o_logits[t:t + 1], sel_bias)[0]
        srt = np.sort(s)[::-1]
        say(f"  token {t}: gpu idx {g_idx[t].tolist()} oracle idx {o_idx[t].tolist()} "
            f"score gaps {np.diff(srt[:g_idx.shape[1] + 1]).tolist()}")
    return bad


def router_logit_bound(inp):
    """Per-logit error allowance of the certified router, [T, N]."""
    def rows(a):
        a = inputs.bf16_widen(a) if a.dtype == np.uint16 else a
        return np.sqrt(np.einsum("ij,ij->i", a.astype(np.float64), a.astype(np.float64)))
    return CERT_C0 * rows(inp.x)[:, None] * rows(inp.w_router)[None, :]


def check_logits(g_logits, o_logits, inp, path):
    """Exact path: the same fp32 value (one ulp where the fp64 sum order
    differs).  Certified path: within the error allowance (plus one ulp)."""
    if path == "certified":
        g64, o64 = g_logits.astype(np.float64), o_logits.astype(np.float64)
        ulp = np.spacing(np.abs(o_logits)).astype(np.float64)
        diff = np.abs(g64 - o64)
        bound = router_logit_bound(inp)
        assert np.isfinite(g64).all() == np.isfinite(o64).all()
        fin = np.isfinite(o64)
        assert (diff[fin] <= bound[fin] + ulp[fin]).all(), \
            f"certified logits off by {np.max(diff[fin] / (bound[fin] + ulp[fin])):.3g} x the bound"
        pos = fin & (bound > 0)   # (an all-zero router has a zero bound)
        rel = np.max(diff[pos] / bound[pos]) if pos.any() else 0.0
        say(f"  certified router: logits max |err| {diff[fin].max():.3e} "
            f"({rel:.2e} of the bound), "
            f"{int((ulp_diff_f32(g_logits, o_logits) <= 1).mean() * 100)}% within one ulp")
        return
    ud = ulp_diff_f32(g_logits, o_logits)
    assert ud.max() <= 1, f"logits differ by up to {ud.max()} ulp"
    if (ud > 0).any():
        say(f"  note: {(ud > 0).sum()} logits differ by one ulp")


def check_routing_and_dispatch(g, o, inp, capacity):
    """Integer results bit-exact, floats within tolerance."""
    s = inp.shape
    path = g.get("router_path", "exact")
    check_logits(g["logits"], o["logits"], inp, path)
    # the selection and dispatch steps, applied to the GPU's own logits
    g_sel = O.topk_select(O.selection_scores(g["logits"], inp.sel_bias), s.top_k)
    assert (g_sel == g["idx"]).all(), "top-K of the GPU logits differs from the GPU idx"
    gd = O.dispatch(g["idx"], s.n_experts, capacity)
    for key in ("counts", "expert_offsets", "slot_row", "row_token"):
        assert (gd[key] == g[key]).all(), f"{key} differs from dispatch of the GPU idx"
    assert gd["n_dropped"] == g["n_dropped"]
    # independent: the oracle's own routing
    bad = report_decision_mismatch(g["logits"], o["logits"], inp.sel_bias, g["idx"], o["idx"])
    assert len(bad) == 0, f"{len(bad)} tokens routed differently"
    for key in ("counts", "expert_offsets", "slot_row", "row_token"):
        assert (o[key] == g[key]).all(), key
    assert o["n_dropped"] == g["n_dropped"]
    werr = np.abs(g["w"].astype(np.float64) - o["w"]) / np.maximum(np.abs(o["w"]), 1e-30)
    wtol = CERT_W_TOL if path == "certified" else W_TOL
    assert werr.max() <= wtol, f"routing weight rel err {werr.max()}"
    assert g["x_perm_ok"], "x_perm rows are not exact copies of x[row_token]"


def check_fused_partials(cfg, t, g, beta=1e-3, device="cuda"):
    """moe_route's routing partials give the aux loss, z-loss and routing
    statistics bit for bit equal to those formed from the logits / routing,
    and moe_layer_forward_stats (which uses them) equals the staged calls."""
    import torch
    T, N, K, d = cfg.T, cfg.n_experts, cfg.top_k, cfg.d_model
    W = moe.make_weights(t)
    f32 = dict(dtype=torch.float32, device=device)
    i32 = dict(dtype=torch.int32, device=device)
    logits = torch.empty(T, N, **f32)
    idx = torch.empty(T, K, **i32)
    w = torch.empty(T, K, **f32)
    parts = moe.alloc_route_partials(cfg, device)
    moe.moe_route(cfg, t["x"], W, logits, idx, w, moe.alloc_workspace(cfg, "route", device),
                  partials=parts)
    torch.cuda.synchronize()
    assert (logits.cpu().numpy().view(np.uint32) == g["logits"].view(np.uint32)).all()
    assert (idx.cpu().numpy() == g["idx"]).all()
    assert (w.cpu().numpy().view(np.uint32) == g["w"].view(np.uint32)).all()
    counts = torch.from_numpy(g["counts"]).to(device)
    ws = moe.alloc_workspace(cfg, "aux", device)
    alpha = cfg.aux_alpha
    if alpha == 0:
        cfg.aux_alpha = 0.01
    a_u, a_f, z_u, z_f = (torch.empty(1, **f32) for _ in range(4))
    moe.moe_aux_loss(cfg, logits, counts, a_u, ws)
    moe.moe_aux_loss(cfg, None, counts, a_f, ws, partials=parts)
    moe.moe_router_z_loss(cfg, logits, beta, z_u, ws)
    moe.moe_router_z_loss(cfg, None, beta, z_f, ws, partials=parts)
    c_u, c_f = torch.empty(N, **i32), torch.empty(N, **i32)
    m_u, m_f = torch.empty(N, **f32), torch.empty(N, **f32)
    moe.moe_routing_stats(cfg, idx, w, c_u, m_u, ws)
    moe.moe_routing_stats(cfg, None, None, c_f, m_f, ws, partials=parts)
    torch.cuda.synchronize()
    assert torch.equal(a_u, a_f), (float(a_u), float(a_f))
    assert torch.equal(z_u, z_f), (float(z_u), float(z_f))
    assert torch.equal(c_u, c_f) and torch.equal(m_u, m_f)
    assert (c_u.cpu().numpy() == g["counts"]).all()
    # the monitored layer call: same kernels, same bits
    dt = torch.float32 if cfg.dtype == moe.MOE_F32 else torch.bfloat16
    out = torch.empty(T, d, dtype=dt, device=device)
    l_aux, l_z, l_m = torch.empty(1, **f32), torch.empty(1, **f32), torch.empty(N, **f32)
    l_c, l_nd = torch.empty(N, **i32), torch.empty(1, **i32)
    moe.moe_layer_forward_stats(cfg, t["x"], W, out, aux_out=l_aux, zloss_beta=beta, zloss_out=l_z,
                                counts_out=l_c, n_dropped_out=l_nd, weight_mean_out=l_m,
                                ws=moe.alloc_workspace(cfg, "layer", device))
    torch.cuda.synchronize()
    cfg.aux_alpha = alpha
    assert torch.equal(out.float().cpu(), torch.from_numpy(g["out"]))
    assert torch.equal(l_aux, a_u) and torch.equal(l_z, z_u) and torch.equal(l_m, m_u)
    assert torch.equal(l_c, c_u) and int(l_nd.item()) == g["n_dropped"]
    return float(a_u.item()), float(z_u.item()), m_u.cpu().numpy()
