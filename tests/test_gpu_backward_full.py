"""Backward parity at the five workload sizes, in the launch configuration
`bench.py --pass train` times (moe_layer_forward_train, then
moe_layer_backward; aux-loss multiplier 1 where the workload has an aux
loss, no z-loss).

Every gradient is compared whole against the oracle's moe_backward run over
the whole batch: d_x [T, d_model], d_w_router, and every routed expert's
d_w1 / d_w2 (passed expert by expert to a sink, so the large layers' [N, f, d]
stacks are never held on the host at once; the relative L2 is taken over the
whole stack), the shared expert's d_ws1 / d_ws2; experts without rows must get
exactly zero gradients.  Routing over every token is bit-exact."""
import gc

import numpy as np
import pytest

from mixture_experts_layer_prefix_amd import configs as C
from mixture_experts_layer_prefix_amd import inputs, moe
from oracle import moe_oracle as O

from moe_testlib import (BF16_TOL, F32_TOL, device_tensors, oracle_expert_source,
                         prefetching_source, rel_l2, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", C.ALL, ids=[s.name for s in C.ALL])
def test_backward_full_size(shape):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    say(f"full-size backward {shape.name}: T={shape.T} d={shape.d_model} f={shape.d_ff} "
        f"N={shape.n_experts} K={shape.top_k} fs={shape.d_ff_shared}")
    inp = inputs.make_inputs(shape, seed=0)
    cfg = moe.config_for(shape)
    cap = cfg.capacity if cfg.capacity > 0 else None
    tol = F32_TOL if shape.dtype == "f32" else BF16_TOL
    g_aux = 1.0 if shape.aux_alpha else 0.0
    t = device_tensors(inp)
    layer = moe.MoETrainLayer(cfg, t)
    layer.forward(t["x"], aux=bool(shape.aux_alpha))
    g_np = inputs.upstream_grad(shape, seed=0)
    d_out = torch.from_numpy(g_np)
    d_out = (d_out.view(torch.bfloat16) if g_np.dtype == np.uint16 else d_out).cuda()
    d_x = layer.backward(t["x"], d_out, aux_grad=g_aux)
    torch.cuda.synchronize()
    gdx = d_x.float().cpu().numpy()
    sv = {k: layer.saved_t[k].cpu().numpy() for k in ("topk_idx", "slot_row", "counts")}
    G = layer.grads_t            # stays on the device; pulled expert by expert
    small = {k: G[k].float().cpu().numpy() for k in ("d_w_router", "d_b_router", "d_b1", "d_b2",
                                                     "d_ws1", "d_ws2") if G.get(k) is not None}
    del d_x, d_out
    say("  gpu done; oracle backward over the whole batch ...")

    get = oracle_expert_source(inp)
    if shape.n_experts * shape.d_model * shape.d_ff >= (1 << 26):
        get = prefetching_source(get, shape.n_experts)
    x = inp.f32("x").astype(np.float64)
    g_out = (inputs.bf16_widen(g_np) if g_np.dtype == np.uint16 else g_np).astype(np.float64)
    shared = (inp.f32("ws1"), inp.f32("ws2")) if shape.d_ff_shared else None

    acc = {"d_w1": [0.0, 0.0], "d_w2": [0.0, 0.0], "d_b1": [0.0, 0.0], "d_b2": [0.0, 0.0]}
    worst = {"d_w1": 0.0, "d_w2": 0.0}
    empty = []

    def sink(e, dW1, db1, dW2, db2):
        g1 = G["d_w1"][e].float().cpu().numpy().astype(np.float64)
        g2 = G["d_w2"][e].float().cpu().numpy().astype(np.float64)
        if not dW1.any() and not dW2.any():
            empty.append(e)
            assert not g1.any() and not g2.any(), f"expert {e} has no rows: gradients must be 0"
            return
        for key, got, ref in (("d_w1", g1, dW1), ("d_w2", g2, dW2)):
            num, den = float(np.sum((got - ref) ** 2)), float(np.sum(ref ** 2))
            acc[key][0] += num
            acc[key][1] += den
            worst[key] = max(worst[key], (num / den) ** 0.5 if den > 0 else 0.0)
        if "d_b1" in small:
            for key, got, ref in (("d_b1", small["d_b1"][e], db1), ("d_b2", small["d_b2"][e], db2)):
                acc[key][0] += float(np.sum((got - ref) ** 2))
                acc[key][1] += float(np.sum(ref ** 2))

    o = O.moe_backward(x, inp.f32("w_router"), get, shape.top_k, g_out,
                       n_experts=shape.n_experts, b_router=inp.b_router,
                       logit_offset=inp.logit_offset, sel_bias=inp.sel_bias, shared=shared,
                       capacity=cap, aux_alpha=shape.aux_alpha, aux_grad=g_aux,
                       expert_grad_sink=sink)
    assert (sv["topk_idx"] == o["idx"]).all() and (sv["slot_row"] == o["slot_row"]).all()
    assert (sv["counts"] == o["counts"]).all()
    say(f"  routing bit-exact; dropped {o['n_dropped']}; {len(empty)} experts without rows "
        f"(gradients exactly zero)")

    errs = {}
    for key in ("d_w1", "d_w2", "d_b1", "d_b2"):
        num, den = acc[key]
        if den > 0:
            errs[key] = (num / den) ** 0.5
    errs["d_x"] = rel_l2(gdx, o["d_x"])
    errs["d_w_router"] = rel_l2(small["d_w_router"], o["d_w_router"])
    if "d_b_router" in small:
        errs["d_b_router"] = rel_l2(small["d_b_router"], o["d_b_router"])
    if shared is not None:
        errs["d_ws1"] = rel_l2(small["d_ws1"], o["d_ws1"])
        errs["d_ws2"] = rel_l2(small["d_ws2"], o["d_ws2"])
    say("  whole-tensor rel-L2: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) +
        f"; worst expert d_w1 {worst['d_w1']:.2e}, d_w2 {worst['d_w2']:.2e} (tol {tol})")
    for k, v in errs.items():
        assert v <= tol, (k, v)
    assert worst["d_w1"] <= 4 * tol and worst["d_w2"] <= 4 * tol
    del layer, G, t, o, inp
    gc.collect()
    torch.cuda.empty_cache()
