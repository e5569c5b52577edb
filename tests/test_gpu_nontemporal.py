"""The combine, combine-backward and unpermute kernels load per-slot rows
non-temporally when those rows exceed half of the MALL; that choice changes
the cache policy of the loads, never the arithmetic.  With the threshold
forced to 0 (MOE_NONTEMPORAL_ROWS_BYTES=0, read on every launch) the small
layers below take the non-temporal variants of every K bucket (1, 2, 4, 8)
in fp32 and bf16; forward outputs, d_x and every gradient must equal the
default variants bit for bit, and the forward output must match the oracle."""
import os

import numpy as np
import pytest

from mixture_experts_layer_prefix_amd import configs as C
from mixture_experts_layer_prefix_amd import inputs, moe

from moe_testlib import BF16_TOL, F32_TOL, device_tensors, oracle_run, rel_l2, say

pytestmark = pytest.mark.gpu

ENV = "MOE_NONTEMPORAL_ROWS_BYTES"

CASES = {
    "k1_bf16": C.SWITCH_CAPACITY.with_(T=256, d_model=128, d_ff=256, n_experts=16),
    "k2_bf16": C.MIXTRAL_PREFILL.with_(T=200, d_model=256, d_ff=384),
    "k4_bf16_shared": C.DEEPSEEK_FINE.with_(T=96, d_model=128, d_ff=128, n_experts=16, top_k=4,
                                            d_ff_shared=128),
    "k8_bf16": C.DEEPSEEK_FINE.with_(T=64, d_model=128, d_ff=64, n_experts=32, top_k=8,
                                     d_ff_shared=0),
    "k2_fp32": C.TINY_FP32,
    "k4_fp32": C.TINY_FP32.with_(T=48, top_k=4),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    moe.lib()


def _run(cfg, t, g_out, aux):
    import torch
    layer = moe.MoETrainLayer(cfg, t)
    out, _ = layer.forward(t["x"], aux=aux)
    d_x = layer.backward(t["x"], g_out, aux_grad=1.0 if aux else 0.0)
    fwd = moe.MoELayer(cfg, t).forward(t["x"], aux=aux)[0]
    torch.cuda.synchronize()
    return out.clone(), fwd.clone(), d_x.clone(), {k: v.clone() for k, v in layer.grads_t.items()}


@pytest.mark.parametrize("name", sorted(CASES))
def test_nontemporal_rows_same_bits(name):
    import torch
    shape = CASES[name]
    inp = inputs.make_inputs(shape, seed=0)
    cfg = moe.config_for(shape)
    t = device_tensors(inp)
    g_np = inputs.upstream_grad(shape, seed=0)
    g_out = torch.from_numpy(g_np)
    g_out = (g_out.view(torch.bfloat16) if g_np.dtype == np.uint16 else g_out).cuda()
    aux = bool(shape.aux_alpha)
    say(f"case {name}: T={shape.T} K={shape.top_k} dtype={shape.dtype}")
    old = os.environ.pop(ENV, None)
    try:
        a = _run(cfg, t, g_out, aux)
        os.environ[ENV] = "0"
        b = _run(cfg, t, g_out, aux)
    finally:
        os.environ.pop(ENV, None)
        if old is not None:
            os.environ[ENV] = old
    for i, what in enumerate(("training forward out", "forward out", "d_x")):
        assert torch.equal(a[i], b[i]), what
    for k in a[3]:
        assert torch.equal(a[3][k], b[3][k]), k
    cap = cfg.capacity if cfg.capacity > 0 else None
    o = oracle_run(inp, cap)
    tol = F32_TOL if shape.dtype == "f32" else BF16_TOL
    err = rel_l2(b[1].float().cpu().numpy(), o["out"])
    say(f"  non-temporal variants equal bit for bit; out rel-L2 {err:.2e}")
    assert err <= tol
