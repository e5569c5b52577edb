"""moe_layer_forward_noalloc (the layer on the library's own device scratch,
no workspace argument) against moe_layer_forward (caller's workspace), both
through the C ABI: calls in a row, each followed by a smaller batch, every
output equal bit for bit (same kernels, same order), so whatever the previous
call left in the scratch does not leak into the next."""
import numpy as np
import pytest

from mixture_experts_layer_prefix_amd import configs as C
from mixture_experts_layer_prefix_amd import inputs, moe

pytestmark = pytest.mark.gpu

# a capacity-limited top-1 layer with the aux loss, and a fine-grained top-4
# layer with a shared expert; each at a larger and then a smaller batch (the
# smaller fine-grained batch takes the decode-shaped GEMM path); then the
# fine-grained layer again with the certified router (its own workspace
# layout in the scratch)
_FINE = dict(d_model=512, d_ff=256, n_experts=16, top_k=4, d_ff_shared=256)
CASES = [
    (C.SWITCH_CAPACITY.with_(name="noalloc_switch", T=512, d_model=256, d_ff=512, n_experts=16),
     "auto"),
    (C.SWITCH_CAPACITY.with_(name="noalloc_switch", T=64, d_model=256, d_ff=512, n_experts=16),
     "auto"),
    (C.DEEPSEEK_FINE.with_(name="noalloc_fine", T=256, **_FINE), "auto"),
    (C.DEEPSEEK_FINE.with_(name="noalloc_fine", T=24, **_FINE), "auto"),
    (C.DEEPSEEK_FINE.with_(name="noalloc_fine", T=320, **_FINE), "certified"),
    (C.DEEPSEEK_FINE.with_(name="noalloc_fine", T=40, **_FINE), "certified"),
]


def _outputs(cfg, device):
    import torch
    dt = torch.float32 if cfg.dtype == moe.MOE_F32 else torch.bfloat16
    return (torch.full((cfg.T, cfg.d_model), float("nan"), dtype=dt, device=device),
            torch.full((1,), float("nan"), dtype=torch.float32, device=device),
            torch.full((cfg.n_experts,), -1, dtype=torch.int32, device=device),
            torch.full((1,), -1, dtype=torch.int32, device=device))


def test_noalloc_layer_equals_layer_forward():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    dev = "cuda"
    for i, (shape, router) in enumerate(CASES):
        print(f"noalloc call {i}: {shape.name} T={shape.T} d={shape.d_model} f={shape.d_ff} "
              f"N={shape.n_experts} K={shape.top_k} fs={shape.d_ff_shared} router={router}",
              flush=True)
        inp = inputs.make_inputs(shape, seed=i)
        t = inputs.to_torch(inp, dev)
        cfg = moe.config_for(shape, router=router)
        assert moe.workspace_size(cfg, "layer") <= moe.NOALLOC_SCRATCH_BYTES
        W = moe.make_weights(t)
        aux = bool(shape.aux_alpha)
        ref, ref_aux, ref_cnt, ref_nd = _outputs(cfg, dev)
        moe.moe_layer_forward(cfg, t["x"], W, ref, ref_aux if aux else None, ref_cnt, ref_nd,
                              moe.alloc_workspace(cfg, "layer", dev))
        got, got_aux, got_cnt, got_nd = _outputs(cfg, dev)
        moe.moe_layer_forward_noalloc(cfg, t["x"], W, got, got_aux if aux else None, got_cnt,
                                      got_nd)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got, ref), f"call {i}: outputs differ"
        assert torch.equal(got_cnt, ref_cnt) and torch.equal(got_nd, ref_nd), f"call {i}: counts"
        if aux:
            assert torch.equal(got_aux, ref_aux), f"call {i}: aux loss"
        print(f"  equal bit for bit; dropped {int(got_nd.item())}", flush=True)
        # a second call on the same inputs reproduces the first
        again = torch.empty_like(got)
        moe.moe_layer_forward_noalloc(cfg, t["x"], W, again)
        torch.cuda.synchronize()
        assert torch.equal(again, got), f"call {i}: repeat differs"
