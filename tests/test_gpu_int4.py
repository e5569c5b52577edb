"""GPU parity of the INT4 weight-only path.

moe_quantize_int4 must reproduce the oracle's codes (packed two per byte) and
scales bit for bit; a layer with INT4 routed experts is compared with the
oracle running the same forward on its own dequantised weights s * q, on the
decode-shaped kernel and on every tile layout of the tiled one."""
import numpy as np
import pytest

from mixture_experts_layer_prefix_amd import configs as C
from mixture_experts_layer_prefix_amd import inputs, moe
from oracle import moe_oracle as O

from moe_testlib import (BF16_TOL, check_routing_and_dispatch, device_tensors, oracle_run,
                         rel_l2, run_layer, run_stages, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    moe.lib()


def _quantize_gpu(a_f32, dtype):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(inputs.bf16_round(a_f32).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a_f32, dtype=np.float32)).cuda()
    q = torch.empty(tuple(t.shape[:-1]) + (t.shape[-1] // 2,), dtype=torch.uint8, device="cuda")
    s = torch.empty(t.shape[:-1], dtype=torch.float32, device="cuda")
    moe.moe_quantize_int4(t, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 192), (300, 1024)])
def test_quantize_bit_exact(dtype, rows, cols):
    rng = np.random.default_rng(rows * 11 + cols)
    a = (rng.standard_normal((rows, cols)) * rng.choice([1e-4, 0.03, 1.0, 300.0],
                                                        size=(rows, 1))).astype(np.float32)
    if rows > 4:
        a[1] = 0.0                                  # zero row: scale 0, codes 0
        a[2, :8] = [7, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, -7]   # exact ties at s = 1
        a[2, 8:] = 0.0
        a[3, 5] = -1e3                              # negative extreme
    if dtype == "bf16":
        a = inputs.bf16_widen(inputs.bf16_round(a))
    say(f"quantize int4 {dtype} [{rows}, {cols}]")
    p, s = _quantize_gpu(a, dtype)
    q_ref, s_ref = O.quantize_int4(a)
    assert (s.view(np.uint32) == s_ref.view(np.uint32)).all(), "scales differ"
    p_ref = O.pack_int4(q_ref)
    assert (p == p_ref).all(), f"{int((p != p_ref).sum())} code bytes differ"
    if rows > 4:
        q = O.unpack_int4(p)
        assert s[1] == 0 and (q[1] == 0).all()
        assert q[2, :8].tolist() == [7, 2, 4, -2, -4, 0, 0, -7]


CASES = {
    "tiled_ragged_w4": C.MIXTRAL_PREFILL.with_(T=300, d_model=256, d_ff=384, weight_quant="int4"),
    "tiled_bm256_w4": C.MIXTRAL_PREFILL.with_(T=1000, d_model=256, d_ff=384, n_experts=4,
                                              weight_quant="int4"),
    # 290 rows per expert (a folded 320-row tile) and Kd = 128 (four k-steps,
    # one load of INT4 code rows)
    "folded_k128_w4": C.MIXTRAL_PREFILL.with_(T=290, d_model=128, d_ff=256, n_experts=2,
                                              weight_quant="int4"),
    "capacity_aux_w4": C.SWITCH_CAPACITY.with_(T=512, d_model=128, d_ff=256, n_experts=16,
                                               weight_quant="int4"),
    "fine_shared_w4": C.DEEPSEEK_FINE.with_(T=256, d_model=256, d_ff=128, n_experts=32, top_k=4,
                                            d_ff_shared=128, weight_quant="int4"),
    "fine_shared_wide_w4": C.DEEPSEEK_FINE.with_(T=200, d_model=384, d_ff=128, n_experts=32,
                                                 top_k=4, d_ff_shared=320, weight_quant="int4"),
    "skinny_decode_w4": C.DECODE.with_(T=8, d_model=256, d_ff=512, n_experts=16,
                                       weight_quant="int4"),
    "skinny_ksplit_w4": C.DECODE.with_(T=12, d_model=256, d_ff=4096, n_experts=16,
                                       weight_quant="int4"),
    # Kd split over four wavefronts into 128-aligned parts that do not divide
    # evenly (4480 = 35 blocks of 128)
    "skinny_ksplit_ragged_w4": C.DECODE.with_(T=12, d_model=256, d_ff=4480, n_experts=16,
                                              weight_quant="int4"),
    # the first GEMM's Kd = 2048 also splits over the four wavefronts (INT4 only)
    "skinny_ksplit_gemm1_w4": C.DECODE.with_(T=10, d_model=2048, d_ff=2560, n_experts=16,
                                             weight_quant="int4"),
    "skinny_shared_w4": C.DEEPSEEK_FINE.with_(T=6, d_model=128, d_ff=256, n_experts=64, top_k=8,
                                              d_ff_shared=128, weight_quant="int4"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_int4(name):
    shape = CASES[name]
    inp = inputs.make_inputs(shape, seed=0)
    cfg = moe.config_for(shape)
    cap = cfg.capacity if cfg.capacity > 0 else None
    say(f"case {name}: T={shape.T} d={shape.d_model} f={shape.d_ff} N={shape.n_experts} "
        f"K={shape.top_k} C={cap} fs={shape.d_ff_shared}")
    t = device_tensors(inp)
    # the device codes of every expert equal the oracle's
    for e in range(shape.n_experts):
        w1, _, w2, _ = inp.expert(e)
        for name_w, w in (("w1", w1), ("w2", w2)):
            q_ref, s_ref = O.quantize_int4(inputs.bf16_widen(w))
            assert (t[name_w][e].cpu().numpy() == O.pack_int4(q_ref)).all(), (e, name_w)
            assert (t[name_w + "_scale"][e].cpu().numpy().view(np.uint32) ==
                    s_ref.view(np.uint32)).all(), (e, name_w)
    g = run_stages(cfg, t)
    o = oracle_run(inp, cap)
    check_routing_and_dispatch(g, o, inp, cap)
    err = rel_l2(g["out"], o["out"])
    say(f"  out rel-L2 {err:.3e} (tol {BF16_TOL})")
    assert err <= BF16_TOL
    # the whole-layer entry point runs the same kernels
    import torch
    lay = run_layer(cfg, t, aux=bool(shape.aux_alpha))
    assert torch.equal(lay["out"].float().cpu(), torch.from_numpy(g["out"]))
    assert (lay["counts"] == g["counts"]).all() and lay["n_dropped"] == g["n_dropped"]


@pytest.mark.parametrize("d_ff", [256, 4096])
def test_skinny_int4_expert_with_more_than_16_rows(d_ff):
    """Decode kernel with INT4 weights (four 16-row tiles per wavefront): one
    expert receives all 40 tokens, i.e. three row groups (16, 16, 8); with
    d_ff = 4096 the second GEMM also splits Kd over the wavefronts."""
    shape = C.DECODE.with_(T=40, d_model=128, d_ff=d_ff, n_experts=8, top_k=1,
                           weight_quant="int4")
    inp = inputs.make_inputs(shape, seed=0)
    off = np.zeros(8, np.float32)
    off[0] = 1e4
    inp.logit_offset = off
    cfg = moe.config_for(shape)
    say(f"case skinny_int4_40_rows: f={d_ff}")
    t = device_tensors(inp)
    g = run_stages(cfg, t)
    o = oracle_run(inp, None)
    check_routing_and_dispatch(g, o, inp, None)
    assert g["counts"][0] == 40
    err = rel_l2(g["out"], o["out"])
    say(f"  out rel-L2 {err:.3e} (tol {BF16_TOL})")
    assert err <= BF16_TOL

