"""Seeded input generators (no GPU)."""
import numpy as np
import torch

from mixture_experts_layer_prefix_amd import configs, inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-8, 8, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38, 1e-40], np.float32)])
    ours = inputs.bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = inputs.bf16_widen(ours)
    assert (back == torch.from_numpy(a).to(torch.bfloat16).float().numpy()).all()


def test_make_inputs_is_deterministic_and_lazy_experts_match():
    s = configs.TINY_FP32.with_(d_ff_shared=32, logit_offset="zipf", sel_bias=True)
    a = inputs.make_inputs(s, seed=3)
    b = inputs.make_inputs(s, seed=3, materialize_experts=False, threads=1)
    assert (a.x == b.x).all() and (a.w_router == b.w_router).all()
    for e in range(s.n_experts):
        for u, v in zip(a.expert(e), b.expert(e)):
            assert (u == v).all()
    c = inputs.make_inputs(s, seed=4)
    assert not (a.x == c.x).all()


def test_shapes_dtypes_and_distributions():
    s = configs.MIXTRAL_PREFILL.with_(T=512, d_model=256, d_ff=512)
    inp = inputs.make_inputs(s)
    assert inp.x.dtype == np.uint16 and inp.x.shape == (512, 256)
    assert inp.w1.shape == (8, 512, 256) and inp.w2.shape == (8, 256, 512)
    x = inp.f32("x")
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    w1 = inp.f32("w1")
    assert abs(w1.std() * 256 ** 0.5 - 1) < 0.01
    z = inputs.make_inputs(configs.SWITCH_CAPACITY.with_(T=16, d_model=64, d_ff=64), materialize_experts=False)
    np.testing.assert_allclose(np.sort(z.logit_offset),
                               np.sort((np.arange(1, 65, dtype=np.float64) ** -1.1).astype(np.float32)))
    u = inputs.make_inputs(configs.DEEPSEEK_FINE.with_(T=8, d_model=64, d_ff=64, d_ff_shared=64),
                           materialize_experts=False)
    assert u.sel_bias.shape == (256,) and (np.abs(u.sel_bias) <= 0.5).all()
    assert u.ws1.shape == (64, 64) and u.ws2.shape == (64, 64)
