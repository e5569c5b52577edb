"""GPU parity of the certified bf16 router (MOE_ROUTER_CERTIFIED): the bf16
matrix-core logits with their error bound, the certification of each token's
Top-K and the fp64 recomputation of the open dot products.

Routing decisions (idx, dispatch) must be bit-exact against the oracle and
against the exact fp64 router; logits within the stated bound; routing
weights within 1e-5.  The cases force the recomputation: rows of W_r that
differ in one bf16 ulp of one element (near ties far inside the bound),
duplicated rows (exact ties, broken by index), an all-zero router, tokens with
non-finite values (whole-row recomputation), and ragged T / N."""
import numpy as np
import pytest

from mixture_experts_layer_prefix_amd import configs as C
from mixture_experts_layer_prefix_amd import inputs, moe

from moe_testlib import (check_routing_and_dispatch, device_tensors, oracle_run,
                         router_logit_bound, run_stages, say, ulp_diff_f32)
from test_gpu_parity import CASES, _compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    moe.lib()


BF16_CASES = [n for n, s in CASES.items() if s.dtype == "bf16"]


@pytest.mark.parametrize("name", BF16_CASES)
def test_certified_small_cases(name):
    shape = CASES[name]
    inp = inputs.make_inputs(shape, seed=0)
    cfg = moe.config_for(shape, router="certified")
    assert moe.router_path(cfg) == "certified"
    _compare(name + "_certified", shape, inp, cfg)


def _both_paths(shape, inp, cap=None):
    """Certified and exact routers on the same inputs; decisions identical to
    each other and to the oracle."""
    t = device_tensors(inp)
    gc_ = run_stages(moe.config_for(shape, router="certified"), t)
    ge = run_stages(moe.config_for(shape, router="exact"), t)
    assert gc_["router_path"] == "certified" and ge["router_path"] == "exact"
    o = oracle_run(inp, cap)
    check_routing_and_dispatch(gc_, o, inp, cap)
    check_routing_and_dispatch(ge, o, inp, cap)
    for key in ("idx", "counts", "expert_offsets", "slot_row", "row_token"):
        assert (gc_[key] == ge[key]).all(), key
    # tokens whose chosen logits match the exact path bit for bit (the
    # recomputed ones, and certified ones whose approximation rounds the same)
    chosen_c = np.take_along_axis(gc_["logits"], gc_["idx"], axis=1)
    chosen_e = np.take_along_axis(ge["logits"], ge["idx"], axis=1)
    same = (ulp_diff_f32(chosen_c, chosen_e) == 0).all(axis=1)
    say(f"  {int(same.sum())} of {shape.T} tokens: chosen logits equal to the exact path's")
    return gc_, ge, o


def test_near_ties_one_ulp_rows():
    """Pairs of router rows one bf16 ulp apart in one element: the logit gap
    (~1e-4) is inside the error bound, so these tokens are recomputed."""
    shape = C.DEEPSEEK_FINE.with_(T=700, d_model=1024, d_ff=64, n_experts=64, top_k=4,
                                  d_ff_shared=0)
    inp = inputs.make_inputs(shape, seed=3)
    w = inp.w_router.copy()
    for a in range(0, 64, 2):
        w[a + 1] = w[a]
        j = (7 * a) % 1024
        w[a + 1, j] = w[a, j] + 1            # next bf16 value (same sign, larger magnitude)
    inp.w_router = w
    say("case near ties: 32 pairs of rows one bf16 ulp apart")
    gc_, ge, o = _both_paths(shape, inp)
    # both members of a pair chosen together is common; their order decides slots
    pairs = (gc_["idx"][:, :-1] // 2 == gc_["idx"][:, 1:] // 2).any(axis=1)
    say(f"  {int(pairs.sum())} tokens chose both rows of a pair")
    assert pairs.sum() > 0


def test_duplicated_rows_exact_ties():
    shape = C.DEEPSEEK_FINE.with_(T=333, d_model=512, d_ff=64, n_experts=48, top_k=6,
                                  d_ff_shared=0)
    inp = inputs.make_inputs(shape, seed=5)
    w = inp.w_router.copy()
    w[7] = w[3]
    w[40] = w[3]
    w[11] = w[30]
    inp.w_router = w
    inp.sel_bias = None      # so that equal logits are equal scores
    say("case duplicated router rows (exact score ties)")
    gc_, _, _ = _both_paths(shape, inp)
    # tied experts appear in index order
    for a, b in ((3, 7), (7, 40), (3, 40), (11, 30)):
        both = np.isin(gc_["idx"], [a, b]).sum(axis=1) == 2
        for row in gc_["idx"][both].tolist():
            assert row.index(a) < row.index(b), (a, b, row)
    assert (np.isin(gc_["idx"], [3, 7]).sum(axis=1) == 2).any()


def test_massive_ties():
    """256 experts whose router rows take 4 distinct values (64 copies each,
    no selection bias): every token's Top-8 sits inside a 64-way tie, so
    every token is recomputed and the ties fall back to index order."""
    shape = C.DEEPSEEK_FINE.with_(T=300, d_model=512, d_ff=64, n_experts=256, top_k=8,
                                  d_ff_shared=0)
    inp = inputs.make_inputs(shape, seed=9)
    w = inp.w_router.copy()
    w[:] = w[np.arange(256) % 4]
    inp.w_router = w
    inp.sel_bias = None
    say("case 64-way ties: 4 distinct router rows over 256 experts")
    gc_, _, _ = _both_paths(shape, inp)
    # the eight winners are the eight lowest indices of the best row class
    best = np.argmax(gc_["logits"][:, :4], axis=1)
    assert (gc_["idx"] == best[:, None] + 4 * np.arange(8)[None, :]).all()


def test_all_zero_router():
    shape = C.MIXTRAL_PREFILL.with_(T=200, d_model=256, d_ff=128, n_experts=40, top_k=3)
    inp = inputs.make_inputs(shape)
    inp.w_router = np.zeros_like(inp.w_router)
    say("case all-zero router: every logit ties")
    gc_, _, _ = _both_paths(shape, inp)
    assert (gc_["idx"] == np.array([0, 1, 2])).all()


def test_non_finite_tokens():
    """A token with an infinite input and one with a NaN: their rows are
    recomputed whole; every decision equals the exact path's."""
    shape = C.DEEPSEEK_FINE.with_(T=70, d_model=256, d_ff=64, n_experts=32, top_k=4,
                                  d_ff_shared=0)
    inp = inputs.make_inputs(shape, seed=2)
    x = inp.x.copy()
    x[5, 17] = 0x7F80        # +inf
    x[40, 3] = 0x7FC0        # NaN
    inp.x = x
    t = device_tensors(inp)
    gc_ = run_stages(moe.config_for(shape, router="certified"), t)
    ge = run_stages(moe.config_for(shape, router="exact"), t)
    say("case non-finite tokens 5 (inf) and 40 (NaN)")
    for key in ("idx", "counts", "expert_offsets", "slot_row", "row_token"):
        assert (gc_[key] == ge[key]).all(), key
    a, b = gc_["logits"][[5, 40]], ge["logits"][[5, 40]]
    assert ((a.view(np.uint32) == b.view(np.uint32)) | (np.isnan(a) & np.isnan(b))).all()
    fin = np.ones(shape.T, bool)
    fin[[5, 40]] = False
    bound = router_logit_bound(inp)[fin]
    diff = np.abs(gc_["logits"][fin].astype(np.float64) - ge["logits"][fin])
    assert (diff <= bound + np.spacing(np.abs(ge["logits"][fin]))).all()


@pytest.mark.parametrize("T,N,K,d", [(1, 8, 2, 128), (50, 1, 1, 64), (1000, 100, 5, 384), (257, 200, 8, 64),
                                     (64, 4, 4, 128), (513, 256, 1, 192), (96, 33, 32, 256)])
def test_ragged_shapes(T, N, K, d):
    shape = C.DEEPSEEK_FINE.with_(T=T, d_model=d, d_ff=64, n_experts=N, top_k=K, d_ff_shared=0)
    inp = inputs.make_inputs(shape, seed=T + N)
    say(f"case T={T} N={N} K={K} d={d}")
    _both_paths(shape, inp)


def test_deepseek_width():
    """The full model width and expert count (d = 7168, N = 256, top-8,
    selection bias) on 512 tokens."""
    shape = C.DEEPSEEK_FINE.with_(T=512, d_ff=64, d_ff_shared=0)
    inp = inputs.make_inputs(shape, seed=11)
    say(f"case DeepSeek width: T={shape.T} d={shape.d_model} N={shape.n_experts} K={shape.top_k}")
    _both_paths(shape, inp)
