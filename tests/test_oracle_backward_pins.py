"""Pins of the oracle's backward pass (CPU only).

moe_backward is the hand-derived chain rule of the forward.  It is pinned to
things that do not share that derivation:
  * central finite differences of the oracle forward itself (moe_forward,
    aux_loss, router_z_loss), on every parameter of a tiny layer with
    capacity drops, a shared expert, biases, logit offsets, a selection bias,
    the aux loss and the z-loss;
  * torch.autograd (fp64, CPU) of a forward written here from the layer's
    definition, with the routing decisions taken from the oracle;
  * invariants: the softmax-over-K part of d_logits sums to zero per token and
    is zero off the selected experts; an expert that receives no token gets
    exactly zero gradients; a dropped slot's routing-weight gradient is zero;
    a token whose only slot is dropped gets d_x = 0."""
import numpy as np
import pytest

from oracle import moe_oracle as O


def _layer(seed, T, d, f, N, K, fs=0, biases=True, offsets=True, sel=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((N, d)) / np.sqrt(d)
    br = rng.standard_normal(N) * 0.1 if biases else None
    off = rng.standard_normal(N) * 0.5 if offsets else None
    sb = rng.uniform(-0.5, 0.5, N) if sel else None
    ex = []
    for _ in range(N):
        ex.append((rng.standard_normal((f, d)) / np.sqrt(d),
                   rng.standard_normal(f) * 0.1 if biases else None,
                   rng.standard_normal((d, f)) / np.sqrt(f),
                   rng.standard_normal(d) * 0.1 if biases else None))
    shared = None
    if fs:
        shared = (rng.standard_normal((fs, d)) / np.sqrt(d), rng.standard_normal((d, fs)) / np.sqrt(fs))
    d_out = rng.standard_normal((T, d))
    return dict(x=x, wr=wr, br=br, off=off, sb=sb, ex=ex, shared=shared, d_out=d_out)


def _loss(L, K, cap, alpha, beta, g_aux, g_z):
    r = O.moe_forward(L["x"], L["wr"], L["ex"], K, b_router=L["br"], logit_offset=L["off"],
                      sel_bias=L["sb"], shared=L["shared"], capacity=cap, aux_alpha=alpha,
                      round_logits=False)
    val = float(np.sum(L["d_out"] * r["out"]))
    if alpha:
        val += g_aux * r["aux"]
    if beta:
        val += g_z * O.router_z_loss(r["logits"], beta)
    return val, r


def _backward(L, K, cap, alpha, beta, g_aux, g_z):
    return O.moe_backward(L["x"], L["wr"], L["ex"], K, L["d_out"], b_router=L["br"],
                          logit_offset=L["off"], sel_bias=L["sb"], shared=L["shared"],
                          capacity=cap, aux_alpha=alpha, aux_grad=g_aux, zloss_beta=beta,
                          zloss_grad=g_z, round_logits=False)


def _min_margin(scores, K):
    """Smallest gap between consecutive sorted scores around and inside the
    top K+1 of each token (the decisions survive a perturbation below it)."""
    s = -np.sort(-scores, axis=1)
    return float(np.min(s[:, :K] - s[:, 1:K + 1]))


def test_finite_differences_every_parameter():
    T, d, f, N, K, fs = 7, 6, 5, 4, 2, 3
    cap, alpha, beta, g_aux, g_z = 3, 0.05, 0.02, 0.7, 1.3
    L = _layer(11, T, d, f, N, K, fs)
    base, r = _loss(L, K, cap, alpha, beta, g_aux, g_z)
    assert r["n_dropped"] > 0, "the case must drop pairs"
    assert _min_margin(r["scores"], K) > 1e-3
    G = _backward(L, K, cap, alpha, beta, g_aux, g_z)
    h = 1e-6

    def fd(get_arr):
        a = get_arr()
        g = np.zeros_like(a)
        for i in np.ndindex(a.shape):
            old = a[i]
            a[i] = old + h
            p, rp = _loss(L, K, cap, alpha, beta, g_aux, g_z)
            a[i] = old - h
            m, rm = _loss(L, K, cap, alpha, beta, g_aux, g_z)
            a[i] = old
            assert (rp["idx"] == r["idx"]).all() and (rm["idx"] == r["idx"]).all()
            g[i] = (p - m) / (2 * h)
        return g

    checks = [("d_x", lambda: L["x"], G["d_x"]),
              ("d_w_router", lambda: L["wr"], G["d_w_router"]),
              ("d_b_router", lambda: L["br"], G["d_b_router"]),
              ("d_ws1", lambda: L["shared"][0], G["d_ws1"]),
              ("d_ws2", lambda: L["shared"][1], G["d_ws2"])]
    for e in range(N):
        checks += [(f"d_w1[{e}]", lambda e=e: L["ex"][e][0], G["d_w1"][e]),
                   (f"d_b1[{e}]", lambda e=e: L["ex"][e][1], G["d_b1"][e]),
                   (f"d_w2[{e}]", lambda e=e: L["ex"][e][2], G["d_w2"][e]),
                   (f"d_b2[{e}]", lambda e=e: L["ex"][e][3], G["d_b2"][e])]
    for name, get_arr, analytic in checks:
        num = fd(get_arr)
        err = np.max(np.abs(num - analytic))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(num))), (name, err)


def test_autograd_of_an_independent_forward():
    torch = pytest.importorskip("torch")
    T, d, f, N, K, fs = 40, 16, 24, 6, 3, 10
    cap, alpha, beta, g_aux, g_z = 17, 0.01, 0.003, 1.0, 2.0
    L = _layer(5, T, d, f, N, K, fs)
    G = _backward(L, K, cap, alpha, beta, g_aux, g_z)
    assert G["n_dropped"] > 0
    idx = torch.from_numpy(G["idx"].astype(np.int64))
    kept = torch.from_numpy(G["slot_row"] >= 0)
    counts = torch.from_numpy(G["counts"].astype(np.float64))

    def P(a):
        return torch.tensor(a, dtype=torch.float64, requires_grad=True)

    x, wr, br = P(L["x"]), P(L["wr"]), P(L["br"])
    W1 = [P(e[0]) for e in L["ex"]]
    B1 = [P(e[1]) for e in L["ex"]]
    W2 = [P(e[2]) for e in L["ex"]]
    B2 = [P(e[3]) for e in L["ex"]]
    S1, S2 = P(L["shared"][0]), P(L["shared"][1])
    logits = x @ wr.T + br + torch.from_numpy(L["off"])
    w = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    out = torch.zeros(T, d, dtype=torch.float64)
    gelu = torch.nn.functional.gelu
    for t in range(T):
        for k in range(K):
            if kept[t, k]:
                e = int(idx[t, k])
                y = W2[e] @ gelu(W1[e] @ x[t] + B1[e]) + B2[e]
                out = out.index_add(0, torch.tensor([t]), (w[t, k] * y)[None])
    out = out + gelu(x @ S1.T) @ S2.T
    p = torch.softmax(logits, dim=1)
    aux = alpha * N * torch.sum(counts / T * p.mean(dim=0))
    lse = torch.logsumexp(logits, dim=1)
    zl = beta * torch.mean(lse ** 2)
    loss = torch.sum(torch.from_numpy(L["d_out"]) * out) + g_aux * aux + g_z * zl
    loss.backward()
    pairs = [(x.grad, G["d_x"]), (wr.grad, G["d_w_router"]), (br.grad, G["d_b_router"]),
             (S1.grad, G["d_ws1"]), (S2.grad, G["d_ws2"])]
    for e in range(N):
        pairs += [(W1[e].grad, G["d_w1"][e]), (B1[e].grad, G["d_b1"][e]),
                  (W2[e].grad, G["d_w2"][e]), (B2[e].grad, G["d_b2"][e])]
    for tg, og in pairs:
        ref = tg.numpy() if tg is not None else np.zeros_like(og)
        assert np.allclose(ref, og, rtol=1e-10, atol=1e-12)


def test_softmax_part_of_d_logits_sums_to_zero():
    T, d, f, N, K = 30, 8, 12, 5, 3
    L = _layer(3, T, d, f, N, K)
    G = _backward(L, K, None, 0.0, 0.0, 1.0, 1.0)
    dl = G["d_logits"]
    assert np.allclose(dl.sum(axis=1), 0.0, atol=1e-12)
    sel = np.zeros((T, N), dtype=bool)
    np.put_along_axis(sel, G["idx"].astype(np.int64), True, axis=1)
    assert (dl[~sel] == 0).all()


def test_expert_without_tokens_gets_zero_gradient():
    T, d, f, N, K = 12, 6, 7, 5, 1
    L = _layer(8, T, d, f, N, K, offsets=False, sel=False)
    L["off"] = np.zeros(N)
    L["off"][4] = -1e4           # expert 4 is never chosen
    G = _backward(L, K, None, 0.0, 0.0, 1.0, 1.0)
    assert G["counts"][4] == 0
    for name in ("d_w1", "d_b1", "d_w2", "d_b2"):
        assert (G[name][4] == 0).all(), name
        assert np.abs(G[name][:4]).sum() > 0


def test_dropped_slots_have_no_weight_gradient_and_dropped_token_no_input_gradient():
    T, d, f, N, K, cap = 10, 6, 7, 3, 1, 2
    L = _layer(9, T, d, f, N, K, offsets=False, sel=False)
    L["off"] = np.array([1e4, 0.0, 0.0])   # every token picks expert 0; 2 are kept
    G = _backward(L, K, cap, 0.0, 0.0, 1.0, 1.0)
    dropped = G["slot_row"][:, 0] < 0
    assert dropped.sum() == T - cap
    assert (G["d_topk_w"][dropped] == 0).all()
    # single slot: w = 1, so d_logits = w (d_w - w d_w) = 0 for every token
    assert (G["d_logits"] == 0).all()
    assert (G["d_x"][dropped] == 0).all()
    assert np.abs(G["d_x"][~dropped]).sum() > 0


def test_gelu_grad_against_finite_differences_and_special_values():
    z = np.linspace(-6, 6, 241)
    h = 1e-6
    num = (O.gelu(z + h) - O.gelu(z - h)) / (2 * h)
    assert np.max(np.abs(num - O.gelu_grad(z))) < 1e-8
    assert O.gelu_grad(np.array([0.0]))[0] == 0.5
    # GELU(z) - GELU(-z) = z  =>  GELU'(z) + GELU'(-z) = 1
    assert np.allclose(O.gelu_grad(z) + O.gelu_grad(-z), 1.0, atol=1e-15)
