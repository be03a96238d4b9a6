"""Pins of the multi-layer chain oracle (oracle/flat_chain.py), CPU only.

The chain oracle runs every flattened (prompt, branch) sequence through L attention layers
(h <- h + Attn(h Wq, h Wk, h Wv) Wo). Pinned by: its one-layer output against the attention
oracle (itself pinned in test_oracle_pins.py) fed the same projections; central finite
differences of its loss for every input and weight; prompt states that agree across the
flattened copies (the prompt never sees a branch).
"""
import math

import torch

from oracle import flattened_chain, flattened_tree_attention
from workloads import make_chain_inputs, make_lm_head


def _chain_inputs(P, lens, W, Hq, Hkv, D, layers, seed):
    return make_chain_inputs(P, lens, W, Hq, Hkv, D, layers, seed)


def test_one_layer_matches_the_attention_oracle():
    P, lens, W, Hq, Hkv, D = 9, [4, 1, 6], 12, 4, 2, 8
    x_p, x_r, off, ws, g_p, g_r = _chain_inputs(P, lens, W, Hq, Hkv, D, 1, seed=3)
    out = flattened_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D)
    wq, wk, wv, wo = ws[0]
    T = x_r.shape[0]
    att = flattened_tree_attention((x_p @ wq).view(P, Hq, D), (x_p @ wk).view(P, Hkv, D),
                                   (x_p @ wv).view(P, Hkv, D), (x_r @ wq).view(T, Hq, D),
                                   (x_r @ wk).view(T, Hkv, D), (x_r @ wv).view(T, Hkv, D),
                                   torch.tensor(off, dtype=torch.int32))
    assert torch.allclose(out["h_p"], x_p + att["o_p"].reshape(P, Hq * D) @ wo, atol=1e-12)
    assert torch.allclose(out["h_r"], x_r + att["o_r"].reshape(T, Hq * D) @ wo, atol=1e-12)


def test_prompt_states_agree_across_copies():
    x_p, x_r, off, ws, g_p, g_r = _chain_inputs(7, [3, 5, 2, 4], 8, 2, 1, 4, 3, seed=4)
    out = flattened_chain(x_p, x_r, off, ws, g_p, g_r, 2, 1, 4)
    for c in out["prompt_copies"][1:]:
        assert torch.allclose(c, out["prompt_copies"][0], atol=1e-13, rtol=0)


def test_gradients_match_central_finite_differences():
    P, lens, W, Hq, Hkv, D, layers = 4, [3, 2], 6, 2, 1, 4, 2
    x_p, x_r, off, ws, g_p, g_r = _chain_inputs(P, lens, W, Hq, Hkv, D, layers, seed=5)
    out = flattened_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D)

    def loss(xp, xr, w):
        return float(flattened_chain(xp, xr, off, w, g_p, g_r, Hq, Hkv, D)["loss"])

    gen = torch.Generator().manual_seed(6)
    h = 1e-6
    # inputs
    for name, grad in [("x_p", out["dx_p"]), ("x_r", out["dx_r"])]:
        d = torch.randn(grad.shape, generator=gen, dtype=torch.float64)
        if name == "x_p":
            fd = (loss(x_p + h * d, x_r, ws) - loss(x_p - h * d, x_r, ws)) / (2 * h)
        else:
            fd = (loss(x_p, x_r + h * d, ws) - loss(x_p, x_r - h * d, ws)) / (2 * h)
        assert abs(fd - float((grad * d).sum())) < 1e-6 * max(1.0, abs(fd)), name
    # every weight of every layer
    for li in range(layers):
        for wi in range(4):
            d = torch.randn(ws[li][wi].shape, generator=gen, dtype=torch.float64)

            def shifted(sign):
                w2 = [list(t) for t in ws]
                w2[li][wi] = ws[li][wi] + sign * h * d
                return [tuple(t) for t in w2]
            fd = (loss(x_p, x_r, shifted(1)) - loss(x_p, x_r, shifted(-1))) / (2 * h)
            an = float((out["dweights"][li][wi] * d).sum())
            assert abs(fd - an) < 1e-6 * max(1.0, abs(fd)), (li, wi, fd, an)


def test_first_token_head_closed_form_with_zero_head():
    # w_lm = 0: every logit is 0, so each branch's first-token cross-entropy is ln(vocab); with
    # no other loss term, dL/dw_lm = sum_i outer(h_last, 1/vocab - e_{y_i}) and
    # dL/dx_p carries h_last's gradient w_lm (sum_i (p - e_y)) = 0
    P, lens, W, Hq, Hkv, D, V = 6, [2, 3, 1], 8, 2, 1, 4, 5
    x_p, x_r, off, ws, g_p, g_r = _chain_inputs(P, lens, W, Hq, Hkv, D, 2, seed=21)
    y = [3, 0, 3]
    zero = torch.zeros(W, V, dtype=torch.float64)
    out = flattened_chain(x_p, x_r, off, ws, g_p * 0, g_r * 0, Hq, Hkv, D, w_lm=zero, first_tokens=y)
    assert abs(float(out["loss"]) - len(lens) * math.log(V)) < 1e-12
    h_last = out["h_p"][P - 1]
    want = torch.zeros(W, V, dtype=torch.float64)
    for yi in y:
        want += torch.outer(h_last, torch.full((V,), 1.0 / V, dtype=torch.float64) - torch.eye(V)[yi].double())
    assert torch.allclose(out["dw_lm"], want, atol=1e-12)
    assert torch.allclose(out["dx_p"], torch.zeros_like(out["dx_p"]), atol=1e-12)


def test_first_token_head_reaches_only_through_the_last_prompt_state():
    # the head term depends on branch inputs only through the prompt (never: a prompt state
    # cannot see a branch), so with zero linear loss the branch inputs get no gradient
    P, lens, W, Hq, Hkv, D = 5, [3, 4], 8, 2, 2, 4
    x_p, x_r, off, ws, g_p, g_r = _chain_inputs(P, lens, W, Hq, Hkv, D, 2, seed=22)
    w_lm, y = make_lm_head(W, 7, len(lens), seed=23)
    out = flattened_chain(x_p, x_r, off, ws, g_p * 0, g_r * 0, Hq, Hkv, D, w_lm=w_lm, first_tokens=y)
    assert float(out["dx_r"].abs().max()) == 0.0
    assert float(out["dx_p"].abs().max()) > 1e-3


def test_first_token_head_gradients_match_finite_differences():
    P, lens, W, Hq, Hkv, D, layers = 4, [3, 2], 6, 2, 1, 4, 2
    x_p, x_r, off, ws, g_p, g_r = _chain_inputs(P, lens, W, Hq, Hkv, D, layers, seed=24)
    w_lm, y = make_lm_head(W, 9, len(lens), seed=25)
    out = flattened_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D, w_lm=w_lm, first_tokens=y)

    def loss(xp, xr, w, lm):
        return float(flattened_chain(xp, xr, off, w, g_p, g_r, Hq, Hkv, D, w_lm=lm, first_tokens=y)["loss"])

    gen = torch.Generator().manual_seed(26)
    h = 1e-6
    d = torch.randn(w_lm.shape, generator=gen, dtype=torch.float64)
    fd = (loss(x_p, x_r, ws, w_lm + h * d) - loss(x_p, x_r, ws, w_lm - h * d)) / (2 * h)
    assert abs(fd - float((out["dw_lm"] * d).sum())) < 1e-6 * max(1.0, abs(fd))
    d = torch.randn(x_p.shape, generator=gen, dtype=torch.float64)
    fd = (loss(x_p + h * d, x_r, ws, w_lm) - loss(x_p - h * d, x_r, ws, w_lm)) / (2 * h)
    assert abs(fd - float((out["dx_p"] * d).sum())) < 1e-6 * max(1.0, abs(fd))
    for li in range(layers):
        for wi in range(4):
            d = torch.randn(ws[li][wi].shape, generator=gen, dtype=torch.float64)
            w2p = [list(t) for t in ws]
            w2m = [list(t) for t in ws]
            w2p[li][wi] = ws[li][wi] + h * d
            w2m[li][wi] = ws[li][wi] - h * d
            fd = (loss(x_p, x_r, [tuple(t) for t in w2p], w_lm) - loss(x_p, x_r, [tuple(t) for t in w2m], w_lm)) / (2 * h)
            assert abs(fd - float((out["dweights"][li][wi] * d).sum())) < 1e-6 * max(1.0, abs(fd)), (li, wi)
