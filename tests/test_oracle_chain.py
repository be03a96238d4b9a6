"""Pins of the multi-layer chain oracle (oracle/flat_chain.py), CPU only.

The chain oracle runs every flattened (prompt, branch) sequence through L attention layers
(h <- h + Attn(h Wq, h Wk, h Wv) Wo). Pinned by: its one-layer output against the attention
oracle (itself pinned in test_oracle_pins.py) fed the same projections; central finite
differences of its loss for every input and weight; prompt states that agree across the
flattened copies (the prompt never sees a branch).
"""
import torch

from oracle import flattened_chain, flattened_tree_attention
from workloads import make_chain_inputs


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
