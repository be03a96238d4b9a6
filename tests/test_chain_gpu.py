"""Multi-layer prefill -> replay chain on the GPU against the fp64 chain oracle.

An L-layer attention chain (h <- h + Attn(h Wq, h Wk, h Wv) Wo, random weights) over a
replay tree: the prompt states go through every layer once and every branch replays each
layer against that layer's prompt K/V, all through the library's autograd attention
(shared_prefix_attention: prefill + replay forward, replay + prefill backward); projections
and residuals are plain torch ops. Backward then carries every branch's prompt-K/V gradient
through the earlier prefill layers ("Splitting Prompt Prefill from Response Replay ...",
§3.2). The oracle (oracle/flat_chain.py) runs every (prompt, branch) pair as its own
sequence through all layers in fp64.

A random language-model head scores each branch's first response token from the final
prompt state (cross-entropy; §3.2, response replay), so that loss reaches the prompt graph
through the prompt's last state.

fp32 (head_dim 64, the library's fp32 path): every output state and every gradient (inputs,
all weights and the head) within 1e-4 x max(1, max |reference|) per tensor; weight gradients
sum over all tokens, so their scale grows with the tree. bf16 attention (head_dim 128; the
projections stay fp32, each layer's Q/K/V are rounded to bf16 before the library call):
relative L2 error within 1e-2 and max abs error within 2e-2 x max(1, max |reference|) per
tensor.
"""
import time

import pytest
import torch

from oracle import flattened_chain
from shared_prefix_attention_prompt_amd import shared_prefix_attention
from tests.gpu_run import log
from workloads import make_chain_inputs, make_lm_head

pytestmark = pytest.mark.gpu


def _gpu_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D, w_lm, first, att_dtype=torch.float32):
    dev = torch.device("cuda:0")
    f = torch.float32
    xp = x_p.to(dev, f).requires_grad_(True)
    xr = x_r.to(dev, f).requires_grad_(True)
    w = [tuple(t.to(dev, f).requires_grad_(True) for t in layer) for layer in ws]
    lm = w_lm.to(dev, f).requires_grad_(True)
    P, T = xp.shape[0], xr.shape[0]
    hp, hr = xp, xr

    def a(x):  # attention operand in the library's dtype
        return x.contiguous().to(att_dtype)
    for wq, wk, wv, wo in w:
        o_p, o_r = shared_prefix_attention(
            a((hp @ wq).view(P, Hq, D)), a((hp @ wk).view(P, Hkv, D)), a((hp @ wv).view(P, Hkv, D)),
            a((hr @ wq).view(T, Hq, D)), a((hr @ wk).view(T, Hkv, D)), a((hr @ wv).view(T, Hkv, D)), off)
        hp = hp + o_p.to(f).reshape(P, Hq * D) @ wo
        hr = hr + o_r.to(f).reshape(T, Hq * D) @ wo
    loss = (hp * g_p.to(dev, f)).sum() + (hr * g_r.to(dev, f)).sum()
    # every branch's first response token, scored from the shared last prompt state
    z = hp[P - 1] @ lm
    y = first.to(dev)
    loss = loss + (torch.logsumexp(z, dim=0) * len(first) - z[y].sum())
    loss.backward()
    torch.cuda.synchronize()
    return {"h_p": hp.detach(), "h_r": hr.detach(), "loss": loss.detach(), "dx_p": xp.grad, "dx_r": xr.grad,
            "dweights": [tuple(t.grad for t in layer) for layer in w], "dw_lm": lm.grad}


def _close(name, got, ref, report, bf16=False):
    got = got.detach().cpu().double()
    scale = max(1.0, float(ref.abs().max()))
    tol = (2e-2 if bf16 else 1e-4) * scale
    err = float((got - ref).abs().max())
    rel = float((got - ref).norm() / ref.norm().clamp_min(1e-300))
    report.append(f"{name} {err:.1e}/{tol:.0e} rel {rel:.1e}")
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.3e}"
    if bf16:
        assert rel <= 1e-2, f"{name}: relative L2 error {rel:.3e} > 1e-2"


@pytest.mark.parametrize("P,lens,W,Hq,Hkv,D,layers,dtype", [
    (150, [40, 90, 7], 128, 2, 1, 64, 2, "f32"),
    (300, [200, 33, 1, 64], 256, 4, 2, 64, 3, "f32"),
    (260, [70, 1, 150], 512, 4, 2, 128, 2, "bf16"),
])
def test_chain_matches_flattened_oracle(P, lens, W, Hq, Hkv, D, layers, dtype):
    log(f"chain P={P} lens={lens} W={W} Hq={Hq} Hkv={Hkv} D={D} layers={layers} attention {dtype}")
    x_p, x_r, off, ws, g_p, g_r = make_chain_inputs(P, lens, W, Hq, Hkv, D, layers, seed=P + layers)
    w_lm, first = make_lm_head(W, 50, len(lens), seed=P + 7)
    att = torch.bfloat16 if dtype == "bf16" else torch.float32
    _gpu_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D, w_lm, first, att)  # warm-up
    t0 = time.perf_counter()
    got = _gpu_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D, w_lm, first, att)
    t_gpu = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref = flattened_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D, w_lm=w_lm, first_tokens=first.tolist())
    t_cpu = time.perf_counter() - t0
    report = []
    bf = dtype == "bf16"
    _close("h_p", got["h_p"], ref["h_p"], report, bf)
    _close("h_r", got["h_r"], ref["h_r"], report, bf)
    _close("dx_p", got["dx_p"], ref["dx_p"], report, bf)
    _close("dx_r", got["dx_r"], ref["dx_r"], report, bf)
    _close("dw_lm", got["dw_lm"], ref["dw_lm"], report, bf)
    for li, (gl, rl) in enumerate(zip(got["dweights"], ref["dweights"])):
        for name, gw, rw in zip(("wq", "wk", "wv", "wo"), gl, rl):
            _close(f"d{name}{li}", gw, rw, report, bf)
    log("  " + ", ".join(report))
    log(f"  fwd+bwd: GPU chain {1e3 * t_gpu:.2f} ms (wall, one step), fp64 flattened oracle {t_cpu:.2f} s")
