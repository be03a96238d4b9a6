"""Multi-layer prefill -> replay chain on the GPU against the fp64 chain oracle.

An L-layer attention chain (h <- h + Attn(h Wq, h Wk, h Wv) Wo, random weights) over a
replay tree: the prompt states go through every layer once and every branch replays each
layer against that layer's prompt K/V, all through the library's autograd attention
(shared_prefix_attention: prefill + replay forward, replay + prefill backward); projections
and residuals are plain torch ops. Backward then carries every branch's prompt-K/V gradient
through the earlier prefill layers ("Splitting Prompt Prefill from Response Replay ...",
§3.2). The oracle (oracle/flat_chain.py) runs every (prompt, branch) pair as its own
sequence through all layers in fp64.

fp32 (head_dim 64, the library's fp32 path): every output state and every gradient (inputs
and all weights) within 1e-4 x max(1, max |reference|) per tensor; weight gradients sum over
all tokens, so their scale grows with the tree.
"""
import time

import pytest
import torch

from oracle import flattened_chain
from shared_prefix_attention_prompt_amd import shared_prefix_attention
from tests.gpu_run import log
from workloads import make_chain_inputs

pytestmark = pytest.mark.gpu


def _gpu_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D):
    dev = torch.device("cuda:0")
    f = torch.float32
    xp = x_p.to(dev, f).requires_grad_(True)
    xr = x_r.to(dev, f).requires_grad_(True)
    w = [tuple(t.to(dev, f).requires_grad_(True) for t in layer) for layer in ws]
    P, T = xp.shape[0], xr.shape[0]
    hp, hr = xp, xr
    for wq, wk, wv, wo in w:
        o_p, o_r = shared_prefix_attention(
            (hp @ wq).view(P, Hq, D).contiguous(), (hp @ wk).view(P, Hkv, D).contiguous(),
            (hp @ wv).view(P, Hkv, D).contiguous(), (hr @ wq).view(T, Hq, D).contiguous(),
            (hr @ wk).view(T, Hkv, D).contiguous(), (hr @ wv).view(T, Hkv, D).contiguous(), off)
        hp = hp + o_p.reshape(P, Hq * D) @ wo
        hr = hr + o_r.reshape(T, Hq * D) @ wo
    loss = (hp * g_p.to(dev, f)).sum() + (hr * g_r.to(dev, f)).sum()
    loss.backward()
    torch.cuda.synchronize()
    return {"h_p": hp.detach(), "h_r": hr.detach(), "loss": loss.detach(), "dx_p": xp.grad, "dx_r": xr.grad,
            "dweights": [tuple(t.grad for t in layer) for layer in w]}


def _close(name, got, ref, report):
    got = got.detach().cpu().double()
    tol = 1e-4 * max(1.0, float(ref.abs().max()))
    err = float((got - ref).abs().max())
    report.append(f"{name} {err:.1e}/{tol:.0e}")
    assert err <= tol, f"{name}: max abs error {err:.3e} > {tol:.3e}"


@pytest.mark.parametrize("P,lens,W,Hq,Hkv,layers", [
    (150, [40, 90, 7], 128, 2, 1, 2),
    (300, [200, 33, 1, 64], 256, 4, 2, 3),
])
def test_chain_matches_flattened_oracle(P, lens, W, Hq, Hkv, layers):
    D = 64
    log(f"chain P={P} lens={lens} W={W} Hq={Hq} Hkv={Hkv} D={D} layers={layers}")
    x_p, x_r, off, ws, g_p, g_r = make_chain_inputs(P, lens, W, Hq, Hkv, D, layers, seed=P + layers)
    _gpu_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D)  # warm-up
    t0 = time.perf_counter()
    got = _gpu_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D)
    t_gpu = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref = flattened_chain(x_p, x_r, off, ws, g_p, g_r, Hq, Hkv, D)
    t_cpu = time.perf_counter() - t0
    report = []
    _close("h_p", got["h_p"], ref["h_p"], report)
    _close("h_r", got["h_r"], ref["h_r"], report)
    _close("dx_p", got["dx_p"], ref["dx_p"], report)
    _close("dx_r", got["dx_r"], ref["dx_r"], report)
    for li, (gl, rl) in enumerate(zip(got["dweights"], ref["dweights"])):
        for name, gw, rw in zip(("wq", "wk", "wv", "wo"), gl, rl):
            _close(f"d{name}{li}", gw, rw, report)
    log("  " + ", ".join(report))
    log(f"  fwd+bwd: GPU chain {1e3 * t_gpu:.2f} ms (wall, one step), fp64 flattened oracle {t_cpu:.2f} s")
