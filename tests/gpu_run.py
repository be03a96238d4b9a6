"""Helpers of the GPU tests: run the whole path through the C ABI and compare with the
oracle. Imported only by GPU tests."""
from __future__ import annotations

import functools
import sys

import torch

from shared_prefix_attention_prompt_amd import ops
from workloads import make_inputs

NAMES = ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r"]


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def config_inputs(cfg: int):
    return make_inputs(cfg)


def upload(w, device="cuda:0"):
    return {k: getattr(w, k).to(device) for k in NAMES if getattr(w, k) is not None}


def run_path(w, t=None, backward=True):
    """Forward (+ backward) of the whole hot path on the GPU; returns GPU tensors."""
    if t is None:
        t = upload(w)
    off = list(w.shape.offsets)
    o_p, lse_p = ops.prefill_fwd(t["q_p"], t["k_p"], t["v_p"], None, off)
    o_r, lse_r = ops.replay_fwd(t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], off)
    out = {"o_p": o_p, "lse_p": lse_p, "o_r": o_r, "lse_r": lse_r}
    if backward:
        dq_r, dk_r, dv_r, dk_acc, dv_acc = ops.replay_bwd(t["k_p"], t["v_p"], t["q_r"], t["k_r"],
                                                          t["v_r"], off, o_r, lse_r, t["do_r"])
        dq_p, dk_p, dv_p = ops.prefill_bwd(t["q_p"], t["k_p"], t["v_p"], o_p, lse_p, t["do_p"],
                                           dk_acc, dv_acc, None, off)
        out.update({"dq_p": dq_p, "dk_p": dk_p, "dv_p": dv_p, "dq_r": dq_r, "dk_r": dk_r,
                    "dv_r": dv_r, "dk_p_acc": dk_acc, "dv_p_acc": dv_acc})
    torch.cuda.synchronize()
    return out


def tolerances(dtype: str):
    """(max abs, relative L2 or None) for the input dtype."""
    return (1e-4, None) if dtype == "f32" else (2e-2, 1e-2)


# A tensor stored in bf16 is rounded once, to nearest even, after fp32 accumulation. That
# rounding alone moves a value x by up to half an ulp of x's binade: 2^(floor(log2|x|) - 8)
# (bf16 keeps 8 significant bits). The test bound for such tensors is therefore
# |got - ref| <= tol_abs + half_ulp, with the binade taken from the larger of |got| and |ref|
# (the fp32 value that was rounded lies between them up to the tolerance). This is a stated
# deviation from the plain max-abs bound: without it a correct kernel fails wherever |x| >= 8,
# since half an ulp there is already >= 2^-5 > 2e-2. The plain max abs error is reported too.
def bf16_half_ulp(x: torch.Tensor) -> torch.Tensor:
    """Half an ulp of bf16 at the binade of each |x| (0 where x == 0)."""
    ax = x.abs()
    e = torch.floor(torch.log2(ax.clamp_min(1e-300)))
    return torch.where(ax > 0, torch.pow(2.0, e - 8), torch.zeros_like(ax))


def compare(name: str, got: torch.Tensor, ref: torch.Tensor, dtype: str, report=None,
            abs_scale: bool = False):
    """Max abs error within the dtype's bound (times max(1, max|ref|) when abs_scale; plus
    the final bf16 rounding of each value for bf16-stored tensors) and, for bf16, relative L2
    error within 1e-2. report gets (name, error after the rounding allowance, rel L2, max|ref|,
    plain max abs error)."""
    stored_bf16 = got.dtype == torch.bfloat16
    got = got.detach().to("cpu").to(torch.float64)
    ref = ref.to(torch.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert torch.isfinite(got).all(), f"{name}: non-finite values"
    plain = (got - ref).abs()
    diff = plain
    if stored_bf16:
        diff = (plain - bf16_half_ulp(torch.maximum(got.abs(), ref.abs()))).clamp_min(0.0)
    err = float(diff.max()) if got.numel() else 0.0
    plain_err = float(plain.max()) if got.numel() else 0.0
    rel = float((got - ref).norm() / ref.norm().clamp_min(1e-300)) if got.numel() else 0.0
    tol_abs, tol_rel = tolerances(dtype)
    if abs_scale and ref.numel():
        tol_abs *= max(1.0, float(ref.abs().max()))
    if report is not None:
        report.append((name, err, rel, float(ref.abs().max()) if ref.numel() else 0.0, plain_err))
    assert err <= tol_abs, (f"{name}: max abs error {err:.3e} (plain {plain_err:.3e}) > {tol_abs:.0e} "
                            f"(rel L2 {rel:.2e})")
    if tol_rel is not None:
        assert rel <= tol_rel, f"{name}: relative L2 error {rel:.3e} > {tol_rel:.0e}"


def sum_rules(w, out):
    """Per kv head, over all prompt and response keys: sum dV = sum of the group's dO over
    all rows; sum dK = 0. Checked relative to the summed magnitudes (any size)."""
    s = w.shape
    grp = s.Hq // s.Hkv
    f = torch.float64
    dv = out["dv_p"].to(f).sum(0) + out["dv_r"].to(f).sum(0)               # [Hkv][D]
    dk = out["dk_p"].to(f).sum(0) + out["dk_r"].to(f).sum(0)
    dv_mag = out["dv_p"].to(f).abs().sum(0) + out["dv_r"].to(f).abs().sum(0)
    dk_mag = out["dk_p"].to(f).abs().sum(0) + out["dk_r"].to(f).abs().sum(0)
    dev = out["dv_p"].device
    do_p = w.do_p.to(dev).to(f).view(s.P, s.Hkv, grp, s.D).sum((0, 2))
    do_r = w.do_r.to(dev).to(f).view(s.T, s.Hkv, grp, s.D).sum((0, 2))
    e_v = float(((dv - do_p - do_r).abs() / dv_mag.clamp_min(1e-30)).max())
    e_k = float((dk.abs() / dk_mag.clamp_min(1e-30)).max())
    return e_v, e_k
