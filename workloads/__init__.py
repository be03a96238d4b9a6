"""Seeded synthetic workloads for shared-prefix attention.

This module only draws random numbers and fixes tensor shapes. It holds none of the
attention arithmetic, so both the fp64 oracle (``oracle/``) and the HIP path
(``shared_prefix_attention_prompt_amd``) can be fed from it without sharing code.

A workload is one replay tree: one prompt of ``P`` tokens and ``G`` response branches of
lengths ``R_i``, packed back to back into ``T_R = sum(R_i)`` rows
("Splitting Prompt Prefill from Response Replay ...", §2.1, replay tree of one shared
prompt root with independent sibling branches).

Layouts (token-major, head_dim contiguous):
  prompt   Q [P][Hq][D],   K/V [P][Hkv][D]
  response Q [T_R][Hq][D], K/V [T_R][Hkv][D]
  offsets  int32 [G+1], offsets[0] = 0, offsets[G] = T_R
  upstream gradients dO_P [P][Hq][D], dO_R [T_R][Hq][D]

Draw order from one CPU ``torch.Generator`` seeded with ``seed``: branch lengths, then
Q_P, K_P, V_P, Q_R, K_R, V_R, dO_P, dO_R. Values are N(0, 1) * std drawn in fp32; for
bf16 workloads they are rounded to bf16 by round-to-nearest-even (``Tensor.to``).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence, Tuple

import torch

__all__ = ["Shape", "Workload", "CONFIGS", "SWEEPS", "config_shape", "make_inputs", "make_shape",
           "config_seed", "workload_name", "pairs_reuse", "pairs_flattened", "algorithmic_flops",
           "make_chain_inputs"]


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one replay tree and the dtype the inputs are stored in."""
    P: int
    lens: Tuple[int, ...]          # R_i, one per branch
    Hq: int
    Hkv: int
    D: int
    dtype: str                     # "f32" or "bf16"
    std: float = 1.0               # standard deviation of Q/K/V (dO is always N(0,1))
    backward: bool = True          # whether dO is drawn and backward is run

    @property
    def G(self) -> int:
        return len(self.lens)

    @property
    def T(self) -> int:
        return int(sum(self.lens))

    @property
    def offsets(self) -> Tuple[int, ...]:
        out = [0]
        for r in self.lens:
            out.append(out[-1] + int(r))
        return tuple(out)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.D) ** 0.5

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]


@dataclasses.dataclass
class Workload:
    """Host tensors of one replay tree (all CPU, contiguous, in ``shape.torch_dtype``)."""
    shape: Shape
    q_p: torch.Tensor
    k_p: torch.Tensor
    v_p: torch.Tensor
    q_r: torch.Tensor
    k_r: torch.Tensor
    v_r: torch.Tensor
    do_p: Optional[torch.Tensor]
    do_r: Optional[torch.Tensor]
    offsets: torch.Tensor          # int32 [G+1]


# The five workloads the method is measured on. Lengths R_i are drawn uniformly
# (inclusive bounds) from the seeded generator when lo != hi.
CONFIGS: Dict[int, dict] = {
    1: dict(workload="tiny_fp32_p256_g4x64_h2_d64", P=256, G=4, R=(64, 64), Hq=2, Hkv=2,
            D=64, dtype="f32", std=1.0, backward=True),
    2: dict(workload="fwd_bf16_p4096_g8x1024_h8_d128", P=4096, G=8, R=(1024, 1024), Hq=8,
            Hkv=8, D=128, dtype="bf16", std=0.5, backward=False),
    3: dict(workload="bf16_p8192_g8xU512-2048_gqa16-4_d128", P=8192, G=8, R=(512, 2048),
            Hq=16, Hkv=4, D=128, dtype="bf16", std=0.5, backward=True),
    4: dict(workload="bf16_p32768_g8xU1024-8192_gqa32-8_d128", P=32768, G=8, R=(1024, 8192),
            Hq=32, Hkv=8, D=128, dtype="bf16", std=0.5, backward=True),
    5: dict(workload="bf16_p131072_g16xU2048-16384_gqa32-8_d128", P=131072, G=16,
            R=(2048, 16384), Hq=32, Hkv=8, D=128, dtype="bf16", std=0.5, backward=True),
}



def _group_sweep_entry(G: int, budget: int = 262144, prompt_frac: float = 0.8) -> dict:
    """One point of the group-size sweep: G branches whose flattened lengths P + R_i add up
    to ``budget`` tokens in expectation (G (L_P + L_R) = budget), with a prompt share of
    ``prompt_frac`` of each flattened sequence; R_i uniform in [L_R/2, 3 L_R/2]."""
    per = budget // G
    lr = int(round(per * (1.0 - prompt_frac)))
    lp = per - lr
    return dict(workload=f"group_g{G}_b{budget // 1024}k_p{lp}_r{lr // 2}-{3 * lr // 2}_gqa28-4_d128",
                P=lp, G=G, R=(lr // 2, 3 * lr // 2), Hq=28, Hkv=4, D=128, dtype="bf16", std=0.5,
                backward=True)


# Group-size and prompt/response-ratio sweep ("Splitting Prompt Prefill from Response
# Replay ...": §4.5 Fig. 18 varies G in {8, 16, 32, 64} at a fixed per-step token budget
# G (L_P + L_R); §1 and §4.3 contrast prompt-heavy with response-heavy reasoning data). The
# trees are synthetic stand-ins: a 256k-token budget (the paper's largest, §4.1) at a 4:1
# prompt:response split for the group sizes, and a response-heavy tree (responses about 4x
# the prompt). Every tree uses the attention layer of the paper's default model (28 query /
# 4 key-value heads, head_dim 128, bf16; §4.1). Keyed by name; seeds 20260100 + index.
SWEEPS: Dict[str, dict] = {}
for _i, _g in enumerate((8, 16, 32, 64)):
    SWEEPS[f"group_g{_g}"] = dict(_group_sweep_entry(_g), seed=20260101 + _i)
SWEEPS["response_heavy"] = dict(
    workload="response_heavy_p2048_g8xU6144-10240_gqa28-4_d128", P=2048, G=8, R=(6144, 10240),
    Hq=28, Hkv=4, D=128, dtype="bf16", std=0.5, backward=True, seed=20260105)


def _entry(cfg):
    if isinstance(cfg, str) and cfg in SWEEPS:
        return SWEEPS[cfg]
    return CONFIGS[int(cfg)]


def workload_name(cfg) -> str:
    """Descriptive name (sizes) of numbered workload ``cfg`` or sweep tree ``cfg``."""
    return _entry(cfg)["workload"]


def config_seed(cfg) -> int:
    """Seed of numbered workload ``cfg`` (20260000 + cfg) or of sweep tree ``cfg``."""
    if isinstance(cfg, str) and cfg in SWEEPS:
        return int(SWEEPS[cfg]["seed"])
    return 20260000 + int(cfg)


def _draw_lens(gen: torch.Generator, G: int, lo: int, hi: int) -> Tuple[int, ...]:
    if lo == hi:
        return tuple([int(lo)] * G)
    r = torch.randint(lo, hi + 1, (G,), generator=gen, dtype=torch.int64)
    return tuple(int(x) for x in r.tolist())


def config_shape(cfg) -> Shape:
    """Shape of numbered workload ``cfg`` (or sweep tree name) with its seeded branch lengths."""
    c = _entry(cfg)
    gen = torch.Generator().manual_seed(config_seed(cfg))
    lens = _draw_lens(gen, c["G"], *c["R"])
    return Shape(P=c["P"], lens=lens, Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], dtype=c["dtype"],
                 std=c["std"], backward=c["backward"])


def make_shape(P: int, lens: Sequence[int], Hq: int, Hkv: int, D: int, dtype: str = "bf16",
               std: float = 0.5, backward: bool = True) -> Shape:
    return Shape(P=int(P), lens=tuple(int(r) for r in lens), Hq=int(Hq), Hkv=int(Hkv),
                 D=int(D), dtype=dtype, std=float(std), backward=bool(backward))


def _randn(gen: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype).contiguous()


def make_inputs(shape_or_cfg, seed: Optional[int] = None) -> Workload:
    """Draw one workload.

    ``shape_or_cfg`` is a config number (1..5), a sweep tree name (``SWEEPS``) or a
    :class:`Shape`. For a number or name the seed defaults to ``config_seed(cfg)`` and the
    branch lengths are the first draw of that same generator, so ``make_inputs(cfg)`` is fully
    determined by ``cfg``.
    """
    if isinstance(shape_or_cfg, (int, str)):
        cfg = shape_or_cfg
        c = _entry(cfg)
        gen = torch.Generator().manual_seed(config_seed(cfg) if seed is None else seed)
        lens = _draw_lens(gen, c["G"], *c["R"])
        shape = Shape(P=c["P"], lens=lens, Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
                      dtype=c["dtype"], std=c["std"], backward=c["backward"])
    else:
        shape = shape_or_cfg
        gen = torch.Generator().manual_seed(0 if seed is None else seed)
    dt = shape.torch_dtype
    P, T, Hq, Hkv, D = shape.P, shape.T, shape.Hq, shape.Hkv, shape.D
    q_p = _randn(gen, (P, Hq, D), shape.std, dt)
    k_p = _randn(gen, (P, Hkv, D), shape.std, dt)
    v_p = _randn(gen, (P, Hkv, D), shape.std, dt)
    q_r = _randn(gen, (T, Hq, D), shape.std, dt)
    k_r = _randn(gen, (T, Hkv, D), shape.std, dt)
    v_r = _randn(gen, (T, Hkv, D), shape.std, dt)
    do_p = do_r = None
    if shape.backward:
        do_p = _randn(gen, (P, Hq, D), 1.0, dt)
        do_r = _randn(gen, (T, Hq, D), 1.0, dt)
    offsets = torch.tensor(shape.offsets, dtype=torch.int32)
    return Workload(shape, q_p, k_p, v_p, q_r, k_r, v_r, do_p, do_r, offsets)


def make_chain_inputs(P: int, lens: Sequence[int], W: int, Hq: int, Hkv: int, D: int, layers: int,
                      seed: int, dtype: torch.dtype = torch.float64):
    """Inputs of an L-layer attention chain over a replay tree, drawn in this order from one
    CPU generator: prompt states x_p [P][W], packed branch states x_r [T_R][W], then per layer
    wq [W][Hq*D], wk [W][Hkv*D], wv [W][Hkv*D] (N(0, 1/W)) and wo [Hq*D][W] (N(0, 1/(Hq*D))),
    then the upstream gradients g_p [P][W] and g_r [T_R][W] (N(0, 1)). Returns
    (x_p, x_r, offsets list, [(wq, wk, wv, wo), ...], g_p, g_r)."""
    g = torch.Generator().manual_seed(int(seed))
    T = int(sum(lens))
    off = [0]
    for r in lens:
        off.append(off[-1] + int(r))

    def rn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, dtype=torch.float64) * std).to(dtype)
    x_p = rn(P, W)
    x_r = rn(T, W)
    ws = [(rn(W, Hq * D, std=W ** -0.5), rn(W, Hkv * D, std=W ** -0.5), rn(W, Hkv * D, std=W ** -0.5),
           rn(Hq * D, W, std=(Hq * D) ** -0.5)) for _ in range(layers)]
    return x_p, x_r, off, ws, rn(P, W), rn(T, W)


def make_lm_head(W: int, vocab: int, G: int, seed: int, dtype: torch.dtype = torch.float64):
    """A random language-model head and the first response token of every branch, drawn from
    their own CPU generator: w_lm [W][vocab] (N(0, 1/W)) and first_tokens [G] (uniform token
    ids in [0, vocab))."""
    g = torch.Generator().manual_seed(int(seed))
    w_lm = (torch.randn(W, vocab, generator=g, dtype=torch.float64) * W ** -0.5).to(dtype)
    first = torch.randint(0, vocab, (G,), generator=g)
    return w_lm, first


# ---- work accounting (counts of (query, key) pairs; no attention arithmetic) ----

def pairs_reuse(shape: Shape) -> int:
    """Visible (query, key) pairs per query head when the prompt is computed once:
    causal prompt triangle + every response row against the whole prompt + each branch's
    own causal triangle (diagonal included)."""
    P = shape.P
    return P * (P + 1) // 2 + shape.T * P + sum(r * (r + 1) // 2 for r in shape.lens)


def pairs_flattened(shape: Shape) -> int:
    """Visible pairs per query head when every (prompt, branch) pair is its own causal
    sequence (prompt recomputed once per branch)."""
    return sum((shape.P + r) * (shape.P + r + 1) // 2 for r in shape.lens)


def algorithmic_flops(shape: Shape, backward: Optional[bool] = None) -> int:
    """4*D flops per visible pair forward (QK^T and PV), 10*D backward (recomputed QK^T
    is not counted: dO V^T, P^T dO, dS^T Q, dS K plus the forward's QK^T), summed over
    the query heads, for the reuse (shared-prefix) work."""
    bwd = shape.backward if backward is None else backward
    per_pair = 4 * shape.D + (10 * shape.D if bwd else 0)
    return shape.Hq * pairs_reuse(shape) * per_pair
