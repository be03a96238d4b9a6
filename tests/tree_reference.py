"""Brute-force shared-prefix attention from a library routine, for pinning the oracle.

The whole replay tree is packed as one sequence [P; R_1; ...; R_G] and evaluated by
``torch.nn.functional.scaled_dot_product_attention`` (fp64, CPU) under an explicit boolean
tree mask built from the dependency rule of Eq. 1 in "Splitting Prompt Prefill from
Response Replay ..." (§3.2): a prompt token sees earlier prompt tokens (itself included);
a response token of branch i sees every prompt token and the tokens of branch i up to
itself; nothing sees a sibling branch. LSE comes from ``torch.logsumexp`` and gradients
from ``torch.autograd``. This shares no code with the oracle (which flattens the tree into
G causal sequences and differentiates by hand).
"""
import torch
import torch.nn.functional as F


def tree_mask(P, offsets):
    off = [int(x) for x in offsets]
    T = off[-1]
    N = P + T
    allowed = torch.zeros(N, N, dtype=torch.bool)
    idx = torch.arange(N)
    allowed[:P, :P] = idx[:P, None] >= idx[None, :P]
    for i in range(len(off) - 1):
        a, b = P + off[i], P + off[i + 1]
        allowed[a:b, :P] = True
        allowed[a:b, a:b] = idx[a:b, None] >= idx[None, a:b]
    return allowed


def tree_attention(q_p, k_p, v_p, q_r, k_r, v_r, offsets, scale=None, do_p=None, do_r=None):
    f64 = torch.float64
    q = torch.cat([q_p, q_r]).to(f64).detach()
    k = torch.cat([k_p, k_r]).to(f64).detach()
    v = torch.cat([v_p, v_r]).to(f64).detach()
    P = q_p.shape[0]
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    if scale is None:
        scale = 1.0 / D ** 0.5
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    ke = k.repeat_interleave(grp, dim=1)
    ve = v.repeat_interleave(grp, dim=1)
    mask = tree_mask(P, offsets)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), ke.transpose(0, 1), ve.transpose(0, 1),
                                       attn_mask=mask, scale=scale).transpose(0, 1)
    logits = torch.einsum("qhd,khd->hqk", q.detach(), ke.detach()) * scale
    lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
    res = {"o_p": o[:P].detach(), "o_r": o[P:].detach(), "lse_p": lse[:, :P], "lse_r": lse[:, P:]}
    if do_p is not None:
        do = torch.cat([do_p, do_r]).to(f64)
        (o * do).sum().backward()
        res.update({"dq_p": q.grad[:P], "dq_r": q.grad[P:], "dk_p": k.grad[:P], "dk_r": k.grad[P:],
                    "dv_p": v.grad[:P], "dv_r": v.grad[P:]})
    return res
