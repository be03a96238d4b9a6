"""Plain fp64 CPU oracle of a multi-layer attention chain over a replay tree.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The GPU library never calls it
and shares no code with it.

What it computes follows "Splitting Prompt Prefill from Response Replay for
Context-Parallel Long-Context LLM Post-Training" (Bao et al.):

* §3.2: training on a replay tree runs the prompt through the model's layers once
  (prefill; every layer keeps the prompt's keys and values) and each response branch
  through the layers against that layer's cached prompt K/V; the prompt-state gradients
  accumulated from all branches then flow back through the prefill layers.
* §2.1 and §3.4 (the b = 0 fallback): the semantics that scheme must reproduce are those
  of G independent sequences (P, R_i), each run through all layers under the ordinary
  causal mask, the prompt recomputed once per branch. That is what this oracle evaluates.

The layer is the attention sub-layer with its projections and a residual connection,
    h <- h + Attn(h Wq, h Wk, h Wv) Wo,
multi-head with grouped-query heads (query head j reads key/value head j // (Hq / Hkv)) and
scale 1/sqrt(D) (§2.2). Normalisation and MLP sub-layers are per-token and do not involve
the tree structure, so they are left out. The loss is linear in the last layer's states:
    loss = sum_i [ <H_i[P:], G_R,i> + (1/G) <H_i[:P], G_P> ]
(each flattened copy i carries its branch's upstream gradient and an equal share of the
prompt's, the reading used by the attention oracle); its value and all its gradients equal
those of the shared-prefix model with loss <H_P, G_P> + sum_i <H_R,i, G_R,i>.

With a language-model head w_lm and the first response token y_i of every branch, the loss
also scores each branch's first token from the final prompt state (§3.2, response replay: the
first response token is predicted by applying the head to the prompt's last hidden state
from the prefill pass, and its loss backpropagates through that state into the prompt graph):
    + sum_i CE(H_i[P - 1] w_lm, y_i),   CE(z, y) = log sum_v exp(z_v) - z_y,
where H_i[P - 1] is copy i's own last prompt state (every copy's equals the shared one).

Arithmetic: fp64 throughout, attention as softmax(scale * Q K^T + M) V with an explicit
causal mask per flattened sequence, gradients by reverse-mode differentiation of these
plain operations (torch.autograd as a library routine).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import torch

__all__ = ["flattened_chain"]

Weights = Sequence[Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]]


def _causal_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float) -> torch.Tensor:
    """q [L][Hq][D], k/v [L][Hkv][D] -> [L][Hq][D]; a token sees itself and earlier tokens."""
    L, Hq, D = q.shape
    group = Hq // k.shape[1]
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    out = []
    for j in range(Hq):
        s = (q[:, j] @ k[:, j // group].T) * scale
        s = s.masked_fill(~mask, float("-inf"))
        out.append(torch.softmax(s, dim=-1) @ v[:, j // group])
    return torch.stack(out, dim=1)


def flattened_chain(x_p: torch.Tensor, x_r: torch.Tensor, offsets: Sequence[int], weights: Weights,
                    g_p: torch.Tensor, g_r: torch.Tensor, Hq: int, Hkv: int, D: int,
                    w_lm: Optional[torch.Tensor] = None, first_tokens: Optional[Sequence[int]] = None) -> Dict:
    """Run every flattened (prompt, branch) sequence through the layers.

    x_p [P][W] and x_r [T_R][W] (branches packed by ``offsets``) are the inputs; weights is one
    (wq [W][Hq*D], wk [W][Hkv*D], wv [W][Hkv*D], wo [Hq*D][W]) tuple per layer; g_p / g_r are
    the upstream gradients of the last layer's states. With w_lm [W][vocab] and first_tokens
    [G], every copy i adds the cross-entropy of its branch's first token y_i scored from its
    last prompt state. Returns the last layer's states of the prompt (from copy 0) and of every
    branch row, the loss, and the gradients of the loss with respect to the inputs, to every
    weight and (with a head) to w_lm.
    """
    off = [int(o) for o in offsets]
    G = len(off) - 1
    P = x_p.shape[0]
    scale = 1.0 / float(D) ** 0.5
    f = torch.float64
    xp = x_p.detach().to(f).clone().requires_grad_(True)
    xr = x_r.detach().to(f).clone().requires_grad_(True)
    ws = [tuple(w.detach().to(f).clone().requires_grad_(True) for w in layer) for layer in weights]
    gp, gr = g_p.to(f), g_r.to(f)
    head = None
    if w_lm is not None:
        head = w_lm.detach().to(f).clone().requires_grad_(True)
        ys = [int(y) for y in first_tokens]
        assert len(ys) == G
    loss = torch.zeros((), dtype=f)
    h_p0 = None
    h_r_rows: List[torch.Tensor] = []
    prompt_copies: List[torch.Tensor] = []
    for i in range(G):
        h = torch.cat([xp, xr[off[i]:off[i + 1]]], dim=0)
        L = h.shape[0]
        for wq, wk, wv, wo in ws:
            q = (h @ wq).view(L, Hq, D)
            k = (h @ wk).view(L, Hkv, D)
            v = (h @ wv).view(L, Hkv, D)
            h = h + _causal_attention(q, k, v, scale).reshape(L, Hq * D) @ wo
        loss = loss + (h[P:] * gr[off[i]:off[i + 1]]).sum() + (h[:P] * gp).sum() / G
        if head is not None:
            z = h[P - 1] @ head                                   # logits of branch i's first token
            loss = loss + (torch.logsumexp(z, dim=0) - z[ys[i]])
        prompt_copies.append(h[:P].detach())
        h_r_rows.append(h[P:].detach())
        if i == 0:
            h_p0 = h[:P].detach()
    loss.backward()
    return {
        "h_p": h_p0, "h_r": torch.cat(h_r_rows, dim=0), "loss": loss.detach(),
        "dx_p": xp.grad, "dx_r": xr.grad,
        "dweights": [tuple(w.grad for w in layer) for layer in ws],
        "prompt_copies": prompt_copies,
        "dw_lm": None if head is None else head.grad,
    }
