"""Plain fp64 CPU oracle for exact shared-prefix attention, forward and backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The GPU library never calls
it, and it shares no code with the GPU library.

What it computes follows "Splitting Prompt Prefill from Response Replay for
Context-Parallel Long-Context LLM Post-Training" (Bao et al., paperpeel text):

* §2.1 (replay tree, flattening) and §3.4 (the b = 0 fallback): a replay tree with prompt
  P and branches R_1..R_G is evaluated as G independent linear sequences (P, R_i), each
  under the ordinary causal mask. The prompt is recomputed once per branch here on
  purpose: this is the no-reuse semantics the shared-prefix path must reproduce.
* §2.2 (attention as Q-KV block interactions): per head,
  O = softmax(Q K^T / sqrt(D_h) + M) V, with M = -inf where a key comes after the query.
  The diagonal is visible (a token sees itself).
* §3.2, Eq. 1: a response token sees the whole prompt and its own branch prefix, never a
  sibling branch; prompt tokens never see responses. The flattening gives exactly this.
* §3.2, the equation after Eq. 1: the prompt K/V gradient is the sum over branches of each
  branch loss's gradient. Here every flattened copy i contributes its prompt-key gradient
  and the copies are summed.

Readings where the pages are silent (each listed in the design notes of the repository):
* softmax scale is 1/sqrt(D) unless given; LSE is the natural log of sum(exp(scaled
  logit)) per query row;
* grouped-query attention maps query head h to key/value head h // (Hq // Hkv);
* the upstream gradient of a prompt row is split over the G flattened copies with weights
  that sum to 1 (default 1/G each); by linearity any such split gives the same gradients;
* "prompt dK/dV" is the total derivative: the prompt queries' own (prefill) contribution
  plus every branch's contribution.

Arithmetic is plain two-pass softmax per query row (row max, then exp and sum), no online
softmax, no tiling beyond processing query rows in slabs. Keys after a slab's last row are
masked for every row of the slab and are skipped; that changes no value.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import torch

f64 = torch.float64

__all__ = ["rows_attention", "flattened_tree_attention", "flattened_sampled_rows",
           "branch_response_grads", "prompt_key_grads"]


def rows_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, counts: torch.Tensor,
                   scale: float, do: Optional[torch.Tensor] = None):
    """Attention of a block of query rows against one key sequence.

    q [n, D], k/v [L, D] (fp64); row j sees keys 0 .. counts[j]-1 (the causal mask of
    §2.2 written as a visible-key count). Returns (o [n, D], lse [n]) and, when ``do`` is
    given, also (dq [n, D], dk [L, D], dv [L, D]) for the loss sum(o * do).
    """
    L = k.shape[0]
    s = (q @ k.T) * scale                                     # scaled logits [n, L]
    hidden = torch.arange(L)[None, :] >= counts[:, None]
    s = s.masked_fill(hidden, float("-inf"))
    m = s.max(dim=1).values                                  # pass 1: row max
    l = torch.exp(s - m[:, None]).sum(dim=1)                 # pass 2: normaliser
    lse = m + torch.log(l)
    p = torch.exp(s - lse[:, None])                          # softmax probabilities
    o = p @ v
    if do is None:
        return o, lse
    # Backward of o = p v with p = softmax(s), s = scale * q k^T.
    dv = p.T @ do
    dp = do @ v.T
    rowdot = (p * dp).sum(dim=1)                             # sum_j p_j dp_j per row
    ds = p * (dp - rowdot[:, None])
    dq = (ds @ k) * scale
    dk = (ds.T @ q) * scale
    return o, lse, dq, dk, dv


def _as64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to("cpu").to(f64)


def _branch_seq(x_p: torch.Tensor, x_r: torch.Tensor, off: Sequence[int], i: int):
    """Flattened sequence (P, R_i) of one per-head slice: prompt rows, then branch i."""
    return torch.cat([x_p, x_r[off[i]:off[i + 1]]], dim=0)


def flattened_tree_attention(q_p, k_p, v_p, q_r, k_r, v_r, offsets, scale: Optional[float] = None,
                             do_p=None, do_r=None, kv_heads: Optional[Iterable[int]] = None,
                             slab: int = 256, prompt_grad_weights: Optional[Sequence[float]] = None,
                             ) -> Dict[str, torch.Tensor]:
    """Forward (and backward when ``do_p``/``do_r`` are given) of one replay tree.

    Inputs use the packed layouts: q_p [P][Hq][D], k_p/v_p [P][Hkv][D], q_r [T][Hq][D],
    k_r/v_r [T][Hkv][D], offsets [G+1]. Any float dtype; everything is computed in fp64.

    ``kv_heads`` restricts the work to those key/value heads and all query heads mapped
    to them; returned per-head tensors then hold only the selected heads, in order
    (``result["q_heads"]``, ``result["kv_heads"]`` list them).

    Returns o_p [P][h][D], lse_p [h][P], o_r [T][h][D], lse_r [h][T] and, with backward,
    dq_p, dk_p, dv_p, dq_r, dk_r, dv_r (kv tensors indexed by selected kv head), plus
    ``prompt_copy_spread``: the largest |difference| between the prompt rows' outputs of
    flattened copy i > 0 and copy 0 (they must agree; their agreement is the shared-prefix
    premise of §3.2).
    """
    q_p, k_p, v_p = _as64(q_p), _as64(k_p), _as64(v_p)
    q_r, k_r, v_r = _as64(q_r), _as64(k_r), _as64(v_r)
    off = [int(x) for x in (offsets.tolist() if torch.is_tensor(offsets) else offsets)]
    P, Hq, D = q_p.shape
    Hkv = k_p.shape[1]
    G = len(off) - 1
    T = off[-1]
    if scale is None:
        scale = 1.0 / D ** 0.5
    group = Hq // Hkv
    kvs = list(range(Hkv)) if kv_heads is None else [int(g) for g in kv_heads]
    qhs = [g * group + j for g in kvs for j in range(group)]
    backward = do_p is not None
    if backward:
        do_p, do_r = _as64(do_p), _as64(do_r)
        w = [1.0 / G] * G if prompt_grad_weights is None else [float(x) for x in prompt_grad_weights]

    nq, nk = len(qhs), len(kvs)
    out = {
        "o_p": torch.zeros(P, nq, D, dtype=f64), "lse_p": torch.zeros(nq, P, dtype=f64),
        "o_r": torch.zeros(T, nq, D, dtype=f64), "lse_r": torch.zeros(nq, T, dtype=f64),
    }
    if backward:
        out.update({
            "dq_p": torch.zeros(P, nq, D, dtype=f64), "dk_p": torch.zeros(P, nk, D, dtype=f64),
            "dv_p": torch.zeros(P, nk, D, dtype=f64), "dq_r": torch.zeros(T, nq, D, dtype=f64),
            "dk_r": torch.zeros(T, nk, D, dtype=f64), "dv_r": torch.zeros(T, nk, D, dtype=f64),
        })
    spread = 0.0

    for i in range(G):
        L = P + off[i + 1] - off[i]
        for a, h in enumerate(qhs):
            g = h // group
            b = kvs.index(g)
            q = _branch_seq(q_p[:, h], q_r[:, h], off, i)
            k = _branch_seq(k_p[:, g], k_r[:, g], off, i)
            v = _branch_seq(v_p[:, g], v_r[:, g], off, i)
            if backward:
                do = torch.cat([do_p[:, h] * w[i], do_r[off[i]:off[i + 1], h]], dim=0)
                dk = torch.zeros(L, D, dtype=f64)
                dv = torch.zeros(L, D, dtype=f64)
            for r0 in range(0, L, slab):
                r1 = min(L, r0 + slab)
                counts = torch.arange(r0, r1) + 1
                if backward:
                    o, lse, dq, dks, dvs = rows_attention(q[r0:r1], k[:r1], v[:r1], counts,
                                                          scale, do[r0:r1])
                    dk[:r1] += dks
                    dv[:r1] += dvs
                else:
                    o, lse = rows_attention(q[r0:r1], k[:r1], v[:r1], counts, scale)
                # scatter rows of the flattened sequence back to prompt / branch rows
                for (s0, s1, dst0, is_prompt) in _split_rows(r0, r1, P, off[i]):
                    if is_prompt:
                        if i == 0:
                            out["o_p"][dst0:dst0 + s1 - s0, a] = o[s0 - r0:s1 - r0]
                            out["lse_p"][a, dst0:dst0 + s1 - s0] = lse[s0 - r0:s1 - r0]
                        else:
                            d_o = (out["o_p"][dst0:dst0 + s1 - s0, a] - o[s0 - r0:s1 - r0]).abs().max()
                            d_l = (out["lse_p"][a, dst0:dst0 + s1 - s0] - lse[s0 - r0:s1 - r0]).abs().max()
                            spread = max(spread, float(d_o), float(d_l))
                        if backward:
                            out["dq_p"][dst0:dst0 + s1 - s0, a] += dq[s0 - r0:s1 - r0]
                    else:
                        out["o_r"][dst0:dst0 + s1 - s0, a] = o[s0 - r0:s1 - r0]
                        out["lse_r"][a, dst0:dst0 + s1 - s0] = lse[s0 - r0:s1 - r0]
                        if backward:
                            out["dq_r"][dst0:dst0 + s1 - s0, a] = dq[s0 - r0:s1 - r0]
            if backward:
                # prompt keys: sum over flattened copies and over the group's query heads
                out["dk_p"][:, b] += dk[:P]
                out["dv_p"][:, b] += dv[:P]
                out["dk_r"][off[i]:off[i + 1], b] += dk[P:]
                out["dv_r"][off[i]:off[i + 1], b] += dv[P:]
    out["prompt_copy_spread"] = torch.tensor(spread, dtype=f64)
    out["q_heads"] = torch.tensor(qhs)
    out["kv_heads"] = torch.tensor(kvs)
    return out


def _split_rows(r0: int, r1: int, P: int, branch_start: int) -> List[Tuple[int, int, int, bool]]:
    """Pieces of flattened rows [r0, r1): (start, end, destination row, is_prompt)."""
    pieces = []
    if r0 < P:
        pieces.append((r0, min(r1, P), r0, True))
    if r1 > P:
        s0 = max(r0, P)
        pieces.append((s0, r1, branch_start + (s0 - P), False))
    return pieces


def flattened_sampled_rows(q_p, k_p, v_p, q_r, k_r, v_r, offsets, prompt_rows: Sequence[int],
                           response_rows: Sequence[int], scale: Optional[float] = None,
                           do_p=None, do_r=None, prompt_grad_weights: Optional[Sequence[float]] = None,
                           ) -> Dict[str, torch.Tensor]:
    """O, LSE (and dQ when dO is given) of selected rows only, for all query heads.

    A row's output, LSE and dQ depend only on that row's own flattened sequence, so they
    can be evaluated one row set at a time. Prompt row r is evaluated in every flattened
    copy (its keys are prompt keys 0..r); its output is taken from copy 0 and its dQ is the
    weighted sum of the copies' dQ, exactly as in :func:`flattened_tree_attention`.
    Response row j of branch i sees prompt keys 0..P-1 and its branch's keys up to itself.

    Returns o_p [n_p][Hq][D], lse_p [Hq][n_p], o_r [n_r][Hq][D], lse_r [Hq][n_r] and, with
    backward, dq_p [n_p][Hq][D], dq_r [n_r][Hq][D].
    """
    off = [int(x) for x in (offsets.tolist() if torch.is_tensor(offsets) else offsets)]
    P, Hq, D = q_p.shape
    Hkv = k_p.shape[1]
    G = len(off) - 1
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / D ** 0.5
    backward = do_p is not None
    if backward:
        w = [1.0 / G] * G if prompt_grad_weights is None else [float(x) for x in prompt_grad_weights]
    prows = torch.tensor(sorted(set(int(r) for r in prompt_rows)), dtype=torch.long)
    rrows = torch.tensor(sorted(set(int(r) for r in response_rows)), dtype=torch.long)
    np_, nr = len(prows), len(rrows)
    out = {"prompt_rows": prows, "response_rows": rrows,
           "o_p": torch.zeros(np_, Hq, D, dtype=f64), "lse_p": torch.zeros(Hq, np_, dtype=f64),
           "o_r": torch.zeros(nr, Hq, D, dtype=f64), "lse_r": torch.zeros(Hq, nr, dtype=f64)}
    if backward:
        out["dq_p"] = torch.zeros(np_, Hq, D, dtype=f64)
        out["dq_r"] = torch.zeros(nr, Hq, D, dtype=f64)

    for h in range(Hq):
        g = h // group
        # per-head fp64 slices (inputs may be large; only one head is held in fp64)
        kp_g, vp_g = _as64(k_p[:, g]), _as64(v_p[:, g])
        kr_g, vr_g = _as64(k_r[:, g]), _as64(v_r[:, g])
        # prompt rows: evaluated in every flattened copy (each copy's prefix is the prompt)
        if np_:
            last = int(prows.max()) + 1
            for i in range(G):
                k = _branch_seq(kp_g, kr_g, off, i)[:last]
                v = _branch_seq(vp_g, vr_g, off, i)[:last]
                q = _as64(q_p[prows, h])
                counts = prows + 1
                if backward:
                    o, lse, dq, _, _ = rows_attention(q, k, v, counts, scale,
                                                      _as64(do_p[prows, h]) * w[i])
                    out["dq_p"][:, h] += dq
                else:
                    o, lse = rows_attention(q, k, v, counts, scale)
                if i == 0:
                    out["o_p"][:, h] = o
                    out["lse_p"][h] = lse
        # response rows, grouped by branch
        for i in range(G):
            sel = ((rrows >= off[i]) & (rrows < off[i + 1])).nonzero().flatten()
            if len(sel) == 0:
                continue
            rows = rrows[sel]
            k = _branch_seq(kp_g, kr_g, off, i)
            v = _branch_seq(vp_g, vr_g, off, i)
            counts = P + (rows - off[i]) + 1
            last = int(counts.max())
            q = _as64(q_r[rows, h])
            if backward:
                o, lse, dq, _, _ = rows_attention(q, k[:last], v[:last], counts, scale,
                                                  _as64(do_r[rows, h]))
                out["dq_r"][sel, h] = dq
            else:
                o, lse = rows_attention(q, k[:last], v[:last], counts, scale)
            out["o_r"][sel, h] = o
            out["lse_r"][h, sel] = lse
    return out


def branch_response_grads(q_p, k_p, v_p, q_r, k_r, v_r, offsets, branch: int, do_r,
                          kv_heads: Optional[Iterable[int]] = None, scale: Optional[float] = None,
                          slab: int = 256) -> Dict[str, torch.Tensor]:
    """dK and dV of one branch's own response keys.

    In the flattened copy (P, R_i) the response keys of branch i are seen only by the
    response rows of that copy, so their gradients need only those rows (each row still
    normalised over its whole flattened sequence). Returns dk_r, dv_r [R_i][h][D] for the
    selected kv heads, plus dq_r, o_r, lse_r of those rows for the group's query heads.
    """
    off = [int(x) for x in (offsets.tolist() if torch.is_tensor(offsets) else offsets)]
    P, Hq, D = q_p.shape
    Hkv = k_p.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / D ** 0.5
    kvs = list(range(Hkv)) if kv_heads is None else [int(g) for g in kv_heads]
    qhs = [g * group + j for g in kvs for j in range(group)]
    i = int(branch)
    R = off[i + 1] - off[i]
    L = P + R
    out = {"dk_r": torch.zeros(R, len(kvs), D, dtype=f64), "dv_r": torch.zeros(R, len(kvs), D, dtype=f64),
           "dq_r": torch.zeros(R, len(qhs), D, dtype=f64), "o_r": torch.zeros(R, len(qhs), D, dtype=f64),
           "lse_r": torch.zeros(len(qhs), R, dtype=f64),
           "q_heads": torch.tensor(qhs), "kv_heads": torch.tensor(kvs)}
    for a, h in enumerate(qhs):
        g = h // group
        b = kvs.index(g)
        k = _branch_seq(_as64(k_p[:, g]), _as64(k_r[:, g]), off, i)
        v = _branch_seq(_as64(v_p[:, g]), _as64(v_r[:, g]), off, i)
        q = _as64(q_r[off[i]:off[i + 1], h])
        do = _as64(do_r[off[i]:off[i + 1], h])
        for r0 in range(0, R, slab):
            r1 = min(R, r0 + slab)
            counts = P + torch.arange(r0, r1) + 1
            last = P + r1
            o, lse, dq, dk, dv = rows_attention(q[r0:r1], k[:last], v[:last], counts, scale, do[r0:r1])
            out["dk_r"][:r1, b] += dk[P:last]
            out["dv_r"][:r1, b] += dv[P:last]
            out["dq_r"][r0:r1, a] = dq
            out["o_r"][r0:r1, a] = o
            out["lse_r"][a, r0:r1] = lse
    return out


def _selected_key_grads(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, counts: torch.Tensor,
                        scale: float, do: torch.Tensor, keys: torch.Tensor):
    """Contribution of a block of query rows to dK and dV of the key positions ``keys``.

    Same arithmetic as :func:`rows_attention` (two-pass softmax over each row's visible keys
    0 .. counts[j]-1, rowdot in its plain form sum_j P_j dP_j), with the backward evaluated only
    for the selected key columns: dS = P o (dP - rowdot), dK = scale dS^T Q, dV = P^T dO.
    """
    L = k.shape[0]
    s = (q @ k.T) * scale
    hidden = torch.arange(L)[None, :] >= counts[:, None]
    s = s.masked_fill(hidden, float("-inf"))
    m = s.max(dim=1).values
    lse = m + torch.log(torch.exp(s - m[:, None]).sum(dim=1))
    p = torch.exp(s - lse[:, None])
    dp = do @ v.T
    rowdot = (p * dp).sum(dim=1)
    pj = p[:, keys]
    dsj = pj * (dp[:, keys] - rowdot[:, None])
    return (dsj.T @ q) * scale, pj.T @ do


def prompt_key_grads(q_p, k_p, v_p, q_r, k_r, v_r, offsets, keys: Sequence[int], do_p, do_r,
                     kv_heads: Optional[Iterable[int]] = None, scale: Optional[float] = None,
                     slab: int = 256) -> Dict[str, torch.Tensor]:
    """dK and dV of selected prompt keys: the total prompt-key gradient of §3.2 (the prompt
    queries' own part plus, by the equation after Eq. 1, the sum over branches of each branch
    loss's gradient), for the selected key/value heads (all query heads of each group).

    A prompt key j is seen by prompt rows r >= j and by every response row of every branch
    (in each flattened copy (P, R_i) it is a prefix key). Each row is normalised over its own
    whole flattened sequence (two-pass softmax), so every row still runs over all its visible
    keys; only the gradient columns of the selected keys are formed. The prompt rows' upstream
    gradient is taken whole on copy 0 (split weights (1, 0, ..., 0); by linearity every split
    with weights summing to 1 gives the same gradient, which the pins check).

    Returns dk_p, dv_p [n_keys][n_kv][D] (fp64), ``keys`` and ``kv_heads``.
    """
    off = [int(x) for x in (offsets.tolist() if torch.is_tensor(offsets) else offsets)]
    P, Hq, D = q_p.shape
    Hkv = k_p.shape[1]
    G = len(off) - 1
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / D ** 0.5
    kvs = list(range(Hkv)) if kv_heads is None else [int(g) for g in kv_heads]
    J = torch.tensor(sorted(set(int(j) for j in keys)), dtype=torch.long)
    assert len(J) and int(J.min()) >= 0 and int(J.max()) < P
    dk = torch.zeros(len(J), len(kvs), D, dtype=f64)
    dv = torch.zeros(len(J), len(kvs), D, dtype=f64)
    for b, g in enumerate(kvs):
        kp_g, vp_g = _as64(k_p[:, g]), _as64(v_p[:, g])
        kr_g, vr_g = _as64(k_r[:, g]), _as64(v_r[:, g])
        for h in range(g * group, (g + 1) * group):
            qp_h, dop_h = _as64(q_p[:, h]), _as64(do_p[:, h])
            # prompt rows (copy 0): row r sees prompt keys 0..r
            for r0 in range(0, P, slab):
                r1 = min(P, r0 + slab)
                sel = (J < r1).nonzero().flatten()
                if len(sel) == 0:
                    continue
                gk, gv = _selected_key_grads(qp_h[r0:r1], kp_g[:r1], vp_g[:r1], torch.arange(r0, r1) + 1,
                                             scale, dop_h[r0:r1], J[sel])
                dk[sel, b] += gk
                dv[sel, b] += gv
            # response rows of every copy: row t of branch i sees all prompt keys and its
            # branch's keys up to itself
            qr_h, dor_h = _as64(q_r[:, h]), _as64(do_r[:, h])
            for i in range(G):
                k = _branch_seq(kp_g, kr_g, off, i)
                v = _branch_seq(vp_g, vr_g, off, i)
                R = off[i + 1] - off[i]
                for t0 in range(0, R, slab):
                    t1 = min(R, t0 + slab)
                    gk, gv = _selected_key_grads(qr_h[off[i] + t0:off[i] + t1], k[:P + t1], v[:P + t1],
                                                 P + torch.arange(t0, t1) + 1, scale,
                                                 dor_h[off[i] + t0:off[i] + t1], J)
                    dk[:, b] += gk
                    dv[:, b] += gv
    return {"dk_p": dk, "dv_p": dv, "keys": J, "kv_heads": torch.tensor(kvs)}
