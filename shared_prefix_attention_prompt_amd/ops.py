"""Torch-facing wrappers of the four C-ABI entry points, and the autograd function.

PyTorch provides device memory and the current HIP stream; every step of the attention
runs in the HIP kernels of libaugtree.so. Tensors must be contiguous, on one GPU, in
float32 or bfloat16, with the layouts of include/augtree.h.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib

_DT = {torch.float32: _lib.AUGTREE_F32, torch.bfloat16: _lib.AUGTREE_BF16}


def _offsets_list(offsets) -> list:
    if torch.is_tensor(offsets):
        return [int(x) for x in offsets.detach().to("cpu").tolist()]
    return [int(x) for x in offsets]


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _expect(name: str, t, shape, dtype) -> None:
    """Raise ValueError unless t is a tensor of exactly this shape and dtype (checked before
    anything reaches the library, so a mismatch never launches a kernel)."""
    if not torch.is_tensor(t):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _tree_sizes(q, k, offsets, q_name: str, k_name: str):
    """(rows, Hq, Hkv, D, dtype) read from a query tensor [rows][Hq][D] and a key tensor
    [rows'][Hkv][D], with the head and dtype rules of the interface checked."""
    for name, t in ((q_name, q), (k_name, k)):
        if not torch.is_tensor(t) or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-d tensor [rows][heads][head_dim]")
    rows, Hq, D = (int(x) for x in q.shape)
    Hkv = int(k.shape[1])
    if q.dtype not in _DT:
        raise ValueError(f"{q_name} has unsupported dtype {q.dtype} (float32 or bfloat16)")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"{q_name} has {Hq} heads, not a multiple of the {Hkv} heads of {k_name}")
    if int(k.shape[2]) != D:
        raise ValueError(f"{k_name} has head_dim {int(k.shape[2])}, {q_name} {D}")
    return rows, Hq, Hkv, D, q.dtype


def _check_offsets(off) -> int:
    if len(off) < 2 or off[0] != 0 or any(b <= a for a, b in zip(off, off[1:])):
        raise ValueError(f"offsets must start at 0 and increase strictly (every branch >= 1 row): {off[:8]}")
    return off[-1]


def _check_tensors(*named):
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev


def _dims(P, offsets, Hq, Hkv, D, scale, dtype):
    if dtype not in _DT:
        raise ValueError(f"unsupported dtype {dtype}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return _lib.make_dims(P, offsets, Hq, Hkv, D, scale, _DT[dtype])


def _workspace(dims, op, device):
    n = _lib.workspace_bytes(dims, op)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def prefill_fwd(q_p, k_p, v_p, scale: Optional[float] = None, offsets: Sequence[int] = (0, 1)
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Causal prompt attention: (o_p [P][Hq][D], lse_p [Hq][P] float32)."""
    P, Hq, Hkv, D, dt = _tree_sizes(q_p, k_p, offsets, "q_p", "k_p")
    _expect("k_p", k_p, (P, Hkv, D), dt)
    _expect("v_p", v_p, (P, Hkv, D), dt)
    dev = _check_tensors(("q_p", q_p), ("k_p", k_p), ("v_p", v_p))
    dims, keep = _dims(P, _offsets_list(offsets), Hq, Hkv, D, scale, dt)
    o_p = torch.empty_like(q_p)
    lse_p = torch.empty(Hq, P, dtype=torch.float32, device=dev)
    ws, n = _workspace(dims, _lib.AUGTREE_OP_PREFILL_FWD, dev)
    st = _lib.augtree_prefill_fwd(dims, q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(), o_p.data_ptr(),
                                  lse_p.data_ptr(), _ptr(ws), n, _stream(dev))
    _lib._check(st, "augtree_prefill_fwd")
    return o_p, lse_p


def replay_fwd(k_p, v_p, q_r, k_r, v_r, offsets, scale: Optional[float] = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Branch rows against the stationary prompt K/V and their own branch:
    (o_r [T][Hq][D], lse_r [Hq][T] float32)."""
    T, Hq, Hkv, D, dt = _tree_sizes(q_r, k_p, offsets, "q_r", "k_p")
    off = _offsets_list(offsets)
    if _check_offsets(off) != T:
        raise ValueError(f"q_r has {T} rows, offsets[-1] = {off[-1]}")
    P = int(k_p.shape[0])
    _expect("k_p", k_p, (P, Hkv, D), dt)
    _expect("v_p", v_p, (P, Hkv, D), dt)
    _expect("k_r", k_r, (T, Hkv, D), dt)
    _expect("v_r", v_r, (T, Hkv, D), dt)
    dev = _check_tensors(("k_p", k_p), ("v_p", v_p), ("q_r", q_r), ("k_r", k_r), ("v_r", v_r))
    dims, keep = _dims(P, off, Hq, Hkv, D, scale, dt)
    o_r = torch.empty_like(q_r)
    lse_r = torch.empty(Hq, T, dtype=torch.float32, device=dev)
    ws, n = _workspace(dims, _lib.AUGTREE_OP_REPLAY_FWD, dev)
    st = _lib.augtree_replay_fwd(dims, k_p.data_ptr(), v_p.data_ptr(), q_r.data_ptr(), k_r.data_ptr(),
                                 v_r.data_ptr(), o_r.data_ptr(), lse_r.data_ptr(), _ptr(ws), n, _stream(dev))
    _lib._check(st, "augtree_replay_fwd")
    return o_r, lse_r


def replay_bwd(k_p, v_p, q_r, k_r, v_r, offsets, o_r, lse_r, do_r, scale: Optional[float] = None):
    """(dq_r, dk_r, dv_r, dk_p_acc, dv_p_acc): branch gradients and the branches' summed
    prompt K/V gradient in float32."""
    T, Hq, Hkv, D, dt = _tree_sizes(q_r, k_p, offsets, "q_r", "k_p")
    off = _offsets_list(offsets)
    if _check_offsets(off) != T:
        raise ValueError(f"q_r has {T} rows, offsets[-1] = {off[-1]}")
    P = int(k_p.shape[0])
    _expect("k_p", k_p, (P, Hkv, D), dt)
    _expect("v_p", v_p, (P, Hkv, D), dt)
    _expect("k_r", k_r, (T, Hkv, D), dt)
    _expect("v_r", v_r, (T, Hkv, D), dt)
    _expect("o_r", o_r, (T, Hq, D), dt)
    _expect("lse_r", lse_r, (Hq, T), torch.float32)
    _expect("do_r", do_r, (T, Hq, D), dt)
    dev = _check_tensors(("k_p", k_p), ("v_p", v_p), ("q_r", q_r), ("k_r", k_r), ("v_r", v_r),
                         ("o_r", o_r), ("lse_r", lse_r), ("do_r", do_r))
    dims, keep = _dims(P, off, Hq, Hkv, D, scale, dt)
    dq_r = torch.empty_like(q_r)
    dk_r = torch.empty_like(k_r)
    dv_r = torch.empty_like(v_r)
    dk_acc = torch.empty(P, Hkv, D, dtype=torch.float32, device=dev)
    dv_acc = torch.empty(P, Hkv, D, dtype=torch.float32, device=dev)
    ws, n = _workspace(dims, _lib.AUGTREE_OP_REPLAY_BWD, dev)
    st = _lib.augtree_replay_bwd(dims, k_p.data_ptr(), v_p.data_ptr(), q_r.data_ptr(), k_r.data_ptr(),
                                 v_r.data_ptr(), o_r.data_ptr(), lse_r.data_ptr(), do_r.data_ptr(),
                                 dq_r.data_ptr(), dk_r.data_ptr(), dv_r.data_ptr(), dk_acc.data_ptr(),
                                 dv_acc.data_ptr(), _ptr(ws), n, _stream(dev))
    _lib._check(st, "augtree_replay_bwd")
    return dq_r, dk_r, dv_r, dk_acc, dv_acc


def prefill_bwd(q_p, k_p, v_p, o_p, lse_p, do_p, dk_p_acc=None, dv_p_acc=None,
                scale: Optional[float] = None, offsets: Sequence[int] = (0, 1)):
    """(dq_p, dk_p, dv_p): prompt gradients including the branches' accumulated prompt
    K/V gradient when given."""
    P, Hq, Hkv, D, dt = _tree_sizes(q_p, k_p, offsets, "q_p", "k_p")
    _expect("k_p", k_p, (P, Hkv, D), dt)
    _expect("v_p", v_p, (P, Hkv, D), dt)
    _expect("o_p", o_p, (P, Hq, D), dt)
    _expect("lse_p", lse_p, (Hq, P), torch.float32)
    _expect("do_p", do_p, (P, Hq, D), dt)
    if (dk_p_acc is None) != (dv_p_acc is None):
        raise ValueError("dk_p_acc and dv_p_acc must both be given or both be None")
    if dk_p_acc is not None:
        _expect("dk_p_acc", dk_p_acc, (P, Hkv, D), torch.float32)
        _expect("dv_p_acc", dv_p_acc, (P, Hkv, D), torch.float32)
    dev = _check_tensors(("q_p", q_p), ("k_p", k_p), ("v_p", v_p), ("o_p", o_p), ("lse_p", lse_p),
                         ("do_p", do_p), ("dk_p_acc", dk_p_acc), ("dv_p_acc", dv_p_acc))
    dims, keep = _dims(P, _offsets_list(offsets), Hq, Hkv, D, scale, dt)
    dq_p = torch.empty_like(q_p)
    dk_p = torch.empty_like(k_p)
    dv_p = torch.empty_like(v_p)
    ws, n = _workspace(dims, _lib.AUGTREE_OP_PREFILL_BWD, dev)
    st = _lib.augtree_prefill_bwd(dims, q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(), o_p.data_ptr(),
                                  lse_p.data_ptr(), do_p.data_ptr(), _ptr(dk_p_acc), _ptr(dv_p_acc),
                                  dq_p.data_ptr(), dk_p.data_ptr(), dv_p.data_ptr(), _ptr(ws), n,
                                  _stream(dev))
    _lib._check(st, "augtree_prefill_bwd")
    return dq_p, dk_p, dv_p


class SharedPrefixAttention(torch.autograd.Function):
    """Drop-in attention over a replay tree: prefill once, replay all branches, and in
    backward sum every branch's prompt K/V gradient into the prompt gradient."""

    @staticmethod
    def forward(ctx, q_p, k_p, v_p, q_r, k_r, v_r, offsets, scale):
        off = _offsets_list(offsets)
        o_p, lse_p = prefill_fwd(q_p, k_p, v_p, scale, off)
        o_r, lse_r = replay_fwd(k_p, v_p, q_r, k_r, v_r, off, scale)
        ctx.save_for_backward(q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r)
        ctx.off = off
        ctx.scale = scale
        return o_p, o_r

    @staticmethod
    def backward(ctx, do_p, do_r):
        q_p, k_p, v_p, q_r, k_r, v_r, o_p, lse_p, o_r, lse_r = ctx.saved_tensors
        do_p = torch.zeros_like(o_p) if do_p is None else do_p.contiguous()
        do_r = torch.zeros_like(o_r) if do_r is None else do_r.contiguous()
        dq_r, dk_r, dv_r, dk_acc, dv_acc = replay_bwd(k_p, v_p, q_r, k_r, v_r, ctx.off, o_r, lse_r,
                                                      do_r, ctx.scale)
        dq_p, dk_p, dv_p = prefill_bwd(q_p, k_p, v_p, o_p, lse_p, do_p, dk_acc, dv_acc, ctx.scale, ctx.off)
        return dq_p, dk_p, dv_p, dq_r, dk_r, dv_r, None, None


def shared_prefix_attention(q_p, k_p, v_p, q_r, k_r, v_r, offsets, scale: Optional[float] = None):
    """(o_p, o_r) with autograd support; see :class:`SharedPrefixAttention`."""
    return SharedPrefixAttention.apply(q_p, k_p, v_p, q_r, k_r, v_r, offsets, scale)


# ---------------------------------------------------------------------------------------
# Single steps (one kernel each; replay_prompt_bwd one or three). The four calls above are
# compositions of these; a prompt key range makes a call act as one stationary prompt-K/V
# shard whose partial states are merged per query row afterwards.
# ---------------------------------------------------------------------------------------
class Tree:
    """Sizes of one replay tree, for the single-step calls."""

    def __init__(self, P: int, offsets: Sequence[int], Hq: int, Hkv: int, D: int,
                 dtype: torch.dtype, device, scale: Optional[float] = None):
        self.P, self.Hq, self.Hkv, self.D = int(P), int(Hq), int(Hkv), int(D)
        self.offsets = [int(x) for x in offsets]
        self.T = self.offsets[-1]
        self.dtype = dtype
        self.device = torch.device(device)
        self.dims, self._keep = _dims(P, self.offsets, Hq, Hkv, D, scale, dtype)

    @classmethod
    def like(cls, q_p, k_p, offsets, scale: Optional[float] = None) -> "Tree":
        return cls(q_p.shape[0], _offsets_list(offsets), q_p.shape[1], k_p.shape[1], q_p.shape[2],
                   q_p.dtype, q_p.device, scale)

    def stream(self) -> int:
        return _stream(self.device)

    def check(self, **named) -> None:
        """Shape, dtype and device of the named tensors against this tree, before any call:
        prompt rows P, branch rows T, query heads Hq, key/value heads Hkv, head_dim D.
        Names: *_p / *_r tensors with q/o/do (Hq heads) or k/v (Hkv heads); lse_* and
        rowdot_* [Hq][rows] float32; *_acc [P][Hkv][D] float32; o_part [T][Hq][D] and
        lse_part [Hq][T] float32."""
        f32 = torch.float32
        for name, t in named.items():
            if t is None:
                continue
            base = name.split("_")[0]
            rows = self.P if name.endswith("_p") or name.endswith("_p_acc") else self.T
            if name in ("o_part", "dq_part"):
                _expect(name, t, (self.T, self.Hq, self.D), f32)
            elif name in ("lse_part",):
                _expect(name, t, (self.Hq, self.T), f32)
            elif name.endswith("_acc"):
                _expect(name, t, (self.P, self.Hkv, self.D), f32)
            elif base in ("lse", "rowdot"):
                _expect(name, t, (self.Hq, rows), f32)
            elif base in ("q", "o", "do", "dq"):
                _expect(name, t, (rows, self.Hq, self.D), self.dtype)
            elif base in ("k", "v", "dk", "dv"):
                _expect(name, t, (rows, self.Hkv, self.D), self.dtype)
            else:
                raise ValueError(f"unknown tensor name {name}")
        for name, t in named.items():
            if t is None:
                continue
            if not t.is_cuda or t.device != self.device:
                raise ValueError(f"{name} must be on {self.device}")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")

    def empty(self, *shape, dtype=None):
        return torch.empty(*shape, dtype=self.dtype if dtype is None else dtype, device=self.device)

    def workspace_bytes(self, op: int) -> int:
        return _lib.workspace_bytes(self.dims, op)

    def workspace(self, op: int, ws=None, key_range=None):
        """(pointer, bytes) of a workspace for operation `op` (over prompt keys key_range =
        (begin, end) for the ops that take one): `ws` when given (a uint8 GPU tensor of at
        least the needed size), else a new one."""
        n = (self.workspace_bytes(op) if key_range is None
             else _lib.range_workspace_bytes(self.dims, op, key_range[0], key_range[1]))
        if ws is None:
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)
        elif ws.numel() < n:
            raise ValueError(f"workspace of {ws.numel()} bytes, {n} needed")
        self._ws_alive = ws
        return ws.data_ptr(), ws.numel()


def _check_range(tr: "Tree", key_begin: int, key_end: int) -> None:
    if not 0 <= key_begin < key_end <= tr.P:
        raise ValueError(f"prompt key range [{key_begin}, {key_end}) not inside [0, {tr.P}) or empty")


def replay_prompt_fwd(tr: Tree, k_p, v_p, q_r, key_begin: int = 0, key_end: Optional[int] = None,
                      out=None, ws=None):
    """Partial state (o_part float32 [T][Hq][D], lse_part [Hq][T]) of every branch row over
    prompt keys [key_begin, key_end)."""
    key_end = tr.P if key_end is None else key_end
    _check_range(tr, key_begin, key_end)
    o, l = out if out is not None else (tr.empty(tr.T, tr.Hq, tr.D, dtype=torch.float32),
                                        tr.empty(tr.Hq, tr.T, dtype=torch.float32))
    tr.check(k_p=k_p, v_p=v_p, q_r=q_r, o_part=o, lse_part=l)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_PROMPT_FWD, ws, (key_begin, key_end))
    st = _lib.augtree_replay_prompt_fwd(tr.dims, k_p.data_ptr(), v_p.data_ptr(), q_r.data_ptr(), key_begin,
                                        key_end, o.data_ptr(), l.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_prompt_fwd")
    return o, l


def replay_local_fwd(tr: Tree, q_r, k_r, v_r, out=None, ws=None):
    """Partial state of every branch row over its own branch (causal)."""
    o, l = out if out is not None else (tr.empty(tr.T, tr.Hq, tr.D, dtype=torch.float32),
                                        tr.empty(tr.Hq, tr.T, dtype=torch.float32))
    tr.check(q_r=q_r, k_r=k_r, v_r=v_r, o_part=o, lse_part=l)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_LOCAL_FWD, ws)
    st = _lib.augtree_replay_local_fwd(tr.dims, q_r.data_ptr(), k_r.data_ptr(), v_r.data_ptr(), o.data_ptr(),
                                       l.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_local_fwd")
    return o, l


def merge_partials(tr: Tree, parts, out=None):
    """Exact log-sum-exp merge of [(o_part, lse_part), ...] -> (o_r dtype, lse_r)."""
    o, l = out if out is not None else (tr.empty(tr.T, tr.Hq, tr.D), tr.empty(tr.Hq, tr.T, dtype=torch.float32))
    if not 1 <= len(parts) <= _lib.AUGTREE_MAX_PARTS:
        raise ValueError(f"{len(parts)} parts, 1..{_lib.AUGTREE_MAX_PARTS} allowed")
    for po, pl in parts:
        tr.check(o_part=po, lse_part=pl)
    tr.check(o_r=o, lse_r=l)
    st = _lib.augtree_merge_partials(tr.dims, [p[0].data_ptr() for p in parts], [p[1].data_ptr() for p in parts],
                                     o.data_ptr(), l.data_ptr(), tr.stream())
    _lib._check(st, "augtree_merge_partials")
    return o, l


def row_dot(tr: Tree, o, d_o, out=None):
    """rowdot [Hq][rows] = sum_d dO * O for rows = o.shape[0] (P or T_R)."""
    rows = int(o.shape[0])
    if rows not in (tr.P, tr.T):
        raise ValueError(f"row_dot over {rows} rows: neither P={tr.P} nor T_R={tr.T}")
    r = out if out is not None else tr.empty(tr.Hq, rows, dtype=torch.float32)
    sfx = "_p" if rows == tr.P else "_r"
    tr.check(**{"o" + sfx: o, "do" + sfx: d_o, "rowdot" + sfx: r})
    st = _lib.augtree_row_dot(tr.dims, rows, o.data_ptr(), d_o.data_ptr(), r.data_ptr(), tr.stream())
    _lib._check(st, "augtree_row_dot")
    return r


def replay_prompt_bwd(tr: Tree, k_p, v_p, q_r, lse_r, rowdot_r, do_r, key_begin: int = 0,
                      key_end: Optional[int] = None, dk_acc=None, dv_acc=None, ws=None):
    """Rows [key_begin, key_end) of the branches' summed prompt K/V gradient (float32
    [P][Hkv][D] buffers, allocated when not given)."""
    key_end = tr.P if key_end is None else key_end
    _check_range(tr, key_begin, key_end)
    if (dk_acc is None) != (dv_acc is None):
        raise ValueError("dk_acc and dv_acc must both be given or both be None")
    if dk_acc is None:
        dk_acc = tr.empty(tr.P, tr.Hkv, tr.D, dtype=torch.float32)
        dv_acc = tr.empty(tr.P, tr.Hkv, tr.D, dtype=torch.float32)
    tr.check(k_p=k_p, v_p=v_p, q_r=q_r, lse_r=lse_r, rowdot_r=rowdot_r, do_r=do_r, dk_acc=dk_acc,
             dv_acc=dv_acc)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_PROMPT_BWD, ws, (key_begin, key_end))
    st = _lib.augtree_replay_prompt_bwd(tr.dims, k_p.data_ptr(), v_p.data_ptr(), q_r.data_ptr(), lse_r.data_ptr(),
                                        rowdot_r.data_ptr(), do_r.data_ptr(), key_begin, key_end, dk_acc.data_ptr(),
                                        dv_acc.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_prompt_bwd")
    return dk_acc, dv_acc


def replay_local_bwd(tr: Tree, q_r, k_r, v_r, lse_r, rowdot_r, do_r, out=None, ws=None):
    dk, dv = out if out is not None else (torch.empty_like(k_r), torch.empty_like(v_r))
    tr.check(q_r=q_r, k_r=k_r, v_r=v_r, lse_r=lse_r, rowdot_r=rowdot_r, do_r=do_r, dk_r=dk, dv_r=dv)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_LOCAL_BWD, ws)
    st = _lib.augtree_replay_local_bwd(tr.dims, q_r.data_ptr(), k_r.data_ptr(), v_r.data_ptr(), lse_r.data_ptr(),
                                       rowdot_r.data_ptr(), do_r.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_local_bwd")
    return dk, dv


def replay_dq(tr: Tree, k_p, v_p, q_r, k_r, v_r, lse_r, rowdot_r, do_r, out=None, ws=None):
    dq = out if out is not None else torch.empty_like(q_r)
    tr.check(k_p=k_p, v_p=v_p, q_r=q_r, k_r=k_r, v_r=v_r, lse_r=lse_r, rowdot_r=rowdot_r, do_r=do_r, dq_r=dq)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_DQ, ws)
    st = _lib.augtree_replay_dq(tr.dims, k_p.data_ptr(), v_p.data_ptr(), q_r.data_ptr(), k_r.data_ptr(),
                                v_r.data_ptr(), lse_r.data_ptr(), rowdot_r.data_ptr(), do_r.data_ptr(),
                                dq.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_dq")
    return dq


def replay_prompt_dq(tr: Tree, k_p, v_p, q_r, lse_r, rowdot_r, do_r, key_begin: int = 0,
                     key_end: Optional[int] = None, out=None, ws=None):
    """float32 dQ partial [T][Hq][D] of every branch row over prompt keys [key_begin, key_end)
    (one stationary prompt-K/V shard's share)."""
    key_end = tr.P if key_end is None else key_end
    _check_range(tr, key_begin, key_end)
    dq = out if out is not None else tr.empty(tr.T, tr.Hq, tr.D, dtype=torch.float32)
    tr.check(k_p=k_p, v_p=v_p, q_r=q_r, lse_r=lse_r, rowdot_r=rowdot_r, do_r=do_r, dq_part=dq)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_PROMPT_DQ, ws, (key_begin, key_end))
    st = _lib.augtree_replay_prompt_dq(tr.dims, k_p.data_ptr(), v_p.data_ptr(), q_r.data_ptr(), lse_r.data_ptr(),
                                       rowdot_r.data_ptr(), do_r.data_ptr(), key_begin, key_end, dq.data_ptr(),
                                       wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_prompt_dq")
    return dq


def replay_local_dq(tr: Tree, q_r, k_r, v_r, lse_r, rowdot_r, do_r, out=None, ws=None):
    """float32 dQ partial [T][Hq][D] of every branch row over its own branch keys."""
    dq = out if out is not None else tr.empty(tr.T, tr.Hq, tr.D, dtype=torch.float32)
    tr.check(q_r=q_r, k_r=k_r, v_r=v_r, lse_r=lse_r, rowdot_r=rowdot_r, do_r=do_r, dq_part=dq)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_REPLAY_LOCAL_DQ, ws)
    st = _lib.augtree_replay_local_dq(tr.dims, q_r.data_ptr(), k_r.data_ptr(), v_r.data_ptr(), lse_r.data_ptr(),
                                      rowdot_r.data_ptr(), do_r.data_ptr(), dq.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_replay_local_dq")
    return dq


def sum_parts(tr: Tree, parts, out=None):
    """dtype [rows][Hq][D] = fixed-order sum of float32 partials of that layout (rows = T_R)."""
    if not 1 <= len(parts) <= _lib.AUGTREE_MAX_PARTS:
        raise ValueError(f"{len(parts)} parts, 1..{_lib.AUGTREE_MAX_PARTS} allowed")
    for p in parts:
        tr.check(dq_part=p)
    dq = out if out is not None else tr.empty(tr.T, tr.Hq, tr.D)
    tr.check(dq_r=dq)
    st = _lib.augtree_sum_parts(tr.dims, tr.T, [p.data_ptr() for p in parts], dq.data_ptr(), tr.stream())
    _lib._check(st, "augtree_sum_parts")
    return dq


def prefill_kv_bwd(tr: Tree, q_p, k_p, v_p, lse_p, rowdot_p, do_p, dk_acc=None, dv_acc=None, out=None, ws=None):
    dk, dv = out if out is not None else (torch.empty_like(k_p), torch.empty_like(v_p))
    if (dk_acc is None) != (dv_acc is None):
        raise ValueError("dk_acc and dv_acc must both be given or both be None")
    tr.check(q_p=q_p, k_p=k_p, v_p=v_p, lse_p=lse_p, rowdot_p=rowdot_p, do_p=do_p, dk_p_acc=dk_acc,
             dv_p_acc=dv_acc, dk_p=dk, dv_p=dv)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_PREFILL_KV_BWD, ws)
    st = _lib.augtree_prefill_kv_bwd(tr.dims, q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(), lse_p.data_ptr(),
                                     rowdot_p.data_ptr(), do_p.data_ptr(), _ptr(dk_acc), _ptr(dv_acc),
                                     dk.data_ptr(), dv.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_prefill_kv_bwd")
    return dk, dv


def prefill_dq(tr: Tree, q_p, k_p, v_p, lse_p, rowdot_p, do_p, out=None, ws=None):
    dq = out if out is not None else torch.empty_like(q_p)
    tr.check(q_p=q_p, k_p=k_p, v_p=v_p, lse_p=lse_p, rowdot_p=rowdot_p, do_p=do_p, dq_p=dq)
    wp, wn = tr.workspace(_lib.AUGTREE_OP_PREFILL_DQ, ws)
    st = _lib.augtree_prefill_dq(tr.dims, q_p.data_ptr(), k_p.data_ptr(), v_p.data_ptr(), lse_p.data_ptr(),
                                 rowdot_p.data_ptr(), do_p.data_ptr(), dq.data_ptr(), wp, wn, tr.stream())
    _lib._check(st, "augtree_prefill_dq")
    return dq


def assign_units(weights: Sequence[float], rounds: int, lanes: int, exact_max: int = 12):
    """Replay-unit assignment (augtree_assign_units): (cell of each unit, objective), where cell
    = round * lanes + lane and the objective is the sum over rounds of the largest lane load."""
    n = len(weights)
    w = (ctypes.c_double * max(n, 1))(*[float(x) for x in weights])
    cells = (ctypes.c_int32 * max(n, 1))()
    cost = ctypes.c_double(0.0)
    _lib._check(_lib.augtree_assign_units(w, int(n), int(rounds), int(lanes), int(exact_max), cells,
                                          ctypes.byref(cost)), "augtree_assign_units")
    return [int(cells[k]) for k in range(n)], float(cost.value)
