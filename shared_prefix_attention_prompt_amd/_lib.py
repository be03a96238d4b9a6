"""ctypes binding of libaugtree.so: the C ABI of include/augtree.h under the same names.

Argument marshalling only. The library is loaded from this package's directory; if it is
missing the import of any entry point raises, there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libaugtree.so")

AUGTREE_F32 = 0
AUGTREE_BF16 = 1
AUGTREE_OK = 0
AUGTREE_ERR_INVALID_ARGUMENT = 1
AUGTREE_ERR_UNSUPPORTED = 2
AUGTREE_ERR_WORKSPACE = 3
AUGTREE_ERR_HIP = 4
AUGTREE_OP_PREFILL_FWD = 0
AUGTREE_OP_REPLAY_FWD = 1
AUGTREE_OP_REPLAY_BWD = 2
AUGTREE_OP_PREFILL_BWD = 3
AUGTREE_OP_REPLAY_PROMPT_BWD = 4
AUGTREE_OP_REPLAY_PROMPT_FWD = 5
AUGTREE_OP_REPLAY_LOCAL_FWD = 6
AUGTREE_OP_REPLAY_LOCAL_BWD = 7
AUGTREE_OP_REPLAY_DQ = 8
AUGTREE_OP_PREFILL_KV_BWD = 9
AUGTREE_OP_PREFILL_DQ = 10
AUGTREE_OP_REPLAY_PROMPT_DQ = 11
AUGTREE_OP_REPLAY_LOCAL_DQ = 12
AUGTREE_MAX_BRANCHES = 128
AUGTREE_MAX_PARTS = 8
AUGTREE_ASSIGN_EXACT_MAX = 16
AUGTREE_NOALLOC_SCRATCH_BYTES = 256 << 20

ENTRY_POINTS = ["augtree_prefill_fwd", "augtree_replay_fwd", "augtree_replay_bwd",
                "augtree_prefill_bwd", "augtree_replay_prompt_fwd", "augtree_replay_local_fwd",
                "augtree_merge_partials", "augtree_row_dot", "augtree_replay_prompt_bwd",
                "augtree_replay_local_bwd", "augtree_replay_dq", "augtree_prefill_kv_bwd",
                "augtree_prefill_dq", "augtree_replay_prompt_dq", "augtree_replay_local_dq",
                "augtree_sum_parts", "augtree_assign_units", "augtree_replay_fwd_noalloc",
                "augtree_workspace_bytes",
                "augtree_range_workspace_bytes",
                "augtree_status_string", "augtree_last_error", "augtree_abi_version"]


class augtree_dims(ctypes.Structure):
    _fields_ = [("prompt_len", ctypes.c_int32), ("num_branches", ctypes.c_int32),
                ("branch_offsets", ctypes.POINTER(ctypes.c_int32)),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class AugtreeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {detail}")


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libaugtree.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -m shared_prefix_attention_prompt_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(augtree_dims)
    st = ctypes.c_int
    lib.augtree_prefill_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_replay_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_replay_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_prefill_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    i32 = ctypes.c_int32
    fpp = ctypes.POINTER(ctypes.c_void_p)
    lib.augtree_replay_prompt_fwd.argtypes = [P, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.augtree_replay_local_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_merge_partials.argtypes = [P, i32, fpp, fpp, vp, vp, vp]
    lib.augtree_row_dot.argtypes = [P, i32, vp, vp, vp, vp]
    lib.augtree_replay_prompt_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.augtree_replay_local_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_replay_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_prefill_kv_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_prefill_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_assign_units.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    lib.augtree_replay_prompt_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, sz, vp]
    lib.augtree_replay_local_dq.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.augtree_sum_parts.argtypes = [P, i32, i32, fpp, vp, vp]
    lib.augtree_replay_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    for name in ENTRY_POINTS[:18]:
        getattr(lib, name).restype = st
    lib.augtree_workspace_bytes.argtypes = [P, ctypes.c_int]
    lib.augtree_workspace_bytes.restype = sz
    lib.augtree_range_workspace_bytes.argtypes = [P, ctypes.c_int, i32, i32]
    lib.augtree_range_workspace_bytes.restype = sz
    lib.augtree_status_string.argtypes = [ctypes.c_int]
    lib.augtree_status_string.restype = ctypes.c_char_p
    lib.augtree_last_error.argtypes = []
    lib.augtree_last_error.restype = ctypes.c_char_p
    lib.augtree_abi_version.argtypes = []
    lib.augtree_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def make_dims(P: int, offsets: Sequence[int], Hq: int, Hkv: int, D: int, scale: float,
              dtype: int):
    """(augtree_dims, keep-alive int32 array of the offsets)."""
    off = (ctypes.c_int32 * len(offsets))(*[int(x) for x in offsets])
    d = augtree_dims(int(P), len(offsets) - 1, ctypes.cast(off, ctypes.POINTER(ctypes.c_int32)),
                     int(Hq), int(Hkv), int(D), float(scale), int(dtype))
    return d, off


def status_string(status: int) -> str:
    return load().augtree_status_string(int(status)).decode()


def last_error() -> str:
    return load().augtree_last_error().decode()


def abi_version() -> int:
    return int(load().augtree_abi_version())


def workspace_bytes(dims: augtree_dims, op: int) -> int:
    return int(load().augtree_workspace_bytes(ctypes.byref(dims), int(op)))


def range_workspace_bytes(dims: augtree_dims, op: int, key_begin: int, key_end: int) -> int:
    return int(load().augtree_range_workspace_bytes(ctypes.byref(dims), int(op), int(key_begin),
                                                    int(key_end)))


def _check(status: int, where: str) -> None:
    if status != AUGTREE_OK:
        raise AugtreeError(status, where, last_error())


def augtree_assign_units(w, num_units, rounds, lanes, exact_max, cell, cost) -> int:
    """w: host double[num_units]; cell: host int32[num_units]; cost: host double (ctypes
    arrays or byref pointers)."""
    return load().augtree_assign_units(w, num_units, rounds, lanes, exact_max, cell, cost)


def augtree_prefill_fwd(dims, q_p, k_p, v_p, o_p, lse_p, ws, ws_bytes, stream) -> int:
    return load().augtree_prefill_fwd(ctypes.byref(dims), q_p, k_p, v_p, o_p, lse_p, ws, ws_bytes, stream)


def augtree_replay_fwd(dims, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, ws, ws_bytes, stream) -> int:
    return load().augtree_replay_fwd(ctypes.byref(dims), k_p, v_p, q_r, k_r, v_r, o_r, lse_r, ws,
                                     ws_bytes, stream)


def augtree_replay_bwd(dims, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, do_r, dq_r, dk_r, dv_r,
                       dk_p_acc, dv_p_acc, ws, ws_bytes, stream) -> int:
    return load().augtree_replay_bwd(ctypes.byref(dims), k_p, v_p, q_r, k_r, v_r, o_r, lse_r, do_r,
                                     dq_r, dk_r, dv_r, dk_p_acc, dv_p_acc, ws, ws_bytes, stream)


def augtree_prefill_bwd(dims, q_p, k_p, v_p, o_p, lse_p, do_p, dk_p_acc, dv_p_acc, dq_p, dk_p,
                        dv_p, ws, ws_bytes, stream) -> int:
    return load().augtree_prefill_bwd(ctypes.byref(dims), q_p, k_p, v_p, o_p, lse_p, do_p, dk_p_acc,
                                      dv_p_acc, dq_p, dk_p, dv_p, ws, ws_bytes, stream)


def augtree_replay_fwd_noalloc(dims, k_p, v_p, q_r, k_r, v_r, o_r, lse_r, stream) -> int:
    return load().augtree_replay_fwd_noalloc(ctypes.byref(dims), k_p, v_p, q_r, k_r, v_r, o_r, lse_r, stream)


def augtree_replay_prompt_fwd(dims, k_p, v_p, q_r, key_begin, key_end, o_part, lse_part, ws, ws_bytes,
                              stream) -> int:
    return load().augtree_replay_prompt_fwd(ctypes.byref(dims), k_p, v_p, q_r, int(key_begin), int(key_end),
                                            o_part, lse_part, ws, ws_bytes, stream)


def augtree_replay_local_fwd(dims, q_r, k_r, v_r, o_part, lse_part, ws, ws_bytes, stream) -> int:
    return load().augtree_replay_local_fwd(ctypes.byref(dims), q_r, k_r, v_r, o_part, lse_part, ws, ws_bytes,
                                           stream)


def augtree_merge_partials(dims, o_parts, lse_parts, o_r, lse_r, stream) -> int:
    n = len(o_parts)
    oa = (ctypes.c_void_p * max(n, 1))(*o_parts)
    la = (ctypes.c_void_p * max(len(lse_parts), 1))(*lse_parts)
    return load().augtree_merge_partials(ctypes.byref(dims), n, oa, la, o_r, lse_r, stream)


def augtree_row_dot(dims, rows, o, d_o, rowdot, stream) -> int:
    return load().augtree_row_dot(ctypes.byref(dims), int(rows), o, d_o, rowdot, stream)


def augtree_replay_prompt_bwd(dims, k_p, v_p, q_r, lse_r, rowdot_r, do_r, key_begin, key_end, dk_p_acc,
                              dv_p_acc, ws, ws_bytes, stream) -> int:
    return load().augtree_replay_prompt_bwd(ctypes.byref(dims), k_p, v_p, q_r, lse_r, rowdot_r, do_r,
                                            int(key_begin), int(key_end), dk_p_acc, dv_p_acc, ws, ws_bytes,
                                            stream)


def augtree_replay_local_bwd(dims, q_r, k_r, v_r, lse_r, rowdot_r, do_r, dk_r, dv_r, ws, ws_bytes,
                             stream) -> int:
    return load().augtree_replay_local_bwd(ctypes.byref(dims), q_r, k_r, v_r, lse_r, rowdot_r, do_r, dk_r,
                                           dv_r, ws, ws_bytes, stream)


def augtree_replay_dq(dims, k_p, v_p, q_r, k_r, v_r, lse_r, rowdot_r, do_r, dq_r, ws, ws_bytes, stream) -> int:
    return load().augtree_replay_dq(ctypes.byref(dims), k_p, v_p, q_r, k_r, v_r, lse_r, rowdot_r, do_r, dq_r,
                                    ws, ws_bytes, stream)


def augtree_prefill_kv_bwd(dims, q_p, k_p, v_p, lse_p, rowdot_p, do_p, dk_p_acc, dv_p_acc, dk_p, dv_p,
                           ws, ws_bytes, stream) -> int:
    return load().augtree_prefill_kv_bwd(ctypes.byref(dims), q_p, k_p, v_p, lse_p, rowdot_p, do_p, dk_p_acc,
                                         dv_p_acc, dk_p, dv_p, ws, ws_bytes, stream)


def augtree_prefill_dq(dims, q_p, k_p, v_p, lse_p, rowdot_p, do_p, dq_p, ws, ws_bytes, stream) -> int:
    return load().augtree_prefill_dq(ctypes.byref(dims), q_p, k_p, v_p, lse_p, rowdot_p, do_p, dq_p, ws,
                                     ws_bytes, stream)


def augtree_replay_prompt_dq(dims, k_p, v_p, q_r, lse_r, rowdot_r, do_r, key_begin, key_end, dq_part, ws,
                             ws_bytes, stream) -> int:
    return load().augtree_replay_prompt_dq(ctypes.byref(dims), k_p, v_p, q_r, lse_r, rowdot_r, do_r,
                                           int(key_begin), int(key_end), dq_part, ws, ws_bytes, stream)


def augtree_replay_local_dq(dims, q_r, k_r, v_r, lse_r, rowdot_r, do_r, dq_part, ws, ws_bytes, stream) -> int:
    return load().augtree_replay_local_dq(ctypes.byref(dims), q_r, k_r, v_r, lse_r, rowdot_r, do_r, dq_part,
                                          ws, ws_bytes, stream)


def augtree_sum_parts(dims, rows, parts, out, stream) -> int:
    n = len(parts)
    arr = (ctypes.c_void_p * max(n, 1))(*parts)
    return load().augtree_sum_parts(ctypes.byref(dims), int(rows), n, arr, out, stream)
