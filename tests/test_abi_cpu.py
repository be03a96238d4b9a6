"""The C-ABI library loads, exports every function include/augtree.h declares, and rejects
bad arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from shared_prefix_attention_prompt_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "augtree.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libaugtree.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(augtree_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_bound_entry_points():
    assert declared_functions() == sorted(_lib.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT (augtree_\w+)", out.stdout))
        assert set(declared_functions()) <= exported


def test_version_and_status_strings():
    assert _lib.abi_version() == 4
    assert _lib.status_string(_lib.AUGTREE_OK) == "AUGTREE_OK"
    assert _lib.status_string(_lib.AUGTREE_ERR_WORKSPACE) == "AUGTREE_ERR_WORKSPACE"
    assert _lib.status_string(99) == "AUGTREE_ERR_UNKNOWN"


def _dims(P=16, off=(0, 4, 9), Hq=4, Hkv=2, D=128, scale=0.088, dtype=_lib.AUGTREE_BF16):
    return _lib.make_dims(P, list(off), Hq, Hkv, D, scale, dtype)


def test_workspace_sizes():
    # transposed copies: H x D x cols bf16 (stored tile by tile) with the prompt padded to 64 columns and every
    # branch padded to 64 columns on its own (30 -> 64, 40 -> 64)
    d, keep = _dims(P=100, off=(0, 30, 70), Hq=4, Hkv=2, D=128)
    T, P, Hq, Hkv, D = 70, 100, 4, 2, 128
    vp_t = Hkv * D * 128 * 2
    resp_kv_t = Hkv * D * 128 * 2
    resp_q_t = Hq * D * 128 * 2
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_PREFILL_FWD) == vp_t
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_PROMPT_FWD) == vp_t
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_LOCAL_FWD) == resp_kv_t
    # row statistics in the same column order: [2][Hq][cols] float32
    resp_st = 2 * Hq * 128 * 4
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_LOCAL_BWD) == 2 * resp_q_t + resp_st
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_DQ) == vp_t + resp_kv_t
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_PREFILL_KV_BWD) == 2 * Hq * D * 128 * 2 + 2 * Hq * 128 * 4
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_PREFILL_DQ) == vp_t
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_PROMPT_BWD) >= 2 * resp_q_t + resp_st
    rf = _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_FWD)
    assert rf >= 2 * T * Hq * D * 4 + 2 * T * Hq * 4 + vp_t + resp_kv_t
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_BWD) >= T * Hq * 4 + 2 * resp_q_t + vp_t + resp_kv_t
    assert _lib.workspace_bytes(d, _lib.AUGTREE_OP_PREFILL_BWD) >= P * Hq * 4 + 2 * Hq * D * 128 * 2 + vp_t
    assert _lib.workspace_bytes(d, 99) == 0
    bad, keep2 = _dims(off=(0, 4, 4))
    assert _lib.workspace_bytes(bad, _lib.AUGTREE_OP_REPLAY_FWD) == 0


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status,needle", [
    (dict(P=0), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "prompt_len"),
    (dict(off=(1, 4)), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "branch_offsets[0]"),
    (dict(off=(0, 4, 4)), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "strictly increasing"),
    (dict(off=(0, 5, 3)), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "strictly increasing"),
    (dict(Hq=3, Hkv=2), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(Hkv=0), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "head counts"),
    (dict(D=96), _lib.AUGTREE_ERR_UNSUPPORTED, "head_dim"),
    (dict(D=128, dtype=_lib.AUGTREE_F32), _lib.AUGTREE_ERR_UNSUPPORTED, "head_dim"),
    (dict(D=0), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "head_dim"),
    (dict(scale=0.0), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "softmax_scale"),
    (dict(scale=float("inf")), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "softmax_scale"),
    (dict(dtype=5), _lib.AUGTREE_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(Hq=65536, Hkv=1), _lib.AUGTREE_ERR_UNSUPPORTED, "bytes per row"),
])
def test_invalid_dims_are_rejected(kw, status, needle):
    d, keep = _dims(**kw)
    st = _lib.augtree_prefill_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == status
    assert needle in _lib.last_error()


def test_too_many_branches_rejected():
    off = list(range(0, 130))
    d, keep = _lib.make_dims(8, off, 2, 2, 128, 0.1, _lib.AUGTREE_BF16)
    assert d.num_branches == 129
    st = _lib.augtree_replay_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.AUGTREE_ERR_INVALID_ARGUMENT and "num_branches" in _lib.last_error()


def test_null_and_misaligned_pointers_rejected():
    d, keep = _dims()
    st = _lib.augtree_prefill_fwd(d, None, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == _lib.AUGTREE_ERR_INVALID_ARGUMENT and "q_p is NULL" in _lib.last_error()
    st = _lib.augtree_prefill_fwd(d, FAKE, FAKE + 2, FAKE, FAKE, FAKE, None, 0, None)
    assert st == _lib.AUGTREE_ERR_INVALID_ARGUMENT and "k_p is not 16-byte aligned" in _lib.last_error()
    st = _lib.augtree_prefill_bwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                  FAKE, 1 << 30, None)
    assert st == _lib.AUGTREE_ERR_INVALID_ARGUMENT and "both" in _lib.last_error()


def test_missing_or_small_workspace_rejected():
    d, keep = _dims()
    need = _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_FWD)
    st = _lib.augtree_replay_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE
    st = _lib.augtree_replay_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE and "needed" in _lib.last_error()
    st = _lib.augtree_replay_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE and "aligned" in _lib.last_error()
    need_b = _lib.workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_BWD)
    st = _lib.augtree_replay_bwd(d, *([FAKE] * 13), None, need_b, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE
    need_p = _lib.workspace_bytes(d, _lib.AUGTREE_OP_PREFILL_FWD)
    st = _lib.augtree_prefill_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need_p - 1, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE
    st = _lib.augtree_replay_local_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE
    st = _lib.augtree_prefill_dq(d, *([FAKE] * 7), None, 0, None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE


def test_last_error_is_per_thread():
    import threading
    d, keep = _dims(P=0)
    _lib.augtree_prefill_fwd(d, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    main_msg = _lib.last_error()
    seen = []
    t = threading.Thread(target=lambda: seen.append(_lib.last_error()))
    t.start()
    t.join()
    assert "prompt_len" in main_msg and seen == [""]


@pytest.mark.parametrize("P,lens,Hq,Hkv", [
    (32768, [1024] * 8, 8, 8),          # many key tiles, short branches: splits of 2..4 parts
    (3000, [700, 45, 1210], 8, 2, ),    # few key tiles: splits up to 16 parts
    (1500, [300, 200, 417], 4, 1),
])
def test_prompt_bwd_range_workspace_covers_every_range(P, lens, Hq, Hkv):
    # The split count of the prompt K/V gradient depends on the number of keys in the range;
    # for ranges that are not whole 256-key blocks it is clamped to the reserve, so no range
    # needs more than the op-wide workspace. Walk every length (every start for the short
    # prompts) on the host.
    off = [0]
    for r in lens:
        off.append(off[-1] + r)
    d, keep = _lib.make_dims(P, off, Hq, Hkv, 128, 128 ** -0.5, _lib.AUGTREE_BF16)
    op = _lib.AUGTREE_OP_REPLAY_PROMPT_BWD
    whole = _lib.workspace_bytes(d, op)
    assert whole > 0
    worst = 0
    starts = range(P) if P <= 3000 else [0, 1, 255, 7423, 25345 - 1]
    for kb in starts:
        for ke in (range(kb + 1, P + 1) if P <= 3000 else [kb + 25345, P] if kb + 25345 <= P else [P]):
            need = _lib.range_workspace_bytes(d, op, kb, ke)
            assert 0 < need <= whole, (kb, ke, need, whole)
            worst = max(worst, need)
    if P == 32768:
        # the length the advisor found (25345 keys: 3 parts) fits the op-wide reserve
        for n in range(1, P + 1):
            assert _lib.range_workspace_bytes(d, op, 0, n) <= whole, n
    assert worst <= whole
    # the fwd range workspace is the range's transposed V
    assert _lib.range_workspace_bytes(d, _lib.AUGTREE_OP_REPLAY_PROMPT_FWD, 0, 65) == Hkv * 128 * 128 * 2
    assert _lib.range_workspace_bytes(d, op, 5, 5) == 0
    assert _lib.range_workspace_bytes(d, op, 0, P + 1) == 0


def test_prompt_bwd_rejects_a_workspace_smaller_than_its_range_needs():
    d, keep = _lib.make_dims(3000, [0, 700, 745, 1955], 8, 2, 128, 128 ** -0.5, _lib.AUGTREE_BF16)
    op = _lib.AUGTREE_OP_REPLAY_PROMPT_BWD
    for kb, ke in [(0, 3000), (13, 1777), (2999, 3000)]:
        need = _lib.range_workspace_bytes(d, op, kb, ke)
        st = _lib.augtree_replay_prompt_bwd(d, *([FAKE] * 6), kb, ke, FAKE, FAKE, FAKE, need - 1, None)
        assert st == _lib.AUGTREE_ERR_WORKSPACE and "needed" in _lib.last_error()


def test_noalloc_rejects_trees_beyond_its_scratch_before_any_call():
    # the size check runs before the scratch lookup and before anything is enqueued
    big, keep = _lib.make_dims(1024, [0, 100000], 32, 8, 128, 128 ** -0.5, _lib.AUGTREE_BF16)
    assert _lib.workspace_bytes(big, _lib.AUGTREE_OP_REPLAY_FWD) > _lib.AUGTREE_NOALLOC_SCRATCH_BYTES
    st = _lib.augtree_replay_fwd_noalloc(big, *([FAKE] * 7), None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE and "static scratch" in _lib.last_error()
    d, keep2 = _dims()
    st = _lib.augtree_replay_fwd_noalloc(d, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == _lib.AUGTREE_ERR_INVALID_ARGUMENT and "v_p is NULL" in _lib.last_error()
