"""The no-allocation replay forward (augtree_replay_fwd_noalloc, for callers that cannot
allocate: graph capture, tight serving loops) through the C ABI gives bitwise the output of
augtree_replay_fwd, on two calls in a row whose second tree is smaller (the static scratch
keeps the first call's contents)."""
import pytest
import torch

from shared_prefix_attention_prompt_amd import _lib
from tests.gpu_run import config_inputs, log, upload
from workloads import make_inputs, make_shape

pytestmark = pytest.mark.gpu


def _call(w, t, noalloc: bool):
    s = w.shape
    dt = _lib.AUGTREE_BF16 if s.dtype == "bf16" else _lib.AUGTREE_F32
    dims, keep = _lib.make_dims(s.P, s.offsets, s.Hq, s.Hkv, s.D, s.D ** -0.5, dt)
    o = torch.full_like(t["q_r"], float("nan"))
    lse = torch.full((s.Hq, s.T), float("nan"), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [t[k].data_ptr() for k in ("k_p", "v_p", "q_r", "k_r", "v_r")] + [o.data_ptr(), lse.data_ptr()]
    if noalloc:
        st = _lib.augtree_replay_fwd_noalloc(dims, *ptrs, stream)
    else:
        need = _lib.workspace_bytes(dims, _lib.AUGTREE_OP_REPLAY_FWD)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        st = _lib.augtree_replay_fwd(dims, *ptrs, ws.data_ptr(), need, stream)
    assert st == _lib.AUGTREE_OK, _lib.last_error()
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_replay_fwd_matches_the_allocating_call_twice():
    big = config_inputs(3)   # the P = 8192, 16/4-head tree: about 188 MB of scratch
    small = make_inputs(make_shape(300, [31, 250, 7], 4, 2, 64, dtype="bf16"), seed=300)
    for name, w in (("P=8192 tree", big), ("small tree", small)):
        t = upload(w)
        need = _lib.workspace_bytes(_lib.make_dims(w.shape.P, w.shape.offsets, w.shape.Hq, w.shape.Hkv,
                                                   w.shape.D, 0.1, _lib.AUGTREE_BF16)[0],
                                    _lib.AUGTREE_OP_REPLAY_FWD)
        log(f"no-alloc replay forward: {name}, {need} of {_lib.AUGTREE_NOALLOC_SCRATCH_BYTES} scratch bytes")
        a_o, a_l = _call(w, t, noalloc=False)
        b_o, b_l = _call(w, t, noalloc=True)
        assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)
        assert bool(torch.isfinite(b_l).all())


def test_noalloc_rejects_a_tree_beyond_the_scratch():
    w = make_inputs(make_shape(64, [9, 5], 2, 1, 64, dtype="bf16"), seed=1)
    t = upload(w)
    dims, keep = _lib.make_dims(64, [0, 70000], 32, 8, 128, 0.1, _lib.AUGTREE_BF16)
    st = _lib.augtree_replay_fwd_noalloc(dims, *([t["q_r"].data_ptr()] * 7), None)
    assert st == _lib.AUGTREE_ERR_WORKSPACE
