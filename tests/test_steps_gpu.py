"""The single-step entry points: composing them reproduces the composite calls bit for bit,
and splitting the prompt keys into stationary shards (one partial state per shard, merged
per query row; the MoveQ semantics of §3.3) matches the oracle."""
import pytest
import torch

from oracle import flattened_tree_attention
from shared_prefix_attention_prompt_amd import ops
from tests.gpu_run import compare, log, run_path, upload
from workloads import make_inputs, make_shape

pytestmark = pytest.mark.gpu


def _steps(w, t):
    s = w.shape
    tr = ops.Tree(s.P, s.offsets, s.Hq, s.Hkv, s.D, s.torch_dtype, "cuda:0")
    o_p, lse_p = ops.prefill_fwd(t["q_p"], t["k_p"], t["v_p"], None, s.offsets)
    a = ops.replay_prompt_fwd(tr, t["k_p"], t["v_p"], t["q_r"])
    b = ops.replay_local_fwd(tr, t["q_r"], t["k_r"], t["v_r"])
    o_r, lse_r = ops.merge_partials(tr, [a, b])
    rd_r = ops.row_dot(tr, o_r, t["do_r"])
    dk_acc, dv_acc = ops.replay_prompt_bwd(tr, t["k_p"], t["v_p"], t["q_r"], lse_r, rd_r, t["do_r"])
    dk_r, dv_r = ops.replay_local_bwd(tr, t["q_r"], t["k_r"], t["v_r"], lse_r, rd_r, t["do_r"])
    dq_r = ops.replay_dq(tr, t["k_p"], t["v_p"], t["q_r"], t["k_r"], t["v_r"], lse_r, rd_r, t["do_r"])
    rd_p = ops.row_dot(tr, o_p, t["do_p"])
    dk_p, dv_p = ops.prefill_kv_bwd(tr, t["q_p"], t["k_p"], t["v_p"], lse_p, rd_p, t["do_p"], dk_acc, dv_acc)
    dq_p = ops.prefill_dq(tr, t["q_p"], t["k_p"], t["v_p"], lse_p, rd_p, t["do_p"])
    torch.cuda.synchronize()
    return {"o_p": o_p, "lse_p": lse_p, "o_r": o_r, "lse_r": lse_r, "dq_p": dq_p, "dk_p": dk_p, "dv_p": dv_p,
            "dq_r": dq_r, "dk_r": dk_r, "dv_r": dv_r, "dk_p_acc": dk_acc, "dv_p_acc": dv_acc}


@pytest.mark.parametrize("P,lens,Hq,Hkv", [(300, [31, 250, 7], 4, 2), (8192, [900, 2048, 513], 16, 4)])
def test_steps_compose_to_the_composite_calls(P, lens, Hq, Hkv):
    w = make_inputs(make_shape(P, lens, Hq, Hkv, 128, dtype="bf16"), seed=P)
    t = upload(w)
    a = run_path(w, t)
    b = _steps(w, t)
    for k in b:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("cuts", [[0, 100, 101, 300, 517], [0, 517], [0, 64, 128, 256, 384, 500, 510, 517]])
def test_moveq_prompt_shards_match_oracle(cuts):
    # Prompt K/V split into stationary shards; every branch row's partial state per shard
    # plus its own-branch partial are merged per row (d+1 parts, at most 8).
    P = cuts[-1]
    w = make_inputs(make_shape(P, [40, 129, 3], 8, 2, 128, dtype="bf16"), seed=len(cuts))
    s = w.shape
    t = upload(w)
    tr = ops.Tree(s.P, s.offsets, s.Hq, s.Hkv, s.D, s.torch_dtype, "cuda:0")
    parts = [ops.replay_prompt_fwd(tr, t["k_p"], t["v_p"], t["q_r"], a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(ops.replay_local_fwd(tr, t["q_r"], t["k_r"], t["v_r"]))
    o_r, lse_r = ops.merge_partials(tr, parts)
    # prompt K/V gradient assembled shard by shard
    full = run_path(w, t)
    dk = torch.empty(s.P, s.Hkv, s.D, dtype=torch.float32, device="cuda:0")
    dv = torch.empty_like(dk)
    rd_r = ops.row_dot(tr, full["o_r"], t["do_r"])
    for a, b in zip(cuts[:-1], cuts[1:]):
        ops.replay_prompt_bwd(tr, t["k_p"], t["v_p"], t["q_r"], full["lse_r"], rd_r, t["do_r"], a, b, dk, dv)
    torch.cuda.synchronize()
    log(f"shards {cuts}")
    ref = flattened_tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, do_p=w.do_p, do_r=w.do_r)
    compare("o_r", o_r, ref["o_r"], "bf16")
    compare("lse_r", lse_r, ref["lse_r"], "bf16")
    # the branch sum of the prompt gradient equals the full call's (same tiles, same order
    # unless the split count differs per range) to fp32 rounding
    assert torch.allclose(dk, full["dk_p_acc"], atol=1e-4, rtol=1e-4)
    assert torch.allclose(dv, full["dv_p_acc"], atol=1e-4, rtol=1e-4)
    # and adding the prefill contribution reproduces the oracle's total prompt gradient
    rd_p = ops.row_dot(tr, full["o_p"], t["do_p"])
    dk_p, dv_p = ops.prefill_kv_bwd(tr, t["q_p"], t["k_p"], t["v_p"], full["lse_p"], rd_p, t["do_p"], dk, dv)
    compare("dk_p", dk_p, ref["dk_p"], "bf16")
    compare("dv_p", dv_p, ref["dv_p"], "bf16")


def test_merge_of_one_part_is_a_copy_and_empty_key_range_rejected():
    w = make_inputs(make_shape(64, [5, 9], 2, 1, 64, dtype="bf16"), seed=3)
    s = w.shape
    t = upload(w)
    tr = ops.Tree(s.P, s.offsets, s.Hq, s.Hkv, s.D, s.torch_dtype, "cuda:0")
    o, l = ops.replay_prompt_fwd(tr, t["k_p"], t["v_p"], t["q_r"])
    m, ml = ops.merge_partials(tr, [(o, l)])
    torch.cuda.synchronize()
    assert torch.equal(ml, l)
    assert torch.equal(m, o.to(torch.bfloat16))
    from shared_prefix_attention_prompt_amd import _lib
    with pytest.raises(ValueError):
        ops.replay_prompt_fwd(tr, t["k_p"], t["v_p"], t["q_r"], 10, 10)
    # the library rejects it too, before any launch
    st = _lib.augtree_replay_prompt_fwd(tr.dims, t["k_p"].data_ptr(), t["v_p"].data_ptr(), t["q_r"].data_ptr(),
                                        10, 10, o.data_ptr(), l.data_ptr(), None, 0, None)
    assert st == _lib.AUGTREE_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("cuts", [[0, 517], [0, 100, 101, 300, 517], [0, 64, 128, 256, 384, 500, 510, 517],
                                  [0, 1, 2, 3, 4, 5, 6, 517]])
def test_moveq_sharded_dq_matches_oracle(cuts):
    # dQ of the branch rows in the prompt-K/V shard layout: each shard's float32 partial over its
    # key range (with the rows' full LSE and row dot), the own-branch partial, and their
    # fixed-order sum, for 1..7 uneven shards
    P = cuts[-1]
    w = make_inputs(make_shape(P, [40, 129, 3], 8, 2, 128, dtype="bf16"), seed=10 + len(cuts))
    s = w.shape
    t = upload(w)
    tr = ops.Tree(s.P, s.offsets, s.Hq, s.Hkv, s.D, s.torch_dtype, "cuda:0")
    full = run_path(w, t)
    rd_r = ops.row_dot(tr, full["o_r"], t["do_r"])
    parts = [ops.replay_prompt_dq(tr, t["k_p"], t["v_p"], t["q_r"], full["lse_r"], rd_r, t["do_r"], a, b)
             for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(ops.replay_local_dq(tr, t["q_r"], t["k_r"], t["v_r"], full["lse_r"], rd_r, t["do_r"]))
    dq = ops.sum_parts(tr, parts)
    torch.cuda.synchronize()
    log(f"dQ shards {cuts}")
    ref = flattened_tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, do_p=w.do_p, do_r=w.do_r)
    compare("dq_r (sharded)", dq, ref["dq_r"], "bf16")
    # the same sums as the one-pass dQ up to float32 rounding of the partials
    assert torch.allclose(dq.float(), full["dq_r"].float(), atol=1e-2, rtol=1e-2)
    # each shard's partial alone is not the whole gradient (the shards really split the keys)
    if len(parts) > 2:
        assert not torch.allclose(parts[0], dq.float(), atol=1e-2)
