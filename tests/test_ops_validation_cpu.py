"""The torch-facing wrappers check every tensor's shape and dtype against the tree
(P, offsets, Hq, Hkv, D) before anything reaches the library: a mismatch raises ValueError
and launches no kernel. These checks come before the device check, so they run on the CPU."""
import pytest
import torch

from shared_prefix_attention_prompt_amd import ops

P, OFF, HQ, HKV, D = 40, [0, 7, 20], 4, 2, 64
T = OFF[-1]
bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def good():
    return dict(q_p=t(P, HQ, D), k_p=t(P, HKV, D), v_p=t(P, HKV, D), q_r=t(T, HQ, D), k_r=t(T, HKV, D),
                v_r=t(T, HKV, D), o_r=t(T, HQ, D), lse_r=t(HQ, T, dtype=torch.float32), do_r=t(T, HQ, D),
                o_p=t(P, HQ, D), lse_p=t(HQ, P, dtype=torch.float32), do_p=t(P, HQ, D))


def call_replay_fwd(x, off=OFF):
    return ops.replay_fwd(x["k_p"], x["v_p"], x["q_r"], x["k_r"], x["v_r"], off)


def call_replay_bwd(x, off=OFF):
    return ops.replay_bwd(x["k_p"], x["v_p"], x["q_r"], x["k_r"], x["v_r"], off, x["o_r"], x["lse_r"], x["do_r"])


def call_prefill_fwd(x, off=OFF):
    return ops.prefill_fwd(x["q_p"], x["k_p"], x["v_p"], None, off)


def call_prefill_bwd(x, off=OFF, acc=None):
    a = (None, None) if acc is None else acc
    return ops.prefill_bwd(x["q_p"], x["k_p"], x["v_p"], x["o_p"], x["lse_p"], x["do_p"], a[0], a[1], None, off)


@pytest.mark.parametrize("call,name,bad,needle", [
    (call_replay_fwd, "q_r", t(T + 1, HQ, D), "offsets[-1]"),          # more rows than the branches hold
    (call_replay_fwd, "k_r", t(T - 1, HKV, D), "k_r has shape"),
    (call_replay_fwd, "v_p", t(P + 3, HKV, D), "v_p has shape"),
    (call_replay_fwd, "k_p", t(P, 3, D), "not a multiple"),
    (call_replay_fwd, "v_r", t(T, HKV, D, dtype=torch.float32), "v_r has dtype"),   # bf16 / fp32 mix
    (call_replay_fwd, "k_p", t(P, HKV, 2 * D), "head_dim"),
    (call_replay_bwd, "lse_r", t(HQ, T, dtype=bf), "lse_r has dtype"),
    (call_replay_bwd, "lse_r", t(HQ, T + 1, dtype=torch.float32), "lse_r has shape"),
    (call_replay_bwd, "do_r", t(T, HQ, D - 1), "do_r has shape"),
    (call_replay_bwd, "o_r", t(T, HQ, D, dtype=torch.float16), "o_r has dtype"),
    (call_prefill_fwd, "k_p", t(P - 1, HKV, D), "k_p has shape"),
    (call_prefill_fwd, "q_p", t(P, HQ, D, dtype=torch.float16), "unsupported dtype"),
    (call_prefill_bwd, "lse_p", t(HQ, P - 1, dtype=torch.float32), "lse_p has shape"),
    (call_prefill_bwd, "do_p", t(P, HQ, D, dtype=torch.float32), "do_p has dtype"),
])
def test_wrappers_reject_mismatched_tensors(call, name, bad, needle):
    x = good()
    x[name] = bad
    with pytest.raises(ValueError, match=None) as e:
        call(x)
    assert needle in str(e.value), str(e.value)


def test_offsets_must_match_the_branch_rows():
    x = good()
    with pytest.raises(ValueError, match="offsets"):
        call_replay_fwd(x, off=[0, 7, 19])
    with pytest.raises(ValueError, match="increase strictly"):
        call_replay_bwd(x, off=[0, 7, 7, 20])


def test_prefill_bwd_accumulators_checked():
    x = good()
    acc = (t(P, HKV, D, dtype=torch.float32), t(P, HKV, D, dtype=bf))
    with pytest.raises(ValueError, match="dv_p_acc has dtype"):
        call_prefill_bwd(x, acc=acc)
    with pytest.raises(ValueError, match="both"):
        call_prefill_bwd(x, acc=(t(P, HKV, D, dtype=torch.float32), None))


def test_well_formed_cpu_tensors_fail_only_on_the_device_check():
    x = good()
    for call in (call_replay_fwd, call_replay_bwd, call_prefill_fwd, call_prefill_bwd):
        with pytest.raises(ValueError, match="GPU tensor"):
            call(x)


def test_tree_single_steps_check_shapes():
    tr = ops.Tree.__new__(ops.Tree)  # sizes only; no library call
    tr.P, tr.Hq, tr.Hkv, tr.D, tr.offsets, tr.T = P, HQ, HKV, D, OFF, T
    tr.dtype, tr.device = bf, torch.device("cpu")
    x = good()
    with pytest.raises(ValueError, match="o_part has shape"):
        tr.check(q_r=x["q_r"], o_part=t(T - 1, HQ, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="dk_acc has dtype"):
        tr.check(dk_acc=t(P, HKV, D))
    with pytest.raises(ValueError, match="rowdot_p has shape"):
        tr.check(rowdot_p=t(HQ, T, dtype=torch.float32))
    with pytest.raises(ValueError, match="must be on"):
        tr.check(q_r=x["q_r"])
    with pytest.raises(ValueError, match="key range"):
        ops._check_range(tr, 5, 5)
    with pytest.raises(ValueError, match="key range"):
        ops._check_range(tr, 0, P + 1)
