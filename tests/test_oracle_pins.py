"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test would fail for a plausible mistake somewhere in the oracle: a wrong mask index
(closed forms with Q = 0, one-hot values), a dropped or mis-signed term of the backward
(finite differences, library attention under the tree mask), a transposed operand
(library attention, finite differences), wrong prompt-gradient aggregation (sum rules,
hand-derived golden values, split independence).
"""
import json
import math
import os

import pytest
import torch

from oracle import (branch_response_grads, flattened_sampled_rows, flattened_tree_attention,
                    prompt_key_grads, rows_attention)
from tests.tree_reference import tree_attention
from workloads import make_inputs, make_shape

HERE = os.path.dirname(os.path.abspath(__file__))
f64 = torch.float64
KEYS = ["o_p", "lse_p", "o_r", "lse_r"]
GKEYS = ["dq_p", "dk_p", "dv_p", "dq_r", "dk_r", "dv_r"]


def _inputs(P, lens, Hq, Hkv, D, seed, std=1.0):
    """Seeded fp32 draw, held in fp64 so that edits made by a test are exact."""
    w = make_inputs(make_shape(P, lens, Hq, Hkv, D, dtype="f32", std=std), seed=seed)
    for name in ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r"]:
        setattr(w, name, getattr(w, name).to(f64))
    return w


def _run(w, **kw):
    return flattened_tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets,
                                    do_p=w.do_p, do_r=w.do_r, **kw)


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log}))


def test_golden_hand_derived_tree():
    g = json.load(open(os.path.join(HERE, "golden", "hand_tiny_tree.json")))
    inp = {k: torch.tensor([_ev(x) for x in v], dtype=f64).view(-1, 1, 1) for k, v in g["inputs"].items()}
    off = [0]
    for r in g["shape"]["lens"]:
        off.append(off[-1] + r)
    out = flattened_tree_attention(inp["q_p"], inp["k_p"], inp["v_p"], inp["q_r"], inp["k_r"],
                                   inp["v_r"], off, scale=g["shape"]["scale"],
                                   do_p=inp["do_p"], do_r=inp["do_r"])
    for name, exprs in g["expected"].items():
        exp = torch.tensor([_ev(x) for x in exprs], dtype=f64)
        got = out[name].flatten()
        assert torch.allclose(got, exp, atol=1e-12, rtol=0), (name, got, exp)


@pytest.mark.parametrize("P,lens,Hq,Hkv,D,seed", [
    (1, [1], 1, 1, 8, 1),
    (2, [1, 2], 2, 1, 8, 2),
    (3, [5, 1, 2], 4, 2, 8, 3),
    (17, [33, 2, 5, 1, 9], 4, 1, 8, 4),
    (64, [33, 5], 2, 2, 64, 5),
    (17, [1, 1, 1], 8, 2, 16, 6),
])
def test_oracle_matches_library_tree_attention(P, lens, Hq, Hkv, D, seed):
    w = _inputs(P, lens, Hq, Hkv, D, seed)
    out = _run(w, slab=7)
    ref = tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets,
                         do_p=w.do_p, do_r=w.do_r)
    for key in KEYS + GKEYS:
        assert torch.allclose(out[key], ref[key], atol=1e-11, rtol=1e-11), key
    assert float(out["prompt_copy_spread"]) < 1e-12


def test_single_branch_is_plain_causal_attention():
    # G = 1: the tree is one linear sequence, so the library's is_causal path applies.
    w = _inputs(13, [11], 2, 2, 8, 11)
    out = _run(w)
    q = torch.cat([w.q_p, w.q_r]).to(f64).transpose(0, 1)
    k = torch.cat([w.k_p, w.k_r]).to(f64).transpose(0, 1)
    v = torch.cat([w.v_p, w.v_r]).to(f64).transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1)
    assert torch.allclose(out["o_p"], o[:13], atol=1e-12)
    assert torch.allclose(out["o_r"], o[13:], atol=1e-12)


def test_zero_queries_closed_form():
    # Q = 0: every visible logit is 0, so LSE = ln(n) and O = mean of the visible V rows,
    # with n = r + 1 for prompt row r and n = P + t + 1 for branch row t.
    P, lens = 5, [3, 1, 4]
    w = _inputs(P, lens, 2, 1, 8, 21)
    w.q_p.zero_()
    w.q_r.zero_()
    out = _run(w)
    off = [0, 3, 4, 8]
    for h in range(2):
        for r in range(P):
            assert abs(float(out["lse_p"][h, r]) - math.log(r + 1)) < 1e-13
            assert torch.allclose(out["o_p"][r, h], w.v_p[:r + 1, 0].to(f64).mean(0), atol=1e-13)
        for i in range(3):
            for t in range(off[i + 1] - off[i]):
                row = off[i] + t
                vis = torch.cat([w.v_p[:, 0], w.v_r[off[i]:row + 1, 0]]).to(f64)
                assert abs(float(out["lse_r"][h, row]) - math.log(P + t + 1)) < 1e-13
                assert torch.allclose(out["o_r"][row, h], vis.mean(0), atol=1e-13)


def test_one_hot_values_expose_the_tree_mask():
    # Q = 0 and V = identity over the packed tokens: O[r, j] = 1/n_r exactly on the keys
    # token r may see (whole prompt prefix / own branch prefix), 0 elsewhere.
    P, lens = 3, [2, 3]
    N = P + sum(lens)
    w = _inputs(P, lens, 1, 1, N, 22)
    w.q_p.zero_()
    w.q_r.zero_()
    eye = torch.eye(N, dtype=f64)
    w.v_p.copy_(eye[:P, None, :])
    w.v_r.copy_(eye[P:, None, :])
    out = _run(w)
    expected_p = torch.tensor([[1, 0, 0, 0, 0, 0, 0, 0], [1, 1, 0, 0, 0, 0, 0, 0],
                               [1, 1, 1, 0, 0, 0, 0, 0]], dtype=f64)
    expected_r = torch.tensor([[1, 1, 1, 1, 0, 0, 0, 0], [1, 1, 1, 1, 1, 0, 0, 0],
                               [1, 1, 1, 0, 0, 1, 0, 0], [1, 1, 1, 0, 0, 1, 1, 0],
                               [1, 1, 1, 0, 0, 1, 1, 1]], dtype=f64)
    expected_p /= expected_p.sum(1, keepdim=True)
    expected_r /= expected_r.sum(1, keepdim=True)
    assert torch.allclose(out["o_p"][:, 0], expected_p, atol=1e-14)
    assert torch.allclose(out["o_r"][:, 0], expected_r, atol=1e-14)


@pytest.mark.parametrize("name", ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r"])
def test_gradients_match_central_finite_differences(name):
    P, lens, Hq, Hkv, D = 4, [3, 2], 4, 2, 4
    w = _inputs(P, lens, Hq, Hkv, D, 31)
    args = {k: getattr(w, k).to(f64) for k in ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r"]}
    do_p, do_r = w.do_p.to(f64), w.do_r.to(f64)

    def loss(a):
        o = flattened_tree_attention(a["q_p"], a["k_p"], a["v_p"], a["q_r"], a["k_r"], a["v_r"],
                                     w.offsets)
        return float((o["o_p"] * do_p).sum() + (o["o_r"] * do_r).sum())

    grads = flattened_tree_attention(args["q_p"], args["k_p"], args["v_p"], args["q_r"], args["k_r"],
                                     args["v_r"], w.offsets, do_p=do_p, do_r=do_r)
    gname = "d" + name
    gen = torch.Generator().manual_seed(7)
    for _ in range(3):
        u = torch.randn(args[name].shape, generator=gen, dtype=f64)
        h = 1e-5
        ap = dict(args)
        am = dict(args)
        ap[name] = args[name] + h * u
        am[name] = args[name] - h * u
        fd = (loss(ap) - loss(am)) / (2 * h)
        an = float((grads[gname] * u).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (gname, fd, an)


def test_shift_rules():
    P, lens, Hq, Hkv, D = 6, [4, 7, 1], 4, 2, 8
    w = _inputs(P, lens, Hq, Hkv, D, 41)
    base = _run(w)
    scale = 1.0 / math.sqrt(D)
    c = torch.randn(Hkv, D, generator=torch.Generator().manual_seed(3), dtype=f64)
    # Adding one vector to every key of a kv head shifts each row's logits by a constant:
    # probabilities, O, dQ and dK stay, LSE moves by scale * q.c.
    wk = _inputs(P, lens, Hq, Hkv, D, 41)
    wk.k_p += c
    wk.k_r += c
    sk = _run(wk)
    grp = Hq // Hkv
    cq = c.repeat_interleave(grp, dim=0).to(f64)
    for key in ["o_p", "o_r", "dq_p", "dq_r", "dk_p", "dk_r", "dv_p", "dv_r"]:
        assert torch.allclose(sk[key], base[key], atol=1e-10), key
    assert torch.allclose(sk["lse_p"], base["lse_p"] + scale * torch.einsum("rhd,hd->hr", w.q_p.to(f64), cq), atol=1e-10)
    assert torch.allclose(sk["lse_r"], base["lse_r"] + scale * torch.einsum("rhd,hd->hr", w.q_r.to(f64), cq), atol=1e-10)
    # Adding one vector to every value: O moves by it, gradients stay.
    wv = _inputs(P, lens, Hq, Hkv, D, 41)
    wv.v_p += c
    wv.v_r += c
    sv = _run(wv)
    assert torch.allclose(sv["o_p"], base["o_p"] + cq[None], atol=1e-10)
    assert torch.allclose(sv["o_r"], base["o_r"] + cq[None], atol=1e-10)
    for key in GKEYS:
        assert torch.allclose(sv[key], base[key], atol=1e-10), key


def test_sum_rules():
    # Per kv head, over all keys: sum dV = sum of the group's upstream gradients over all
    # rows (each row's probabilities sum to 1); sum dK = 0 (each row's dS sums to 0).
    P, lens, Hq, Hkv, D = 9, [5, 3, 8, 2], 8, 2, 8
    w = _inputs(P, lens, Hq, Hkv, D, 51)
    out = _run(w)
    grp = Hq // Hkv
    for g in range(Hkv):
        sdv = out["dv_p"][:, g].sum(0) + out["dv_r"][:, g].sum(0)
        sdo = (w.do_p[:, g * grp:(g + 1) * grp].to(f64).sum((0, 1))
               + w.do_r[:, g * grp:(g + 1) * grp].to(f64).sum((0, 1)))
        assert torch.allclose(sdv, sdo, atol=1e-11)
        sdk = out["dk_p"][:, g].sum(0) + out["dk_r"][:, g].sum(0)
        assert sdk.abs().max() < 1e-11


def test_branch_permutation():
    P, lens, Hq, Hkv, D = 7, [3, 6, 2], 2, 1, 8
    w = _inputs(P, lens, Hq, Hkv, D, 61)
    base = _run(w)
    perm = [2, 0, 1]
    off = [0, 3, 9, 11]
    idx = torch.cat([torch.arange(off[i], off[i + 1]) for i in perm])
    wp = _inputs(P, lens, Hq, Hkv, D, 61)
    for name in ["q_r", "k_r", "v_r", "do_r"]:
        setattr(wp, name, getattr(w, name)[idx].clone())
    wp.offsets = torch.tensor([0, 2, 5, 11], dtype=torch.int32)
    pm = _run(wp)
    for key in ["o_p", "lse_p", "dq_p", "dk_p", "dv_p"]:
        assert torch.allclose(pm[key], base[key], atol=1e-12), key
    for key in ["o_r", "dq_r", "dk_r", "dv_r"]:
        assert torch.allclose(pm[key], base[key][idx], atol=1e-12), key
    assert torch.allclose(pm["lse_r"], base["lse_r"][:, idx], atol=1e-12)


def test_slab_size_and_prompt_gradient_split_do_not_matter():
    P, lens, Hq, Hkv, D = 20, [9, 4, 13], 4, 2, 8
    w = _inputs(P, lens, Hq, Hkv, D, 71)
    a = _run(w, slab=3)
    b = _run(w, slab=1024)
    c = _run(w, prompt_grad_weights=[1.0, 0.0, 0.0])
    for key in KEYS + GKEYS:
        assert torch.allclose(a[key], b[key], atol=1e-12), key
        assert torch.allclose(a[key], c[key], atol=1e-12), key


def test_kv_head_selection_matches_full():
    P, lens, Hq, Hkv, D = 10, [4, 6], 8, 4, 8
    w = _inputs(P, lens, Hq, Hkv, D, 81)
    full = _run(w)
    sel = _run(w, kv_heads=[2])
    qh = [4, 5]
    for key in ["o_p", "o_r", "dq_p", "dq_r"]:
        assert torch.allclose(sel[key], full[key][:, qh], atol=1e-13), key
    for key in ["lse_p", "lse_r"]:
        assert torch.allclose(sel[key], full[key][qh], atol=1e-13), key
    for key in ["dk_p", "dv_p", "dk_r", "dv_r"]:
        assert torch.allclose(sel[key], full[key][:, [2]], atol=1e-13), key


def test_sampled_rows_match_library_tree_attention():
    P, lens, Hq, Hkv, D = 12, [5, 9, 1], 4, 2, 8
    w = _inputs(P, lens, Hq, Hkv, D, 91)
    ref = tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, do_p=w.do_p, do_r=w.do_r)
    prow, rrow = [0, 5, 11], [0, 4, 5, 13, 14]
    s = flattened_sampled_rows(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, prow, rrow,
                               do_p=w.do_p, do_r=w.do_r)
    assert torch.allclose(s["o_p"], ref["o_p"][prow], atol=1e-12)
    assert torch.allclose(s["lse_p"], ref["lse_p"][:, prow], atol=1e-12)
    assert torch.allclose(s["dq_p"], ref["dq_p"][prow], atol=1e-12)
    assert torch.allclose(s["o_r"], ref["o_r"][rrow], atol=1e-12)
    assert torch.allclose(s["lse_r"], ref["lse_r"][:, rrow], atol=1e-12)
    assert torch.allclose(s["dq_r"], ref["dq_r"][rrow], atol=1e-12)


def test_branch_response_grads_match_library_tree_attention():
    P, lens, Hq, Hkv, D = 11, [6, 9, 3], 4, 2, 8
    w = _inputs(P, lens, Hq, Hkv, D, 101)
    ref = tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, do_p=w.do_p, do_r=w.do_r)
    b = branch_response_grads(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, 1, w.do_r,
                              kv_heads=[1], slab=4)
    rows = slice(6, 15)
    assert torch.allclose(b["dk_r"], ref["dk_r"][rows][:, [1]], atol=1e-12)
    assert torch.allclose(b["dv_r"], ref["dv_r"][rows][:, [1]], atol=1e-12)
    assert torch.allclose(b["dq_r"], ref["dq_r"][rows][:, [2, 3]], atol=1e-12)
    assert torch.allclose(b["o_r"], ref["o_r"][rows][:, [2, 3]], atol=1e-12)


@pytest.mark.parametrize("P,lens,Hq,Hkv,D,kv,keys,slab,seed", [
    (13, [5, 9, 1], 4, 2, 8, [1], [0, 3, 7, 12], 4, 121),
    (20, [1, 30], 2, 2, 16, [0, 1], [19, 0, 1, 10], 3, 122),
    (9, [4, 4, 4, 4], 6, 2, 8, [1], list(range(9)), 256, 123),
    (33, [2, 40, 3], 8, 1, 8, [0], [0, 16, 31, 32], 5, 124),
])
def test_prompt_key_grads_match_library_tree_attention(P, lens, Hq, Hkv, D, kv, keys, slab, seed):
    # the selected prompt keys' total gradient (prompt rows + every branch, all query heads of
    # the group) equals the library attention routine's autograd gradient under the tree mask
    w = _inputs(P, lens, Hq, Hkv, D, seed)
    ref = tree_attention(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, do_p=w.do_p, do_r=w.do_r)
    g = prompt_key_grads(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, keys, w.do_p, w.do_r,
                         kv_heads=kv, slab=slab)
    J = sorted(set(keys))
    assert g["keys"].tolist() == J
    assert torch.allclose(g["dk_p"], ref["dk_p"][J][:, kv], atol=1e-12), (g["dk_p"] - ref["dk_p"][J][:, kv]).abs().max()
    assert torch.allclose(g["dv_p"], ref["dv_p"][J][:, kv], atol=1e-12)


def test_prompt_key_grads_detect_a_key_off_by_one():
    # a gradient of key j reported for key j+1 (a misrouted row) fails the comparison above:
    # neighbouring keys' gradients differ by far more than the tolerance
    w = _inputs(13, [5, 9, 1], 4, 2, 8, 121)
    g = prompt_key_grads(w.q_p, w.k_p, w.v_p, w.q_r, w.k_r, w.v_r, w.offsets, list(range(13)), w.do_p,
                         w.do_r, kv_heads=[0])
    assert float((g["dk_p"][1:] - g["dk_p"][:-1]).abs().amax(dim=(1, 2)).min()) > 1e-3
    assert float((g["dv_p"][1:] - g["dv_p"][:-1]).abs().amax(dim=(1, 2)).min()) > 1e-3


def test_rows_attention_single_visible_key():
    # One visible key: softmax weight 1, O = v_0, LSE = logit, dQ = 0 (dS = 0).
    q = torch.randn(3, 4, dtype=f64)
    k = torch.randn(5, 4, dtype=f64)
    v = torch.randn(5, 4, dtype=f64)
    do = torch.randn(3, 4, dtype=f64)
    o, lse, dq, dk, dv = rows_attention(q, k, v, torch.ones(3, dtype=torch.long), 0.5, do)
    assert torch.allclose(o, v[0].expand(3, 4), atol=1e-15)
    assert torch.allclose(lse, 0.5 * q @ k[0], atol=1e-15)
    assert dq.abs().max() < 1e-15 and dk.abs().max() < 1e-15
    assert torch.allclose(dv[0], do.sum(0), atol=1e-14) and dv[1:].abs().max() == 0


def test_generator_is_deterministic_and_follows_config_lengths():
    from workloads import config_shape
    a = make_inputs(make_shape(8, [3, 5], 2, 1, 16, dtype="bf16"), seed=5)
    b = make_inputs(make_shape(8, [3, 5], 2, 1, 16, dtype="bf16"), seed=5)
    for name in ["q_p", "k_p", "v_p", "q_r", "k_r", "v_r", "do_p", "do_r"]:
        assert torch.equal(getattr(a, name), getattr(b, name))
    s3 = config_shape(3)
    assert s3.G == 8 and all(512 <= r <= 2048 for r in s3.lens)
    assert config_shape(3) == s3


def test_sweep_trees_keep_the_token_budget_and_regimes():
    # Group-size sweep: G in {8, 16, 32, 64} at a per-step budget G (L_P + L_R) of 256k tokens
    # (in expectation; branch lengths are drawn around the target), 4:1 prompt:response; and
    # one response-heavy tree. All on 28 query / 4 key-value heads, head_dim 128, bf16.
    from workloads import SWEEPS, config_seed, config_shape, workload_name
    seen = set()
    for g in (8, 16, 32, 64):
        name = f"group_g{g}"
        s = config_shape(name)
        assert s.G == g and (s.Hq, s.Hkv, s.D, s.dtype) == (28, 4, 128, "bf16")
        budget = s.G * s.P + s.T
        assert abs(budget - 262144) < 0.05 * 262144, (name, budget)
        mean_r = s.T / s.G
        assert 3.0 < s.P / mean_r < 5.5, (name, s.P, mean_r)
        lo, hi = SWEEPS[name]["R"]
        assert all(lo <= r <= hi for r in s.lens)
        assert config_shape(name) == s
        assert workload_name(name).startswith(f"group_g{g}_b256k")
        seen.add(config_seed(name))
    s = config_shape("response_heavy")
    assert s.T / s.G > 3 * s.P
    seen.add(config_seed("response_heavy"))
    assert len(seen) == 5 and not seen & {config_seed(c) for c in range(1, 6)}
