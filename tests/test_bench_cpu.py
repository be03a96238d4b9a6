"""CPU checks of bench.py's accounting and stream schedules (no GPU)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import SWEEPS, algorithmic_flops, config_shape, make_shape  # noqa: E402


@pytest.mark.parametrize("cfg", [1, 3, 4, 5] + sorted(SWEEPS))
def test_stage_flops_add_up_to_the_step(cfg):
    # forward 4*D per pair (F1-F3), backward 10*D per pair (8*D key-stationary + 2*D dQ)
    s = config_shape(cfg)
    assert sum(bench.stage_flops(s).values()) == algorithmic_flops(s)


def test_stage_bytes_per_row_and_head():
    s = make_shape(10, [3, 4], 4, 2, 128)
    b = bench.stage_bytes(s)
    assert b["merge"] == s.T * s.Hq * (2 * 4 * 128 + 2 * 4 + 2 * 128 + 4)
    assert b["row_dot_r"] == s.T * s.Hq * (2 * 2 * 128 + 4)
    assert b["row_dot_p"] == s.P * s.Hq * (2 * 2 * 128 + 4)


@pytest.mark.parametrize("nstreams", [1, 3])
@pytest.mark.parametrize("backward", [True, False])
def test_schedules_run_every_stage_once_after_its_inputs(nstreams, backward):
    stages = bench.STAGES if backward else bench.STAGES[:4]
    plan = bench.schedule(stages, nstreams)
    runs = [(si, n) for kind, si, n in plan if kind == "run"]
    assert sorted(n for _, n in runs) == sorted(stages)
    # producer of each stage's inputs (the path's data dependencies)
    needs = {"merge": ["replay_prompt_fwd", "replay_local_fwd"], "row_dot_r": ["merge"],
             "replay_prompt_bwd": ["row_dot_r"], "replay_local_bwd": ["row_dot_r"],
             "replay_dq": ["row_dot_r"], "row_dot_p": ["prefill_fwd"],
             "prefill_kv_bwd": ["row_dot_p", "replay_prompt_bwd"], "prefill_dq": ["row_dot_p"]}
    done = {}        # stage -> (stream, position in that stream's order)
    marks = {}       # mark -> set of stages complete when it fires
    seen = {i: set() for i in range(3)}  # stages complete on each stream at this point
    for kind, si, name in plan:
        if kind == "mark":
            marks[name] = set(seen[si])
        elif kind == "wait":
            assert name in marks, f"wait on {name} before it is recorded"
            seen[si] |= marks[name]
        else:
            for dep in needs.get(name, []):
                if dep in stages:
                    assert dep in seen[si], f"{name} on stream {si} may start before {dep}"
            seen[si].add(name)
            done[name] = si


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_stored_counters_only_for_their_sources_and_workload(monkeypatch):
    # the committed counter records carry the digest of the kernel sources they were taken on:
    # the bench reports them for that workload only, and not at all once a source changes
    from workloads import workload_name
    wl = workload_name(4)
    tr = bench.stored_traffic("replay_prompt_bwd", wl)
    mf = bench.stored_mfma("replay_prompt_bwd", wl)
    assert tr is not None and tr["bytes_per_launch"] > 0
    assert mf is not None and mf["issued_flops"] >= mf["algorithmic_flops"] > 0
    assert 0.0 < mf["busy"] <= 1.0
    assert bench.stored_traffic("replay_prompt_bwd", workload_name(5)) is None
    assert bench.stored_mfma("replay_prompt_bwd", "no such workload") is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.stored_traffic("replay_prompt_bwd", wl) is None
    assert bench.stored_mfma("replay_prompt_bwd", wl) is None


def test_stored_counter_records_match_their_summaries():
    # every figure in the JSON records appears in the committed markdown summary it names, so
    # the bench line and the readable summaries cannot drift apart
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for stage, r in rec["stages"].items():
        md = open(os.path.join(ROOT, "profiles", r["summary"])).read()
        assert f"| {r['fetch_kib']:.0f} | {r['write_kib']:.0f} | {r['bytes_per_launch'] / 1e9:.3f} |" in md, stage
    mf = json.load(open(os.path.join(ROOT, "profiles", "mfma.json")))
    for wl, w in mf["workloads"].items():
        md = open(os.path.join(ROOT, "profiles", f"mfma_{wl}.md")).read()
        for stage, r in w["stages"].items():
            assert f"| {r['counter_ms']:.3f} | {r['issued_flops'] / 1e12:.3f} | {r['algorithmic_flops'] / 1e12:.3f} |" in md, (wl, stage)
