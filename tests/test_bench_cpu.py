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
