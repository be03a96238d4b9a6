"""Replay-unit assignment (augtree_assign_units, a host-only entry point) against its oracle.

Objective ("Splitting Prompt Prefill from Response Replay ...", §3.4): units with work
estimates on rounds x lanes, every cell non-empty, minimising the sum over rounds of the
largest lane load. The brute-force oracle is pinned by closed forms; the library's exact path
must reach the brute-force optimum, its greedy path must reproduce the oracle's restatement
of largest-first balancing step for step.
"""
import random
import time

import pytest

from oracle import brute_force_assign, greedy_assign, grid_cost
from shared_prefix_attention_prompt_amd import _lib
from shared_prefix_attention_prompt_amd.ops import assign_units


def test_brute_force_closed_forms():
    w = [5.0, 3.0, 2.0, 7.0]
    assert brute_force_assign(w, 1, 1)[0] == sum(w)          # one cell: everything
    assert brute_force_assign(w, 1, 4)[0] == max(w)          # one unit per lane
    assert brute_force_assign(w, 4, 1)[0] == sum(w)          # one unit per round
    assert brute_force_assign([4.0, 4.0], 1, 2)[0] == 4.0
    # two rounds of two lanes: the two largest share a round (7 + 3 = 10), not 7 + 5 = 12
    assert brute_force_assign(w, 2, 2)[0] == 10.0
    assert grid_cost([1.0, 2.0, 3.0], [0, 1, 1], 1, 2) == 5.0


@pytest.mark.parametrize("seed", range(40))
def test_exact_path_reaches_the_optimum(seed):
    rng = random.Random(seed)
    rounds, lanes = rng.choice([(1, 1), (1, 2), (2, 1), (1, 3), (3, 1), (2, 2), (1, 4), (2, 3), (3, 2)])
    cells_n = rounds * lanes
    n = rng.randint(cells_n, min(cells_n + 3, 7 if cells_n <= 3 else 6))
    if seed % 2:
        w = [float(rng.randint(0, 20)) for _ in range(n)]   # exact in binary: costs compare equal
    else:
        w = [rng.uniform(0.0, 10.0) for _ in range(n)]
    cells, cost = assign_units(w, rounds, lanes, exact_max=12)
    ref, _ = brute_force_assign(w, rounds, lanes)
    assert sorted(set(cells)) == list(range(rounds * lanes))      # every cell used
    assert abs(grid_cost(w, cells, rounds, lanes) - cost) <= 1e-12 * max(1.0, cost)
    assert abs(cost - ref) <= 1e-12 * max(1.0, ref), (w, rounds, lanes, cells, cost, ref)


@pytest.mark.parametrize("seed", range(20))
def test_greedy_path_follows_largest_first_balancing(seed):
    rng = random.Random(1000 + seed)
    rounds, lanes = rng.randint(1, 4), rng.randint(1, 8)
    n = rng.randint(rounds * lanes, 300)
    w = [float(rng.choice([rng.randint(1, 50), rng.randint(1, 5)])) if seed % 3 == 0 else rng.uniform(0, 100)
         for _ in range(n)]
    cells, cost = assign_units(w, rounds, lanes, exact_max=0)
    ref_cost, ref_cells = greedy_assign(w, rounds, lanes)
    assert cells == ref_cells
    assert cost == ref_cost


def test_greedy_is_never_better_than_exact():
    rng = random.Random(7)
    for _ in range(30):
        rounds, lanes = rng.randint(1, 2), rng.randint(1, 3)
        n = rng.randint(rounds * lanes, 9)
        w = [rng.uniform(0, 10) for _ in range(n)]
        _, exact = assign_units(w, rounds, lanes, exact_max=12)
        _, greedy = assign_units(w, rounds, lanes, exact_max=0)
        assert exact <= greedy + 1e-12 * greedy


@pytest.mark.parametrize("kw,needle", [
    (dict(weights=[1.0, 2.0], rounds=2, lanes=2), "fewer units than grid cells"),
    (dict(weights=[1.0, -1.0], rounds=1, lanes=1), "finite and >= 0"),
    (dict(weights=[1.0, float("nan")], rounds=1, lanes=1), "finite and >= 0"),
    (dict(weights=[1.0], rounds=0, lanes=1), ">= 1"),
    (dict(weights=[1.0], rounds=1, lanes=1, exact_max=17), "exact_max"),
])
def test_invalid_arguments_are_rejected(kw, needle):
    with pytest.raises(_lib.AugtreeError) as e:
        assign_units(**kw)
    assert e.value.status == _lib.AUGTREE_ERR_INVALID_ARGUMENT and needle in str(e.value)


def test_solve_time():
    # host solve time (the paper's planner figure is 0.018 ms at 16 blocks to 1.70 ms at 8192
    # blocks for its whole planner, §4.4 Fig. 15b); printed for the record, bounded loosely
    rng = random.Random(3)
    rows = []
    for n, rounds, lanes, exact in [(8, 2, 4, 12), (12, 2, 4, 12), (16, 2, 4, 16), (64, 2, 4, 12),
                                    (1024, 2, 8, 12), (8192, 4, 16, 12)]:
        w = [rng.uniform(1, 100) for _ in range(n)]
        t0 = time.perf_counter()
        assign_units(w, rounds, lanes, exact_max=exact)
        rows.append(f"U={n} {rounds}x{lanes} {'exact' if n <= exact else 'greedy'} "
                    f"{1e3 * (time.perf_counter() - t0):.3f} ms")
    print("; ".join(rows))
    assert all(float(r.split()[-2]) < 10_000 for r in rows)
