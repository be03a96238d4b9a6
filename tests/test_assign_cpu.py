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


# ---- pins of the greedy restatement, independent of the library ----

def test_greedy_one_unit_per_cell_closed_form():
    # U = rounds x lanes: while cells are empty every unit takes an empty cell; the k-th largest
    # unit then joins round k // lanes (a round already holding a larger unit costs nothing more),
    # so the cost is the sum of each consecutive group's first (largest) weight, which is also the
    # optimum for groups of equal size (sorted consecutive grouping minimises the sum of maxima).
    rng = random.Random(11)
    for _ in range(25):
        rounds, lanes = rng.randint(1, 4), rng.randint(1, 5)
        n = rounds * lanes
        w = [float(rng.randint(0, 30)) for _ in range(n)]
        cost, cells = greedy_assign(w, rounds, lanes)
        order = sorted(range(n), key=lambda k: (-w[k], k))
        ws = [w[k] for k in order]
        assert cost == sum(ws[r * lanes] for r in range(rounds))
        assert [cells[k] for k in order] == list(range(n))
        if n <= 6:
            assert cost == brute_force_assign(w, rounds, lanes)[0]


def test_greedy_one_lane_per_round_costs_the_total():
    # one lane per round: every round's max is its only load, so any assignment costs sum(w)
    rng = random.Random(12)
    for _ in range(20):
        rounds = rng.randint(1, 6)
        w = [rng.uniform(0, 9) for _ in range(rng.randint(rounds, 20))]
        cost, cells = greedy_assign(w, rounds, 1)
        assert abs(cost - sum(w)) <= 1e-12 * sum(w)
        assert sorted(set(cells)) == list(range(rounds))


def lpt(w, m):
    """Largest processing time first (Graham's list scheduling of jobs sorted by decreasing
    length): each job goes to the machine with the least load, ties to the lower index."""
    load = [0.0] * m
    cells = [0] * len(w)
    for k in sorted(range(len(w)), key=lambda k: (-w[k], k)):
        j = min(range(m), key=lambda j: (load[j], j))
        cells[k] = j
        load[j] += w[k]
    return max(load), cells


def test_greedy_single_round_is_lpt_scheduling():
    # One round of s lanes: the objective is the largest lane load (the makespan) and the
    # greedy rule reduces to LPT list scheduling.
    rng = random.Random(13)
    for _ in range(40):
        lanes = rng.randint(1, 7)
        w = [float(rng.randint(1, 40)) for _ in range(rng.randint(lanes, 40))]
        assert greedy_assign(w, 1, lanes) == lpt(w, lanes)
    # Graham's worst case of LPT (R. L. Graham, "Bounds on multiprocessing timing anomalies",
    # SIAM J. Appl. Math. 17, 1969): on m machines, jobs 2m-1, 2m-1, 2m-2, 2m-2, ..., m+1, m+1,
    # m, m, m give LPT makespan 4m - 1 against the optimum 3m.
    for m in (2, 3, 4):
        w = [float(x) for j in range(2 * m - 1, m, -1) for x in (j, j)] + [float(m)] * 3
        cost, _ = greedy_assign(w, 1, m)
        assert cost == 4 * m - 1
        if len(w) <= 7:
            assert brute_force_assign(w, 1, m)[0] == 3 * m


def test_greedy_hand_traced_grid():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_greedy_2x2.json")))
    cost, cells = greedy_assign(g["weights"], g["rounds"], g["lanes"])
    assert cells == g["cells"] and cost == g["cost"]
    lib_cells, lib_cost = assign_units(g["weights"], g["rounds"], g["lanes"], exact_max=0)
    assert lib_cells == g["cells"] and lib_cost == g["cost"]
    assert brute_force_assign(g["weights"], g["rounds"], g["lanes"])[0] == g["cost"]


def test_greedy_pins_catch_a_wrong_tie_break():
    # The pins must reject a plausible misreading: sending ties on the rise to the lower
    # index (instead of the less loaded cell) changes the hand-traced grid's last step.
    def greedy_lower_index(w, rounds, lanes):
        ncell = rounds * lanes
        load, count, rmax = [0.0] * ncell, [0] * ncell, [0.0] * rounds
        cells = [0] * len(w)
        for k in sorted(range(len(w)), key=lambda k: (-w[k], k)):
            empty = any(n == 0 for n in count)
            c = min((c for c in range(ncell) if not (empty and count[c])),
                    key=lambda c: (max(rmax[c // lanes], load[c] + w[k]) - rmax[c // lanes], c))
            cells[k] = c
            count[c] += 1
            load[c] += w[k]
            rmax[c // lanes] = max(rmax[c // lanes], load[c])
        return sum(rmax), cells
    assert greedy_lower_index([6.0, 5.0, 4.0, 2.0, 1.0], 2, 2)[1] != [0, 1, 2, 3, 3]
