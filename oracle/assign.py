"""Plain CPU oracle of the planner's replay-unit assignment (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the library never calls it and
shares no code with it.

"Splitting Prompt Prefill from Response Replay ...", §3.4 (replay units and grid
assignment): U replay units with work estimates w_k are placed on b rounds x s lanes so as to
minimise  sum over rounds tau of max over lanes j of (sum of w_k placed in cell (tau, j)).
Reading: every cell holds at least one unit (the planner drops candidates with empty lanes;
with empty cells allowed one round would always be optimal). The exact solution is written
here as brute force over every assignment; the large-U rule ("largest-first greedy
balancing") is restated step by step with the tie-breaks the library documents.
"""
from __future__ import annotations

import itertools
from typing import List, Sequence, Tuple

__all__ = ["grid_cost", "brute_force_assign", "greedy_assign"]


def grid_cost(w: Sequence[float], cells: Sequence[int], rounds: int, lanes: int) -> float:
    """The objective of an assignment: sum over rounds of the largest lane load."""
    load = [0.0] * (rounds * lanes)
    for k, c in enumerate(cells):
        load[c] += w[k]
    return sum(max(load[r * lanes:(r + 1) * lanes]) for r in range(rounds))


def brute_force_assign(w: Sequence[float], rounds: int, lanes: int) -> Tuple[float, List[int]]:
    """Least objective over every assignment that leaves no cell empty (tiny U only)."""
    ncell = rounds * lanes
    best, arg = float("inf"), None
    for cells in itertools.product(range(ncell), repeat=len(w)):
        if len(set(cells)) != ncell:
            continue
        c = grid_cost(w, cells, rounds, lanes)
        if c < best:
            best, arg = c, list(cells)
    return best, arg


def greedy_assign(w: Sequence[float], rounds: int, lanes: int) -> Tuple[float, List[int]]:
    """Largest-first greedy: units by decreasing weight (equal weights: lower index first);
    while some cell is empty, a unit may only go to an empty cell; it goes to the allowed cell
    whose use raises the objective least, equal rises going to the less loaded cell and then
    to the lower cell index."""
    ncell = rounds * lanes
    order = sorted(range(len(w)), key=lambda k: (-w[k], k))
    load = [0.0] * ncell
    count = [0] * ncell
    rmax = [0.0] * rounds
    cells = [0] * len(w)
    for k in order:
        empty_left = any(n == 0 for n in count)
        best = None
        for c in range(ncell):
            if empty_left and count[c] != 0:
                continue
            r = c // lanes
            rise = max(rmax[r], load[c] + w[k]) - rmax[r]
            key = (rise, load[c], c)
            if best is None or key < best[0]:
                best = (key, c)
        c = best[1]
        cells[k] = c
        count[c] += 1
        load[c] += w[k]
        rmax[c // lanes] = max(rmax[c // lanes], load[c])
    return sum(rmax), cells
