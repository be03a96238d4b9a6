"""fp64 CPU oracle for exact shared-prefix attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import anything under ``oracle/``. The GPU library (``shared_prefix_attention_prompt_amd``)
never does, and the two share no code: only the seeded input generator in ``workloads``
feeds both.

Every function here is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``
(hand-derived golden values, closed forms, a library attention routine under an explicit
tree mask, finite differences, and invariants of the mathematics).
"""
from .flat_attention import (rows_attention, flattened_tree_attention,  # noqa: F401
                             flattened_sampled_rows, branch_response_grads, prompt_key_grads)
from .flat_chain import flattened_chain  # noqa: F401
from .assign import brute_force_assign, greedy_assign, grid_cost  # noqa: F401
