"""Exact shared-prefix attention (prompt prefill + response replay) on MI355X.

The kernels are hand-written HIP for gfx950 in ``csrc/``, built into ``libaugtree.so``
(C ABI: ``include/augtree.h``). ``_lib`` is the ctypes binding of that ABI, ``ops`` the
torch-facing wrappers and the autograd function. Importing this package does not load
the library; the first call does, and fails loudly if it has not been built.
"""
from .ops import (SharedPrefixAttention, prefill_bwd, prefill_fwd, replay_bwd,  # noqa: F401
                  replay_fwd, shared_prefix_attention)

__all__ = ["SharedPrefixAttention", "shared_prefix_attention", "prefill_fwd", "replay_fwd",
           "replay_bwd", "prefill_bwd"]
