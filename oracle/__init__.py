"""CPU oracle for the streaming KV-cache hot path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import anything from this package.  The product path (the HIP library
and its Python binding) never imports, links or calls it, and it imports
nothing from the product path.

Everything here is plain NumPy in float64, written from the pages' own
description of the method (see ``skv_oracle`` for the passage behind each
function).  The pages print no worked numerical example, so the values of
real-model attention are "parity unpinned" by the pages; the tests under
``tests/test_oracle_*.py`` pin every function instead against closed forms,
brute force, library routines and the configuration arithmetic the pages print.
"""
from .skv_oracle import (  # noqa: F401
    THETA_DEFAULT,
    rope_split,
    axis_frequencies,
    rope_3d,
    token_grid_positions,
    CacheList,
    visible_history,
    attention,
    cross_attention,
    block_causal_visible,
    block_causal_attention,
    StreamingOracle,
)
