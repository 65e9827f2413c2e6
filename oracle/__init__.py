"""CPU oracle (float64 NumPy) for causal softmax attention (and the same
attention under the full and sliding-window join predicates), the
Nadaraya-Watson control, the long-table <-> matrix adapter and the Q / K / V
input projections.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.  It shares
no code with the GPU path.

Parity pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``.  No function here is "parity unpinned".
"""
from .attention import (DEFAULT_SCALE, MASKS, backward, backward_head, forward, forward_head,
                        forward_head_relational, loss)
from .nw import nw_average
from . import projection, tables

__all__ = ["DEFAULT_SCALE", "MASKS", "forward", "forward_head", "forward_head_relational", "backward",
           "backward_head", "loss", "nw_average", "projection", "tables"]
