"""fp64 CPU oracle for exact softmax attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table
or constant generator with the HIP library; both sides are fed from the
``workloads`` input generators only.

It computes the plain definition of attention (scores, mask, softmax,
dropout, weighted sum of values) with every N x N matrix materialized in
float64, one (batch, head) slice at a time; the tiled method on the pages
reaches this same result, so the definition is the oracle.

Parity status of each function (see the pins in ``tests/test_oracle_*.py``):

* ``forward_head`` / ``forward``: pinned (brute force at 50 digits, closed
  forms, invariants, torch SDPA in fp64).
* ``backward_head`` / ``backward``: pinned (central finite differences,
  torch autograd in fp64, identities).
* ``backward_rows`` (dQ of selected rows) and ``backward_cols`` (dK, dV of
  selected keys): pinned by central finite differences with respect to those
  rows of Q, K and V.
* ``dropout_keep``: pinned for the mixing function by the published
  MurmurHash3 test vectors; the chaining of (seed, b, h, i, j) is this
  library's own definition ("parity unpinned" beyond that definition and the
  statistical checks).
"""
from .dropout_hash import fmix32, head_key, dropout_threshold, dropout_keep  # noqa: F401
from .attention import (  # noqa: F401
    valid_mask,
    forward_head,
    backward_head,
    forward,
    backward,
    forward_rows,
    backward_rows,
    backward_cols,
)
