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
* ``fmix32``: pinned by the published MurmurHash3_x86_32 test vectors.
* ``mix32``: pinned to fmix32 by the identity mix32(x ^ (x >> 16)) == fmix32(x).
* ``head_key`` / ``row_words``: fmix32 chains, pinned against fmix32 composed
  step by step.
* ``dropout_keep`` / ``keep_halves``: the way (seed, b, h, i, j) are chained
  and split into 16-bit halves is this library's own definition ("parity
  unpinned" beyond that definition, the bijection it implies and the
  statistical checks).
"""
from .dropout_hash import fmix32, mix32, head_key, row_words, dropout_threshold, keep_halves, dropout_keep  # noqa: F401
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
