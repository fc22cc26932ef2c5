"""CPU oracle for the WAITS prefill KV-selection path (score -> select -> compact).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in
this package.  The GPU library and its Python binding never touch it, and it
shares no code, constants or helpers with them.

* ``waits_oracle`` -- the plain definition in float64 numpy (library matmul,
  exp and sort as steps; nothing blocked, fused or reordered beyond splitting
  query rows into chunks, which does not change any sum's terms).
* ``brute`` -- the same definition in scalar pure-Python loops with
  ``math.fsum``, for tiny inputs only; it pins the numpy oracle.

Pins (see ``tests/test_oracle.py``): closed forms for uniform attention
(harmonic numbers), the H2O / TOVA / SnapKV limits checked against
``scipy.special.softmax``, the attention-mass invariant, causal support
invariance, GQA head-permutation invariance, brute force on N <= 64, and a
full lexicographic sort for top-k.  No function here is "parity unpinned".
"""
from .waits_oracle import (  # noqa: F401
    sigmoid_weights,
    live_rows,
    head_scores,
    waits_scores,
    waits_lse,
    select_topk,
    waits_select,
    waits_compact,
)
