"""CPU oracle for the WAITS prefill KV-selection path (score -> select -> compact),
for the prefill attention forward whose row normaliser WAITS pass 1 can reuse,
and for decode attention over the compacted cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in
this package.  The GPU library and its Python binding never touch it, and it
shares no code, constants or helpers with them.

* ``waits_oracle`` -- the plain definition in float64 numpy (library matmul,
  exp and sort as steps; nothing blocked, fused or reordered beyond splitting
  query rows into chunks, which does not change any sum's terms).
* ``attention_oracle`` -- causal prefill attention (output and row
  log-sum-exp), in float64 numpy.
* ``decode_oracle`` -- decode attention of one new query per head over the
  kept cache rows, in float64 numpy.
* ``brute`` -- the same definitions in scalar pure-Python loops with
  ``math.fsum``, for tiny inputs only; they pin the numpy oracles.

Pins (see ``tests/test_oracle.py``): closed forms for uniform attention
(harmonic numbers), the H2O / TOVA / SnapKV limits checked against
``scipy.special.softmax``, the attention-mass invariant, causal support
invariance, GQA head-permutation invariance, brute force on N <= 64, and a
full lexicographic sort for top-k; for decode (``tests/test_decode_oracle.py``)
closed forms (uniform, one and two rows), the prefill oracle's last causal row
(TOVA limit and lse), brute force, and softmax invariants; for prefill
attention (``tests/test_attention_oracle.py``) the WAITS row normaliser, the
running-mean closed form, rows 0 and N-1 (decode), brute force, causality
and the GQA map.  No function here
is "parity unpinned".
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
from .attention_oracle import prefill_attention  # noqa: F401
from .decode_oracle import waits_decode  # noqa: F401
