"""WAITS prefill KV selection (score -> top-k select -> compact) on AMD MI355X,
and decode attention over the compacted cache.

The computation runs in ``libwaits.so`` (hand-written HIP kernels for
gfx950, C ABI in ``include/waits.h``); ``waits`` is its Python binding.
"""
from . import waits  # noqa: F401
from .waits import (  # noqa: F401
    WaitsError,
    attention,
    colsum,
    compact,
    decode,
    lse,
    score,
    score_select_compact,
    select,
    select_compact,
)
