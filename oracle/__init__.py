"""fp64 CPU oracle for shifted-window multi-head self-attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The HIP library never imports, links or calls anything here, and this package
includes nothing from the HIP library.

Two formulations, written separately and required to agree:
  * ``direct_forward`` (C, OpenMP): per real query, enumerate its key set
    directly from per-axis segments; usable at full size on selected queries;
  * ``literal_forward`` (numpy): pad, roll, partition, masked window
    attention, reverse; for small grids.

``literal_lse`` (numpy) gives each query's log-sum-exp of its visible logits
(the softmax's normaliser, which a forward pass can keep for the backward).
``literal_backward`` (numpy) gives the gradients of the literal form, window
by window, for all windows or a chosen subset.  ``layer_forward`` (numpy) adds
the query/key/value and output projections of a Swin block around the
direct form.
"""
from .direct import check, default_scale, direct_forward, local_coord, visible
from .backward import literal_backward, token_windows, window_tokens
from .layer import layer_forward, linear
from .literal import (literal_bias, literal_forward, literal_lse, literal_unwindows, literal_visibility,
                      literal_windows, pad_flags)

__all__ = [
    "check", "default_scale", "direct_forward", "local_coord", "visible",
    "literal_bias", "literal_forward", "literal_lse", "literal_unwindows", "literal_visibility",
    "literal_windows", "pad_flags", "literal_backward", "token_windows", "window_tokens",
    "layer_forward", "linear",
]
