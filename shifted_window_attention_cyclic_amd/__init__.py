"""Shifted-window multi-head self-attention for MI355X (gfx950).

The computation lives in the HIP library ``libswa.so`` (C ABI in
``include/swa.h``); this package holds its sources, its build and a thin
ctypes binding with the same entry-point names.
"""
from .binding import (EXPORTS, SwaError, WindowAttention, load_library, make_config,
                      swa_backward, swa_backward_lse, swa_backward_noalloc, swa_create, swa_debug_visibility,
                      swa_destroy, swa_forward, swa_forward_lse, swa_gather,
                      swa_get_info, swa_layer_attention, swa_layer_forward, swa_projection, swa_scatter,
                      swa_status_string)

__all__ = [
    "EXPORTS", "SwaError", "WindowAttention", "load_library", "make_config", "swa_backward",
    "swa_backward_lse", "swa_backward_noalloc", "swa_create", "swa_forward_lse",
    "swa_debug_visibility", "swa_destroy", "swa_forward", "swa_gather", "swa_get_info",
    "swa_layer_attention", "swa_layer_forward", "swa_projection", "swa_scatter", "swa_status_string",
]
