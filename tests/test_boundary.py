"""The C ABI without a GPU: the library loads, exports every function that
include/swa.h declares, and rejects malformed arguments before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

from shifted_window_attention_cyclic_amd import binding
from shifted_window_attention_cyclic_amd.inputs import WORKLOADS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "swa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_\w+)\s*\(", text)))


def declared_arity():
    """Parameter count of every function the header declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(swa_\w+)\s*\(([^)]*)\)\s*;", text):
        params = params.strip()
        out[name] = 0 if params in ("", "void") else params.count(",") + 1
    return out


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("swa_create", "swa_forward", "swa_destroy"):
        assert n in names
    assert set(names) == set(binding.EXPORTS)


def test_binding_signatures_match_the_header(lib):
    arity = declared_arity()
    assert set(arity) == set(declared_functions())
    for name, n in arity.items():
        assert len(getattr(lib, name).argtypes) == n, name


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(5):
        assert lib.swa_status_string(s)
    assert lib.swa_status_string(99) == b"unknown status"


def test_null_handles(lib):
    assert lib.swa_destroy(None) == binding.SWA_OK
    assert lib.swa_forward(None, None, None, None, None, None, None) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_gather(None, None, None, None) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_scatter(None, None, None, None) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_debug_visibility(None, 0, None, None) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_get_info(None, None) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_backward(*([None] * 12)) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_backward_noalloc(*([None] * 11)) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_layer_forward(*([None] * 10)) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_layer_attention(*([None] * 7)) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_forward_lse(*([None] * 8)) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_backward_lse(*([None] * 14)) == binding.SWA_ERR_INVALID_ARGUMENT
    # NULL pointers, an unknown dtype and a bad shape are refused before any device call
    assert lib.swa_projection(binding.SWA_BF16, None, None, None, 1, 8, 32, 8, None, None, None,
                              None) == binding.SWA_ERR_INVALID_ARGUMENT
    assert lib.swa_projection(7, None, None, None, 1, 8, 32, 8, None, None, None,
                              None) == binding.SWA_ERR_INVALID_ARGUMENT
    buf = ctypes.create_string_buffer(4096 + 16)
    a = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16
    for rows, fout, fin, split in ((1, 8, 48, 8), (1, 12, 32, 12), (1, 4, 32, 4), (1, 32, 32, 8),
                                   (1 << 31, 8, 32, 8), (1, 1 << 16, 32, 1 << 15), (1, 8, 1 << 17, 8)):
        assert lib.swa_projection(binding.SWA_BF16, a, a, a, rows, fout, fin, split, a, a, a,
                                  None) == binding.SWA_ERR_UNSUPPORTED
    assert lib.swa_projection(binding.SWA_BF16, a, a, a, -1, 8, 32, 8, a, a, a,
                              None) == binding.SWA_ERR_INVALID_ARGUMENT
    # no rows: nothing to do, and no device needed
    assert lib.swa_projection(binding.SWA_F32, a, a, a, 0, 24, 32, 8, a, a, a, None) == binding.SWA_OK
    h = ctypes.c_void_p(1234)
    assert lib.swa_create(None, ctypes.byref(h)) == binding.SWA_ERR_INVALID_ARGUMENT
    assert h.value is None  # *out cleared on failure


def create_status(lib, problem, variant="fused"):
    cfg = binding.make_config(problem, variant)
    h = ctypes.c_void_p()
    st = lib.swa_create(ctypes.byref(cfg), ctypes.byref(h))
    if st == binding.SWA_OK:
        lib.swa_destroy(h)
    return st, lib.swa_last_error().decode()


BASE = WORKLOADS["c3_bf16_540x1080"]
BAD = [
    ("batch0", BASE.with_(batch=0), binding.SWA_ERR_INVALID_ARGUMENT),
    ("heads0", BASE.with_(heads=0), binding.SWA_ERR_INVALID_ARGUMENT),
    ("shift_eq_window", BASE.with_(shift=(0, 12, 6)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("negative_shift", BASE.with_(shift=(0, -1, 6)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("window_gt_extent", BASE.with_(window=(1, 600, 12)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("window0", BASE.with_(window=(1, 0, 12)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("not_divisible", BASE.with_(extent=(1, 545, 1080), padded=(1, 545, 1080)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("padded_below_extent", BASE.with_(padded=(1, 530, 1080)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("pad_on_cyclic_axis", BASE.with_(extent=(1, 540, 1070), padded=(1, 540, 1080)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("extent0", BASE.with_(extent=(0, 540, 1080)), binding.SWA_ERR_INVALID_ARGUMENT),
    ("head_dim48", BASE.with_(head_dim=48), binding.SWA_ERR_UNSUPPORTED),
    ("head_dim256", BASE.with_(head_dim=256), binding.SWA_ERR_UNSUPPORTED),
    ("head_dim128_f32", WORKLOADS["c1_f32_16x32"].with_(head_dim=128), binding.SWA_ERR_UNSUPPORTED),
    # N = 10800: its bias slice (179 x 239 floats) alone leaves no LDS for any schedule
    ("bf16_window_90x120", BASE.with_(window=(1, 90, 120), shift=(0, 45, 60)), binding.SWA_ERR_UNSUPPORTED),
    ("f32_window_27x27", WORKLOADS["c1_f32_16x32"].with_(extent=(1, 27, 27), padded=(1, 27, 27),
                                                          window=(1, 27, 27), shift=(0, 13, 13)),
     binding.SWA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,problem,status", BAD, ids=[b[0] for b in BAD])
def test_invalid_configs_rejected_before_hip(lib, name, problem, status):
    st, msg = create_status(lib, problem)
    assert st == status, (st, msg)
    assert msg


def test_bad_dtype_and_variant(lib):
    cfg = binding.make_config(BASE)
    cfg.dtype = 7
    h = ctypes.c_void_p()
    assert lib.swa_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.SWA_ERR_INVALID_ARGUMENT
    cfg = binding.make_config(BASE)
    cfg.variant = 5
    assert lib.swa_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.SWA_ERR_INVALID_ARGUMENT
    cfg = binding.make_config(BASE)
    cfg.cyclic[2] = 2
    assert lib.swa_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.SWA_ERR_INVALID_ARGUMENT
    cfg = binding.make_config(BASE)
    cfg.scale = float("nan")
    assert lib.swa_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.SWA_ERR_INVALID_ARGUMENT
    cfg.scale = -0.125
    assert lib.swa_create(ctypes.byref(cfg), ctypes.byref(h)) == binding.SWA_ERR_INVALID_ARGUMENT


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_valid_configs_need_a_device(lib, name):
    st, msg = create_status(lib, WORKLOADS[name])
    assert st == binding.SWA_ERR_HIP, msg


def test_binding_refuses_cpu_tensors():
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        binding._dev(t, "q")


# Every bf16 schedule packs source row + 1 of a token into the 28 low bits of a
# table word, so a bf16 problem with 2^28 - 1 or more token rows (real tokens,
# or window slots in the staged layout) is refused before any device call.
# 180x360 grids with one 32-wide head: 64,800 tokens per batch item.
ROW_LIMIT = (1 << 28) - 1
C2 = WORKLOADS["c2_bf16_180x360"]


@pytest.mark.parametrize("variant", ["fused", "staged"])
def test_bf16_row_word_limit_refused(lib, variant):
    p = C2.with_(batch=4200, heads=1)  # 272,160,000 tokens: past the 28-bit row word
    assert p.tokens >= ROW_LIMIT and p.window_tokens <= 512
    st, msg = create_status(lib, p, variant)
    assert st == binding.SWA_ERR_UNSUPPORTED, (st, msg)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_bf16_row_word_limit_just_below_is_valid(lib):
    p = C2.with_(batch=4100, heads=1)  # 265,680,000 tokens: inside the 28-bit row word
    assert p.tokens < ROW_LIMIT
    st, msg = create_status(lib, p)
    assert st == binding.SWA_ERR_HIP, (st, msg)  # valid: only the missing device stops it
