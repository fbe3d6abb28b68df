"""ctypes binding of libswa.so (include/swa.h), same entry-point names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity and passed as raw pointers with torch's current HIP stream.  Every
step of the computation runs in the library's kernels; there is no fallback.
If the library is missing, loading raises.
"""
import ctypes
import os

import torch

from .build import LIBRARY

SWA_OK, SWA_ERR_INVALID_ARGUMENT, SWA_ERR_UNSUPPORTED, SWA_ERR_OUT_OF_MEMORY, SWA_ERR_HIP = range(5)
SWA_F32, SWA_BF16 = 0, 1
SWA_VARIANT_FUSED, SWA_VARIANT_STAGED = 0, 1
SWA_SCHEDULE_AUTO, SWA_SCHEDULE_STREAM, SWA_SCHEDULE_BLOCK, SWA_SCHEDULE_KEYBLOCK = 0, 1, 2, 3
SCHEDULES = {"auto": SWA_SCHEDULE_AUTO, "stream": SWA_SCHEDULE_STREAM, "block": SWA_SCHEDULE_BLOCK,
             "keyblock": SWA_SCHEDULE_KEYBLOCK}
SWA_LAYER_AUTO, SWA_LAYER_FUSED, SWA_LAYER_UNFUSED = 0, 1, 2
LAYER_PATHS = {"auto": SWA_LAYER_AUTO, "fused": SWA_LAYER_FUSED, "unfused": SWA_LAYER_UNFUSED}

EXPORTS = ("swa_create", "swa_forward", "swa_forward_lse", "swa_backward", "swa_backward_lse",
           "swa_backward_noalloc", "swa_layer_forward",
           "swa_layer_attention", "swa_projection", "swa_destroy", "swa_get_info", "swa_status_string",
           "swa_last_error", "swa_gather", "swa_scatter", "swa_debug_visibility")


class swa_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int), ("heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("grid", ctypes.c_int * 3), ("padded", ctypes.c_int * 3), ("window", ctypes.c_int * 3),
        ("shift", ctypes.c_int * 3), ("cyclic", ctypes.c_int * 3),
        ("dtype", ctypes.c_int), ("scale", ctypes.c_float), ("variant", ctypes.c_int),
        ("schedule", ctypes.c_int), ("layer", ctypes.c_int),
    ]


class swa_info(ctypes.Structure):
    _fields_ = [
        ("windows", ctypes.c_int64), ("window_tokens", ctypes.c_int32), ("tokens", ctypes.c_int64),
        ("window_major_elems", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t),
        ("nominal_flops", ctypes.c_double), ("algorithmic_bytes", ctypes.c_double),
        ("schedule", ctypes.c_int32), ("workgroups", ctypes.c_int32),
        ("backward_workspace_bytes", ctypes.c_size_t), ("layer_workspace_bytes", ctypes.c_size_t),
        ("layer_flops", ctypes.c_double), ("backward_schedule", ctypes.c_int32),
        ("layer_path", ctypes.c_int32), ("backward_workgroups", ctypes.c_int32),
    ]


class SwaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: str = LIBRARY):
    """Loads libswa.so and declares its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, st = ctypes.c_void_p, ctypes.c_int
    lib.swa_create.argtypes = [ctypes.POINTER(swa_config), ctypes.POINTER(vp)]
    lib.swa_create.restype = st
    lib.swa_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.swa_forward.restype = st
    lib.swa_forward_lse.argtypes = [vp] * 8
    lib.swa_forward_lse.restype = st
    lib.swa_backward.argtypes = [vp] * 12
    lib.swa_backward.restype = st
    lib.swa_backward_lse.argtypes = [vp] * 14
    lib.swa_backward_lse.restype = st
    lib.swa_backward_noalloc.argtypes = [vp] * 11
    lib.swa_backward_noalloc.restype = st
    lib.swa_layer_forward.argtypes = [vp] * 10
    lib.swa_layer_forward.restype = st
    lib.swa_layer_attention.argtypes = [vp] * 7
    lib.swa_layer_attention.restype = st
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.swa_projection.argtypes = [st, vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.swa_projection.restype = st
    lib.swa_destroy.argtypes = [vp]
    lib.swa_destroy.restype = st
    lib.swa_get_info.argtypes = [vp, ctypes.POINTER(swa_info)]
    lib.swa_get_info.restype = st
    lib.swa_status_string.argtypes = [st]
    lib.swa_status_string.restype = ctypes.c_char_p
    lib.swa_last_error.argtypes = []
    lib.swa_last_error.restype = ctypes.c_char_p
    lib.swa_gather.argtypes = [vp, vp, vp, vp]
    lib.swa_gather.restype = st
    lib.swa_scatter.argtypes = [vp, vp, vp, vp]
    lib.swa_scatter.restype = st
    lib.swa_debug_visibility.argtypes = [vp, ctypes.c_int64, vp, vp]
    lib.swa_debug_visibility.restype = st
    _lib = lib
    return lib


def _check(status):
    if status != SWA_OK:
        lib = load_library()
        raise SwaError(status, f"{lib.swa_status_string(status).decode()}: "
                               f"{lib.swa_last_error().decode()}")


def make_config(problem, variant: str = "fused", schedule: str = "auto", layer: str = "auto") -> swa_config:
    """swa_config from a problem description (attributes batch, heads, head_dim,
    extent, padded, window, shift, cyclic, dtype ("f32"/"bf16"), scale)."""
    c = swa_config()
    c.batch, c.heads, c.head_dim = problem.batch, problem.heads, problem.head_dim
    for a in range(3):
        c.grid[a] = problem.extent[a]
        c.padded[a] = problem.padded[a]
        c.window[a] = problem.window[a]
        c.shift[a] = problem.shift[a]
        c.cyclic[a] = int(problem.cyclic[a])
    c.dtype = SWA_F32 if problem.dtype == "f32" else SWA_BF16
    c.scale = float(problem.scale or 0.0)
    c.variant = {"fused": SWA_VARIANT_FUSED, "staged": SWA_VARIANT_STAGED}[variant]
    c.schedule = SCHEDULES[schedule]
    c.layer = LAYER_PATHS[layer]
    return c


def swa_create(cfg: swa_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().swa_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def swa_destroy(handle) -> None:
    _check(load_library().swa_destroy(handle))


def swa_get_info(handle) -> swa_info:
    info = swa_info()
    _check(load_library().swa_get_info(handle, ctypes.byref(info)))
    return info


def swa_status_string(status: int) -> str:
    return load_library().swa_status_string(status).decode()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def swa_forward(handle, q, k, v, table, out, stream=None) -> None:
    dt = q.dtype
    _check(load_library().swa_forward(handle, _dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt),
                                      _dev(table, "table", torch.float32), _dev(out, "out", dt),
                                      _stream(stream)))


def swa_forward_lse(handle, q, k, v, table, out, lse, stream=None) -> None:
    dt = q.dtype
    _check(load_library().swa_forward_lse(handle, _dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt),
                                          _dev(table, "table", torch.float32), _dev(out, "out", dt),
                                          _dev(lse, "lse", torch.float32), _stream(stream)))


def swa_backward_lse(handle, q, k, v, table, out, lse, dout, dq, dk, dv, dtable, workspace, stream=None) -> None:
    dt = q.dtype
    _check(load_library().swa_backward_lse(handle, _dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt),
                                           _dev(table, "table", torch.float32), _dev(out, "out", dt),
                                           _dev(lse, "lse", torch.float32), _dev(dout, "dout", dt),
                                           _dev(dq, "dq", dt), _dev(dk, "dk", dt), _dev(dv, "dv", dt),
                                           _dev(dtable, "dtable", torch.float32), _dev(workspace, "workspace"),
                                           _stream(stream)))


def swa_backward(handle, q, k, v, table, dout, dq, dk, dv, dtable, workspace, stream=None) -> None:
    dt = q.dtype
    _check(load_library().swa_backward(handle, _dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt),
                                       _dev(table, "table", torch.float32), _dev(dout, "dout", dt),
                                       _dev(dq, "dq", dt), _dev(dk, "dk", dt), _dev(dv, "dv", dt),
                                       _dev(dtable, "dtable", torch.float32), _dev(workspace, "workspace"),
                                       _stream(stream)))


def swa_backward_noalloc(handle, q, k, v, table, dout, dq, dk, dv, dtable, stream=None) -> None:
    dt = q.dtype
    _check(load_library().swa_backward_noalloc(handle, _dev(q, "q"), _dev(k, "k", dt), _dev(v, "v", dt),
                                               _dev(table, "table", torch.float32), _dev(dout, "dout", dt),
                                               _dev(dq, "dq", dt), _dev(dk, "dk", dt), _dev(dv, "dv", dt),
                                               _dev(dtable, "dtable", torch.float32), _stream(stream)))


def swa_layer_forward(handle, x, w_qkv, b_qkv, table, w_o, b_o, y, workspace, stream=None) -> None:
    dt = x.dtype
    f32 = torch.float32
    _check(load_library().swa_layer_forward(handle, _dev(x, "x"), _dev(w_qkv, "w_qkv", dt), _dev(b_qkv, "b_qkv", f32),
                                            _dev(table, "table", f32), _dev(w_o, "w_o", dt), _dev(b_o, "b_o", f32),
                                            _dev(y, "y", dt), _dev(workspace, "workspace"), _stream(stream)))


def swa_layer_attention(handle, x, w_qkv, b_qkv, table, out, stream=None) -> None:
    dt = x.dtype
    f32 = torch.float32
    _check(load_library().swa_layer_attention(handle, _dev(x, "x"), _dev(w_qkv, "w_qkv", dt),
                                              _dev(b_qkv, "b_qkv", f32), _dev(table, "table", f32),
                                              _dev(out, "out", dt), _stream(stream)))


def swa_projection(x, w, bias, outputs, split=None, stream=None) -> None:
    """outputs[n // split][m, n % split] = (x @ w.T + bias)[m, n]; x [rows, in],
    w [out, in], bias [out] fp32, outputs: 1 to 3 tensors of rows * split
    elements (split defaults to out)."""
    dt = x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    rows, fin = x.shape
    fout = w.shape[0]
    if tuple(w.shape) != (fout, fin) or tuple(bias.shape) != (fout,):
        raise ValueError("w must be [out, in] and bias [out]")
    split = fout if split is None else int(split)
    need = (fout + split - 1) // split
    if len(outputs) != need:
        raise ValueError(f"{need} output tensors expected")
    for i, o in enumerate(outputs):
        if o.numel() != rows * split:
            raise ValueError(f"output {i} must hold rows * split elements")
    ptrs = [_dev(o, f"out{i}", dt) for i, o in enumerate(outputs)] + [None] * (3 - need)
    _check(load_library().swa_projection(SWA_F32 if dt == torch.float32 else SWA_BF16, _dev(x, "x"),
                                         _dev(w, "w", dt), _dev(bias, "bias", torch.float32), rows, fout, fin,
                                         split, *ptrs, _stream(stream)))


def swa_gather(handle, src, dst_window_major, stream=None) -> None:
    _check(load_library().swa_gather(handle, _dev(src, "src"), _dev(dst_window_major, "dst", src.dtype),
                                     _stream(stream)))


def swa_scatter(handle, src_window_major, dst, stream=None) -> None:
    _check(load_library().swa_scatter(handle, _dev(src_window_major, "src"),
                                      _dev(dst, "dst", src_window_major.dtype), _stream(stream)))


def swa_debug_visibility(handle, window_index: int, dev_out, stream=None) -> None:
    _check(load_library().swa_debug_visibility(handle, int(window_index),
                                               _dev(dev_out, "out", torch.uint8), _stream(stream)))


class WindowAttention:
    """Owns one handle for a problem; checks tensor shapes before each call."""

    def __init__(self, problem, variant: str = "fused", schedule: str = "auto", layer: str = "auto"):
        self.problem = problem
        self.dtype = torch.float32 if problem.dtype == "f32" else torch.bfloat16
        self.handle = swa_create(make_config(problem, variant, schedule, layer))
        self.info = swa_get_info(self.handle)

    @property
    def io_shape(self):
        p = self.problem
        return (p.batch,) + tuple(p.extent) + (p.heads, p.head_dim)

    @property
    def window_major_shape(self):
        p = self.problem
        return (self.info.windows, self.info.window_tokens, p.heads, p.head_dim)

    def _shape(self, t, shape, name):
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")

    def forward(self, q, k, v, table, out=None, stream=None):
        for name, t in (("q", q), ("k", k), ("v", v)):
            self._shape(t, self.io_shape, name)
        w = self.problem.window
        self._shape(table, (2 * w[0] - 1, 2 * w[1] - 1, 2 * w[2] - 1, self.problem.heads), "table")
        if out is None:
            out = torch.empty_like(q)
        self._shape(out, self.io_shape, "out")
        swa_forward(self.handle, q, k, v, table, out, stream)
        return out

    def forward_lse(self, q, k, v, table, out=None, lse=None, stream=None):
        """forward() that also returns each query's log-sum-exp [B, T, H, W, heads] (fp32)."""
        for name, t in (("q", q), ("k", k), ("v", v)):
            self._shape(t, self.io_shape, name)
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(self.io_shape[:-1], dtype=torch.float32, device=q.device)
        swa_forward_lse(self.handle, q, k, v, table, out, lse, stream)
        return out, lse

    def backward(self, q, k, v, table, dout, stream=None):
        """Gradients (dq, dk, dv, dtable) of sum(dout * forward(q, k, v, table))."""
        for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
            self._shape(t, self.io_shape, name)
        w = self.problem.window
        self._shape(table, (2 * w[0] - 1, 2 * w[1] - 1, 2 * w[2] - 1, self.problem.heads), "table")
        nws = self.info.backward_workspace_bytes
        if nws == 0:
            raise SwaError(SWA_ERR_UNSUPPORTED, "the backward kernels do not take this window")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dtable = torch.empty_like(table)
        ws = torch.empty((nws + 15) // 16 * 4, dtype=torch.float32, device=q.device)
        swa_backward(self.handle, q, k, v, table, dout, dq, dk, dv, dtable, ws, stream)
        return dq, dk, dv, dtable

    def backward_lse(self, q, k, v, table, out, lse, dout, stream=None):
        """backward() from the forward's output and log-sum-exp (forward_lse)."""
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
            self._shape(t, self.io_shape, name)
        self._shape(lse, self.io_shape[:-1], "lse")
        nws = self.info.backward_workspace_bytes
        if nws == 0:
            raise SwaError(SWA_ERR_UNSUPPORTED, "the backward kernels do not take this window")
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dtable = torch.empty_like(table)
        ws = torch.empty((nws + 15) // 16 * 4, dtype=torch.float32, device=q.device)
        swa_backward_lse(self.handle, q, k, v, table, out, lse, dout, dq, dk, dv, dtable, ws, stream)
        return dq, dk, dv, dtable

    @property
    def channels(self):
        return self.problem.heads * self.problem.head_dim

    def layer_workspace(self, device="cuda"):
        """A workspace for layer_forward (o of the layer on the fused path; q, k, v and o
        on the unfused one)."""
        n = self.info.layer_workspace_bytes
        return torch.empty(n // (2 if self.dtype == torch.bfloat16 else 4), dtype=self.dtype, device=device)

    def layer_forward(self, x, w_qkv, b_qkv, table, w_o, b_o, y=None, workspace=None, stream=None):
        """y = attention(x w_qkv^T + b_qkv split into q, k, v) w_o^T + b_o."""
        p, C = self.problem, self.channels
        self._shape(x, (p.batch,) + tuple(p.extent) + (C,), "x")
        self._shape(w_qkv, (3 * C, C), "w_qkv")
        self._shape(b_qkv, (3 * C,), "b_qkv")
        self._shape(w_o, (C, C), "w_o")
        self._shape(b_o, (C,), "b_o")
        w = p.window
        self._shape(table, (2 * w[0] - 1, 2 * w[1] - 1, 2 * w[2] - 1, p.heads), "table")
        if y is None:
            y = torch.empty_like(x)
        self._shape(y, x.shape, "y")
        if workspace is None:
            workspace = self.layer_workspace(x.device)
        if workspace.numel() * workspace.element_size() < self.info.layer_workspace_bytes:
            raise ValueError("workspace too small")
        swa_layer_forward(self.handle, x, w_qkv, b_qkv, table, w_o, b_o, y, workspace, stream)
        return y

    def gather(self, src, dst=None, stream=None):
        self._shape(src, self.io_shape, "src")
        if dst is None:
            dst = torch.empty(self.window_major_shape, dtype=src.dtype, device=src.device)
        self._shape(dst, self.window_major_shape, "dst")
        swa_gather(self.handle, src, dst, stream)
        return dst

    def scatter(self, src, dst=None, stream=None):
        self._shape(src, self.window_major_shape, "src")
        if dst is None:
            dst = torch.empty(self.io_shape, dtype=src.dtype, device=src.device)
        self._shape(dst, self.io_shape, "dst")
        swa_scatter(self.handle, src, dst, stream)
        return dst

    def visibility(self, window_index, stream=None):
        n = self.info.window_tokens
        out = torch.empty((n, n), dtype=torch.uint8, device="cuda")
        swa_debug_visibility(self.handle, window_index, out, stream)
        return out

    def close(self):
        if self.handle is not None:
            swa_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
