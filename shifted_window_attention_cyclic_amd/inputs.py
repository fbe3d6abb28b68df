"""Problem shapes and seeded synthetic inputs.

This module holds no attention arithmetic: only the workload shapes and the
random draws that both the library's tests and the oracle's tests feed in.
Shapes follow the grids the pages work on: the 0.25 degree field and the
1/12 degree field at patch size 4 (TERRA page, Table V patch size; BEAST's
0.25 degree atmosphere), with heads and window sizes in the range of TERRA's
Table V.  The sixth and seventh workloads are the layer shapes of Table V's
Small model (d = 1024 over N_h = 8 heads of 128, w = 8) and Large model
(d = 8192 over N_h = 64 heads of 128, w = 32).  32-wide windows tile neither
360 nor 1080 longitude points, so the Large shape takes the 0.25 degree
grid's 180 latitude rows (padded to 192) and 384 longitude points, the next
multiple of 32.  All tensors are [B, T, H, W, heads, head_dim],
C-contiguous, over the REAL extents; axis 0 is time, 1 latitude, 2
longitude.
"""
from dataclasses import dataclass, replace
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Problem:
    name: str
    dtype: str  # "f32" or "bf16": the Q/K/V/O element type
    batch: int
    heads: int
    head_dim: int
    extent: Tuple[int, int, int]  # real (T, H, W)
    padded: Tuple[int, int, int]  # padded (T^, H^, W^)
    window: Tuple[int, int, int]
    shift: Tuple[int, int, int]
    cyclic: Tuple[int, int, int] = (0, 0, 1)  # longitude cyclic, time and latitude masked
    scale: Optional[float] = None  # None: 1/sqrt(head_dim)
    seed: int = 0
    table_std: float = 0.02

    @property
    def ndim(self) -> int:
        return 3 if (self.extent[0] > 1 or self.window[0] > 1) else 2

    @property
    def tokens(self) -> int:
        return self.batch * self.extent[0] * self.extent[1] * self.extent[2]

    @property
    def window_tokens(self) -> int:
        return self.window[0] * self.window[1] * self.window[2]

    @property
    def windows(self) -> int:
        """Windows over the padded grid, all batches."""
        n = self.batch
        for a in range(3):
            n *= self.padded[a] // self.window[a]
        return n

    @property
    def table_shape(self) -> Tuple[int, int, int, int]:
        w = self.window
        return (2 * w[0] - 1, 2 * w[1] - 1, 2 * w[2] - 1, self.heads)

    @property
    def io_shape(self) -> Tuple[int, ...]:
        return (self.batch,) + tuple(self.extent) + (self.heads, self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def with_(self, **kw) -> "Problem":
        return replace(self, **kw)


# The workloads.  Seeds are 1000 + index.
WORKLOADS = {
    "c1_f32_16x32": Problem("c1_f32_16x32", "f32", 1, 3, 32, (1, 16, 32), (1, 16, 32),
                            (1, 8, 8), (0, 4, 4), seed=1000),
    "c2_bf16_180x360": Problem("c2_bf16_180x360", "bf16", 1, 6, 32, (1, 180, 360), (1, 180, 360),
                               (1, 12, 12), (0, 6, 6), seed=1001),
    "c3_bf16_540x1080": Problem("c3_bf16_540x1080", "bf16", 1, 8, 64, (1, 540, 1080),
                                (1, 540, 1080), (1, 12, 12), (0, 6, 6), seed=1002),
    "c4_bf16_181x360_pad190": Problem("c4_bf16_181x360_pad190", "bf16", 2, 8, 64, (1, 181, 360),
                                      (1, 190, 360), (1, 10, 10), (0, 5, 5), seed=1003),
    "c5_bf16_4x180x360_3d": Problem("c5_bf16_4x180x360_3d", "bf16", 1, 12, 64, (4, 180, 360),
                                    (4, 180, 360), (2, 12, 12), (1, 6, 6), seed=1004),
    # TERRA, Table V, Small model: 8 heads of 128, 8 x 8 windows (N = 64); 180
    # latitude rows padded to 184 so that the windows tile the grid
    "c6_bf16_180x360_pad184_d128": Problem("c6_bf16_180x360_pad184_d128", "bf16", 1, 8, 128, (1, 180, 360),
                                           (1, 184, 360), (1, 8, 8), (0, 4, 4), seed=1005),
    # TERRA, Table V, Large model: 64 heads of 128, 32 x 32 windows (N = 1024)
    "c7_bf16_180x384_pad192_d128_w32": Problem("c7_bf16_180x384_pad192_d128_w32", "bf16", 1, 64, 128,
                                               (1, 180, 384), (1, 192, 384), (1, 32, 32), (0, 16, 16),
                                               seed=1006),
    # the 1/12 degree field with a batch of 4: 2.39 GB per tensor, past 2^31 bytes
    "c3b4_bf16_540x1080": Problem("c3b4_bf16_540x1080", "bf16", 4, 8, 64, (1, 540, 1080),
                                  (1, 540, 1080), (1, 12, 12), (0, 6, 6), seed=1007),
}
ORDER = list(WORKLOADS)


def torch_dtype(p: Problem):
    return torch.float32 if p.dtype == "f32" else torch.bfloat16


def make_inputs(p: Problem, seed: Optional[int] = None, qkv_std: float = 1.0):
    """Seeded draws in a fixed order: Q, K, V ~ N(0, qkv_std^2) in fp32, then
    the bias table ~ N(0, table_std^2) in fp32.  Q/K/V are rounded to the
    problem's dtype (round-to-nearest-even for bf16) and returned as CPU
    tensors of that dtype; the table stays fp32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(p.seed if seed is None else seed)
    dt = torch_dtype(p)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = (torch.randn(p.io_shape, generator=g, dtype=torch.float32) * qkv_std).to(dt)
    out["table"] = torch.randn(p.table_shape, generator=g, dtype=torch.float32) * p.table_std
    return out


def small_variant(p: Problem, lat: int, lon: int, t: Optional[int] = None) -> Problem:
    """The same heads, window, shift and dtype on a smaller grid that still
    spans several windows (and keeps a pad tail when the original has one)."""
    T = p.extent[0] if t is None else t
    pad_h = p.padded[1] - p.extent[1]
    return p.with_(name=p.name + f"_small{T}x{lat}x{lon}", extent=(T, lat, lon),
                   padded=(T, lat + pad_h, lon))


def make_layer_inputs(p: Problem, seed: Optional[int] = None):
    """Seeded draws for the projection layer, in a fixed order: the token
    embeddings X ~ N(0, 1) [B, T, H, W, C] (C = heads * head_dim), the
    weights W_qkv [3C, C] and W_o [C, C] ~ N(0, 1/C) (so that Q, K, V come
    out near unit variance), the biases b_qkv [3C] and b_o [C] ~ N(0, 0.02^2)
    and the attention's bias table ~ N(0, table_std^2).  X and the weights
    are rounded to the problem's dtype; biases and table stay fp32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(p.seed if seed is None else seed)
    dt = torch_dtype(p)
    C = p.heads * p.head_dim
    out = {"x": torch.randn((p.batch,) + tuple(p.extent) + (C,), generator=g).to(dt)}
    out["w_qkv"] = (torch.randn((3 * C, C), generator=g) / C ** 0.5).to(dt)
    out["b_qkv"] = torch.randn(3 * C, generator=g) * 0.02
    out["w_o"] = (torch.randn((C, C), generator=g) / C ** 0.5).to(dt)
    out["b_o"] = torch.randn(C, generator=g) * 0.02
    out["table"] = torch.randn(p.table_shape, generator=g, dtype=torch.float32) * p.table_std
    return out
