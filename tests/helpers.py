"""Shared test helpers: inputs on the device, oracle evaluation, error metric."""
import numpy as np
import torch

import oracle
from shifted_window_attention_cyclic_amd.inputs import make_inputs

# Tolerances on max|O_gpu - O_ref| / max|O_ref| (relative max-abs error)
TOL = {"f32": 1e-5, "bf16": 1e-2}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 copy (bf16 values are exact in fp32)."""
    return t.detach().to("cpu", torch.float32).numpy()


def device_inputs(p, seed=None):
    x = make_inputs(p, seed=seed)
    return x, {n: t.cuda() for n, t in x.items()}


def oracle_full(p, x):
    out, _ = oracle.direct_forward(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                   host_f32(x["table"]))
    return out


def oracle_at(p, x, token_index):
    out, _ = oracle.direct_forward(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                   host_f32(x["table"]), query_index=token_index)
    return out


def sample_tokens(p, count=256, seed=0):
    """Flat token indices that cover every kind of window edge (first and last
    rows/columns, shift boundaries, pad neighbours) plus random ones."""
    B, (T, H, W) = p.batch, p.extent
    s, w = p.shift, p.window

    def edges(E, s_, w_):
        c = {0, 1, E - 1, E - 2, s_ % E, (s_ - 1) % E, (s_ + w_) % E, (s_ + w_ - 1) % E,
             E // 2, (E - s_) % E, (E - s_ - 1) % E}
        return sorted(x for x in c if 0 <= x < E)

    ts, ys, xs = edges(T, s[0], w[0]), edges(H, s[1], w[1]), edges(W, s[2], w[2])
    idx = set()
    for b in sorted({0, B - 1}):
        for t in ts:
            for y in ys:
                for x_ in xs:
                    idx.add(((b * T + t) * H + y) * W + x_)
    rng = np.random.default_rng(seed)
    idx.update(int(i) for i in rng.integers(0, p.tokens, size=count))
    return np.array(sorted(idx), dtype=np.int64)
