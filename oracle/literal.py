"""Literal form of the oracle, in numpy fp64, for small grids.

Test infrastructure only.  It follows the pipeline the TERRA page describes
in its abstract (tokens leave the spatial layout for a window layout, the
Transformer attends inside windows with shifted-window execution, and tokens
return to the spatial layout) with the padded resolution of its Table I:

  1. pad each axis at its end to the padded extent, flagging pad tokens;
  2. roll the padded grid by -s on every axis (rolled[c'] = padded[(c'+s) mod P]);
  3. cut the rolled grid into windows, local order row-major (t, y, x);
  4. per (window, head): logits = scale * Q K^T + relative-position bias;
  5. mask a pair when the key is pad, or when query and key lie on opposite
     sides of the wrap of a masked axis (c' >= P - s is the wrapped part);
  6. softmax over the visible keys, then the weighted sum of V;
  7. undo the partition and the roll, and crop the padding.

This is a second formulation beside the C direct form, written separately;
tests require the two to agree to rounding.

A problem is any object with ``batch, heads, head_dim, extent, padded,
window, shift, cyclic`` (3-tuples, time/latitude/longitude) and optionally
``scale``.
"""
import math

import numpy as np


def _scale(prob):
    s = getattr(prob, "scale", None)
    return float(s) if s else 1.0 / math.sqrt(prob.head_dim)


def _counts(prob):
    nw = tuple(prob.padded[a] // prob.window[a] for a in range(3))
    return nw, int(np.prod(nw)), int(np.prod(prob.window))


def pad_flags(prob):
    """Step 1's pad flag over the padded grid [P_t, P_y, P_x] (True = pad)."""
    flag = np.ones(tuple(prob.padded), dtype=bool)
    T, H, W = prob.extent
    flag[:T, :H, :W] = False
    return flag


def _pad(prob, x):
    B, (T, H, W) = prob.batch, prob.extent
    out = np.zeros((B,) + tuple(prob.padded) + x.shape[4:], dtype=np.float64)
    out[:, :T, :H, :W] = x
    return out


def _roll(prob, x, sign):
    # sign = -1: rolled[c'] = x[(c' + s) mod P]; sign = +1 undoes it.
    return np.roll(x, shift=tuple(sign * s for s in prob.shift), axis=(1, 2, 3))


def _partition(prob, x):
    """[B, P_t, P_y, P_x, ...] -> [B, nW, N, ...] with windows row-major."""
    (wt, wy, wx), B = prob.window, x.shape[0]
    (nt, ny, nx), nW, N = _counts(prob)
    rest = x.shape[4:]
    y = x.reshape((B, nt, wt, ny, wy, nx, wx) + rest)
    r = len(rest)
    y = y.transpose((0, 1, 3, 5, 2, 4, 6) + tuple(range(7, 7 + r)))
    return y.reshape((B, nW, N) + rest)


def _unpartition(prob, y):
    (wt, wy, wx), B = prob.window, y.shape[0]
    (nt, ny, nx), nW, N = _counts(prob)
    rest = y.shape[3:]
    r = len(rest)
    x = y.reshape((B, nt, ny, nx, wt, wy, wx) + rest)
    x = x.transpose((0, 1, 4, 2, 5, 3, 6) + tuple(range(7, 7 + r)))
    return x.reshape((B,) + tuple(prob.padded) + rest)


def literal_windows(prob, x):
    """Steps 1-3 applied to a [B, T, H, W, heads, d] tensor: the window-major
    tensor [B, nW, N, heads, d] (pad slots hold zeros)."""
    x = np.asarray(x, dtype=np.float64)
    return _partition(prob, _roll(prob, _pad(prob, x), -1))


def literal_unwindows(prob, y):
    """Step 7: window-major [B, nW, N, heads, d] back to [B, T, H, W, heads, d]."""
    T, H, W = prob.extent
    return _roll(prob, _unpartition(prob, np.asarray(y, dtype=np.float64)), +1)[:, :T, :H, :W]


def _window_local_coords(prob):
    """[N, 3] position of each local index inside its window (rolled frame)."""
    wt, wy, wx = prob.window
    t, y, x = np.meshgrid(np.arange(wt), np.arange(wy), np.arange(wx), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)


def literal_bias(prob, table):
    """Step 4's bias per head: [heads, N, N], entry [h, n, m] =
    table[l(n) - l(m) + w - 1, h] using positions inside the window."""
    lc = _window_local_coords(prob)
    rel = lc[:, None, :] - lc[None, :, :] + (np.asarray(prob.window) - 1)
    tab = np.asarray(table, dtype=np.float64)
    return np.moveaxis(tab[rel[..., 0], rel[..., 1], rel[..., 2]], -1, 0)


def literal_visibility(prob):
    """Step 5 as a boolean [nW, N, N]: entry [w, n, m] is True when key m may
    be attended by query n in window w (both real, same side of every wrap)."""
    rolled_pad = _partition(prob, _roll(prob, pad_flags(prob)[None, ..., None], -1))[0, ..., 0]
    P = np.asarray(prob.padded)
    s = np.asarray(prob.shift)
    # wrapped part of each masked axis in the rolled frame: c' >= P - s
    coords = np.stack(np.meshgrid(*[np.arange(p) for p in prob.padded], indexing="ij"), axis=-1)
    wrapped = coords >= (P - s)
    for a in range(3):
        if prob.cyclic[a]:
            wrapped[..., a] = False
    wrapped_w = _partition(prob, wrapped[None])[0]  # [nW, N, 3]
    same = np.all(wrapped_w[:, :, None, :] == wrapped_w[:, None, :, :], axis=-1)
    real = ~rolled_pad
    return same & real[:, :, None] & real[:, None, :]


def literal_forward(prob, q, k, v, table):
    """Steps 1-7: fp64 output [B, T, H, W, heads, d] for real query tokens."""
    qw, kw, vw = (literal_windows(prob, a) for a in (q, k, v))  # [B, nW, N, h, d]
    bias = literal_bias(prob, table)  # [h, N, N]
    vis = literal_visibility(prob)  # [nW, N, N]
    logits = np.einsum("bwnhe,bwmhe->bwhnm", qw, kw) * _scale(prob) + bias[None, None]
    logits = np.where(vis[None, :, None], logits, -np.inf)
    has_key = vis.any(axis=-1)  # pad queries see nothing; their rows are cropped
    mx = np.where(has_key[None, :, None, :, None], logits.max(axis=-1, keepdims=True), 0.0)
    e = np.where(vis[None, :, None], np.exp(logits - mx), 0.0)
    den = e.sum(axis=-1, keepdims=True)
    p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
    ow = np.einsum("bwhnm,bwmhe->bwnhe", p, vw)
    return literal_unwindows(prob, ow)


def literal_lse(prob, q, k, table):
    """Steps 1-6 up to the softmax's normaliser: fp64 log-sum-exp (natural log)
    of each real query's logits over its visible keys, [B, T, H, W, heads].
    The softmax weight of a visible key is exp(logit - lse)."""
    qw, kw = literal_windows(prob, q), literal_windows(prob, k)  # [B, nW, N, h, d]
    bias = literal_bias(prob, table)  # [h, N, N]
    vis = literal_visibility(prob)  # [nW, N, N]
    logits = np.einsum("bwnhe,bwmhe->bwhnm", qw, kw) * _scale(prob) + bias[None, None]
    logits = np.where(vis[None, :, None], logits, -np.inf)
    has_key = vis.any(axis=-1)[None, :, None, :]  # [1, nW, 1, N]
    mx = np.where(has_key, logits.max(axis=-1), 0.0)
    den = np.where(vis[None, :, None], np.exp(logits - mx[..., None]), 0.0).sum(axis=-1)
    with np.errstate(divide="ignore"):
        lse = np.where(den > 0, mx + np.log(np.where(den > 0, den, 1.0)), -np.inf)  # [B, nW, h, N]
    return literal_unwindows(prob, np.moveaxis(lse, 2, 3))

