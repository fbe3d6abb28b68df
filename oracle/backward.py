"""Backward pass of the oracle, in numpy fp64 (test infrastructure only).

The pages train the model (TERRA page, abstract: training of high-resolution
Earth models; its Table V models are trained), so the layer's gradients are
those of the forward pass the literal form computes, window by window:

  forward, per (window, head):  S = scale * Q K^T + B,  S = -inf where masked,
                                P = softmax over keys,  O = P V
  backward, given dO:           dV = P^T dO
                                dP = dO V^T
                                D  = row sums of P * dP
                                dS = P * (dP - D)
                                dQ = scale * dS K
                                dK = scale * dS^T Q
                                dB[n, m] = dS[n, m], summed into the table entry
                                           that B[n, m] was read from, over all
                                           windows and batch items of the head

Pad tokens have no output, so their dO is 0; masked pairs have P = 0, so they
add nothing.  Every real token lies in exactly one window of the shifted
partition, so its dQ, dK and dV come from that window alone.  ``windows``
selects a subset of windows (indices into the window-major order, batch
included): the gradients of the tokens in them are complete, the rest are
zero, and the table gradient holds those windows' share only.
"""
import numpy as np

from .literal import _partition, _roll, _scale, _window_local_coords, literal_bias, literal_visibility


def _relative_index(prob):
    """[N, N, 3] table index (t, y, x) that the bias of (query n, key m) uses."""
    lc = _window_local_coords(prob)
    return lc[:, None, :] - lc[None, :, :] + (np.asarray(prob.window) - 1)


def window_tokens(prob):
    """[nW, N]: for each window (of one batch item) and local slot, the flat
    index (t * H + y) * W + x of the real token there, or -1 for a pad slot:
    steps 1-3 of the literal form applied to a grid of token indices."""
    T, H, W = prob.extent
    idx = np.full(tuple(prob.padded), -1, dtype=np.int64)
    idx[:T, :H, :W] = np.arange(T * H * W).reshape(T, H, W)
    return _partition(prob, _roll(prob, idx[None, ..., None], -1))[0, ..., 0]


def token_windows(prob):
    """[T, H, W]: the window (of one batch item) each real token lies in."""
    tok = window_tokens(prob)
    T, H, W = prob.extent
    out = np.empty(T * H * W, dtype=np.int64)
    w, n = np.nonzero(tok >= 0)
    out[tok[w, n]] = w
    return out.reshape(T, H, W)


def literal_backward(prob, q, k, v, table, dout, windows=None):
    """Gradients (dq, dk, dv, dtable) of sum(dout * forward(q, k, v, table)),
    fp64.  dq, dk, dv: [B, T, H, W, heads, d]; dtable: the table's shape."""
    B, (T, H, W) = prob.batch, prob.extent
    heads, d = prob.heads, prob.head_dim
    flat = [np.asarray(a).reshape(B, T * H * W, heads, d) for a in (q, k, v, dout)]
    tok = window_tokens(prob)  # [nW, N]
    nW, N = tok.shape
    chosen = range(B * nW) if windows is None else sorted(set(int(w) for w in windows))
    bias = literal_bias(prob, table)  # [h, N, N]
    vis = literal_visibility(prob)  # [nW, N, N]
    scale = _scale(prob)
    grads = [np.zeros((B, T * H * W, heads, d), dtype=np.float64) for _ in range(3)]
    dbias = np.zeros(bias.shape, dtype=np.float64)  # [h, N, N], summed over windows
    for bw in chosen:
        b, w = divmod(bw, nW)
        real = tok[w] >= 0
        rows = tok[w][real]
        Q, K, V, dO = (np.zeros((N, heads, d), dtype=np.float64) for _ in range(4))
        for dst, src in zip((Q, K, V, dO), flat):
            dst[real] = src[b, rows]  # pad slots stay 0 (pad queries have no dO)
        logits = np.einsum("nhe,mhe->hnm", Q, K) * scale + bias
        m = vis[w][None]
        logits = np.where(m, logits, -np.inf)
        has_key = m.any(axis=-1, keepdims=True)
        mx = np.where(has_key, logits.max(axis=-1, keepdims=True), 0.0)
        e = np.where(m, np.exp(logits - mx), 0.0)
        den = e.sum(axis=-1, keepdims=True)
        P = np.divide(e, den, out=np.zeros_like(e), where=den > 0)  # [h, N, N]
        dV = np.einsum("hnm,nhe->mhe", P, dO)
        dP = np.einsum("nhe,mhe->hnm", dO, V)
        D = (P * dP).sum(axis=-1, keepdims=True)
        dS = P * (dP - D)
        dQ = scale * np.einsum("hnm,mhe->nhe", dS, K)
        dK = scale * np.einsum("hnm,nhe->mhe", dS, Q)
        for g, val in zip(grads, (dQ, dK, dV)):
            g[b, rows] = val[real]
        dbias += dS
    # the table entry each bias element was read from
    rel = _relative_index(prob)
    dtable = np.zeros(np.asarray(table).shape, dtype=np.float64)
    for h in range(heads):
        np.add.at(dtable[..., h], (rel[..., 0], rel[..., 1], rel[..., 2]), dbias[h])
    shape = (B, T, H, W, heads, d)
    return grads[0].reshape(shape), grads[1].reshape(shape), grads[2].reshape(shape), dtable


__all__ = ["literal_backward", "token_windows", "window_tokens"]
