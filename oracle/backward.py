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

from .literal import (_partition, _roll, _scale, _window_local_coords, literal_bias,
                      literal_unwindows, literal_visibility, literal_windows, pad_flags)


def _relative_index(prob):
    """[N, N, 3] table index (t, y, x) that the bias of (query n, key m) uses."""
    lc = _window_local_coords(prob)
    return lc[:, None, :] - lc[None, :, :] + (np.asarray(prob.window) - 1)


def token_windows(prob):
    """[T, H, W] window-major index (over one batch item) of the window each real
    token lies in."""
    P = tuple(prob.padded)
    ids = np.arange(int(np.prod(P))).reshape(P)
    rolled = _partition(prob, _roll(prob, ids[None, ..., None], -1))[0, ..., 0]  # [nW, N]
    win_of = np.empty(int(np.prod(P)), dtype=np.int64)
    win_of[rolled.ravel()] = np.repeat(np.arange(rolled.shape[0]), rolled.shape[1])
    T, H, W = prob.extent
    return win_of.reshape(P)[:T, :H, :W]


def literal_backward(prob, q, k, v, table, dout, windows=None):
    """Gradients (dq, dk, dv, dtable) of sum(dout * forward(q, k, v, table)),
    fp64.  dq, dk, dv: [B, T, H, W, heads, d]; dtable: the table's shape."""
    qw, kw, vw, dow = (literal_windows(prob, a) for a in (q, k, v, dout))  # [B, nW, N, h, d]
    B, nW, N = qw.shape[:3]
    sel = np.zeros((B, nW), dtype=bool)
    if windows is None:
        sel[:] = True
    else:
        flat = np.asarray(windows, dtype=np.int64)
        sel.reshape(-1)[flat] = True
    bias = literal_bias(prob, table)  # [h, N, N]
    vis = literal_visibility(prob)  # [nW, N, N]
    scale = _scale(prob)
    dqw, dkw, dvw = np.zeros_like(qw), np.zeros_like(kw), np.zeros_like(vw)
    dbias = np.zeros(bias.shape, dtype=np.float64)  # [h, N, N], summed over windows
    for b in range(B):
        for w in range(nW):
            if not sel[b, w]:
                continue
            Q, K, V, dO = qw[b, w], kw[b, w], vw[b, w], dow[b, w]  # [N, h, d]
            logits = np.einsum("nhe,mhe->hnm", Q, K) * scale + bias
            m = vis[w][None]
            logits = np.where(m, logits, -np.inf)
            has_key = m.any(axis=-1, keepdims=True)
            mx = np.where(has_key, logits.max(axis=-1, keepdims=True), 0.0)
            e = np.where(m, np.exp(logits - mx), 0.0)
            den = e.sum(axis=-1, keepdims=True)
            P = np.divide(e, den, out=np.zeros_like(e), where=den > 0)  # [h, N, N]
            dvw[b, w] = np.einsum("hnm,nhe->mhe", P, dO)
            dP = np.einsum("nhe,mhe->hnm", dO, V)
            D = (P * dP).sum(axis=-1, keepdims=True)
            dS = P * (dP - D)
            dqw[b, w] = scale * np.einsum("hnm,mhe->nhe", dS, K)
            dkw[b, w] = scale * np.einsum("hnm,nhe->mhe", dS, Q)
            dbias += dS
    # the table entry each bias element was read from
    rel = _relative_index(prob)
    dtable = np.zeros(np.asarray(table).shape, dtype=np.float64)
    for h in range(dbias.shape[0]):
        np.add.at(dtable[..., h], (rel[..., 0], rel[..., 1], rel[..., 2]), dbias[h])
    return (literal_unwindows(prob, dqw), literal_unwindows(prob, dkw), literal_unwindows(prob, dvw),
            dtable)


__all__ = ["literal_backward", "token_windows", "pad_flags"]
