"""The attention layer around the window attention, in numpy fp64 (test
infrastructure only).

TERRA's models are stacks of Swin blocks (TERRA page, abstract; Table V: the
embedding width d and N_h heads).  In a Swin block the window attention sits
between a linear projection of each token to its queries, keys and values
and a linear projection of the attended values back to the embedding width.
For one token grid:

    QKV = X W_qkv^T + b_qkv         X: [B, T, H, W, C], C = heads * head_dim
    Q = QKV[.., 0:C], K = QKV[.., C:2C], V = QKV[.., 2C:3C], each read as
        [heads, head_dim] (the channels of one head are contiguous)
    O = shifted-window attention of Q, K, V with the bias table
    Y = O W_o^T + b_o               O read as [.., C] the same way

Weights have the [out_features, in_features] layout of a linear layer and
the biases are fp32 vectors.  The projections are plain matrix products in
fp64; the attention step is the C direct form, which reads fp32, so it takes
the fp64 projections rounded to fp32 (relative error 2^-24, far below every
tolerance this oracle serves).
"""
import numpy as np

from .backward import token_windows
from .direct import direct_forward


def linear(x, w, b):
    """x w^T + b in fp64: x [.., in], w [out, in] (a linear layer's layout), b [out]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T + np.asarray(b, dtype=np.float64)


def _needed_tokens(prob, query_index):
    """Flat token indices whose keys and values the queries can see: every
    token of the windows that hold them."""
    tw = token_windows(prob).ravel()  # window of each token of one batch item
    per_item = tw.size
    nW = int(tw.max()) + 1
    qi = np.asarray(query_index, dtype=np.int64)
    qwin = np.unique((qi // per_item) * nW + tw[qi % per_item])
    all_win = (np.arange(prob.batch)[:, None] * nW + tw[None, :]).ravel()
    return np.nonzero(np.isin(all_win, qwin))[0]


def layer_forward(prob, x, w_qkv, b_qkv, table, w_o, b_o, query_index=None):
    """fp64 Y [B, T, H, W, C], or [len(query_index), C] for flat real-token
    indices ((b*T + t)*H + y)*W + x.  With query_index, only the tokens of
    the windows of those queries are projected."""
    B, (T, H, W) = prob.batch, prob.extent
    heads, d = prob.heads, prob.head_dim
    C = heads * d
    M = B * T * H * W
    x = np.asarray(x).reshape(M, C)
    rows = np.arange(M) if query_index is None else _needed_tokens(prob, query_index)
    qkv = linear(x[rows], np.reshape(w_qkv, (3 * C, C)), np.reshape(b_qkv, 3 * C))  # [len(rows), 3C]
    shape = (B, T, H, W, heads, d)
    q, k, v = (np.zeros((M, C), dtype=np.float32) for _ in range(3))
    for i, dst in enumerate((q, k, v)):
        dst[rows] = qkv[:, i * C:(i + 1) * C]
    o, _ = direct_forward(prob, q.reshape(shape), k.reshape(shape), v.reshape(shape), table,
                          query_index=query_index)
    return linear(o.reshape(o.shape[:-2] + (C,)), np.reshape(w_o, (C, C)), b_o)


__all__ = ["layer_forward", "linear"]
