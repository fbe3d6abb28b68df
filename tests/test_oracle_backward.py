"""Pins of the oracle's backward pass (CPU only).

The gradients are pinned to things outside the backward code itself: central
finite differences of the C direct-form forward (an independent formulation
of the forward pass), torch's autograd on dense attention for a single global
window, and invariants that hold exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from shifted_window_attention_cyclic_amd.inputs import Problem


def _prob(name, B, heads, d, extent, padded, window, shift, cyclic=(0, 0, 1), scale=None):
    return Problem(name, "f32", B, heads, d, extent, padded, window, shift, cyclic, scale=scale)


CASES = {
    # ragged latitude padded 9 -> 12, longitude cyclic
    "ragged_2d": _prob("ragged_2d", 2, 2, 4, (1, 9, 12), (1, 12, 12), (1, 4, 6), (0, 2, 3)),
    # 3-D, time padded 3 -> 4 and masked
    "time_pad_3d": _prob("time_pad_3d", 1, 2, 3, (3, 4, 6), (4, 4, 6), (2, 2, 3), (1, 1, 1)),
    # every axis cyclic, explicit scale
    "all_cyclic": _prob("all_cyclic", 1, 1, 5, (1, 6, 8), (1, 6, 8), (1, 3, 4), (0, 1, 2), (1, 1, 1),
                        scale=0.3),
}


def _inputs(p, seed=0):
    """Inputs on a grid of 2^-8, so that they and the finite-difference steps
    below are exact in the float32 the C oracle reads."""
    rng = np.random.default_rng(seed)
    shape = (p.batch,) + tuple(p.extent) + (p.heads, p.head_dim)
    q, k, v, dout = (np.round(rng.standard_normal(shape) * 256) / 256 for _ in range(4))
    table = np.round(0.5 * rng.standard_normal(p.table_shape) * 256) / 256
    return q, k, v, table, dout


def _loss(p, q, k, v, table, dout):
    """sum(dout * O) with O from the C direct form (independent of the literal form)."""
    out, _ = oracle.direct_forward(p, q, k, v, table)
    return float((out * dout).sum())


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_central_differences(name):
    p = CASES[name]
    q, k, v, table, dout = _inputs(p)
    dq, dk, dv, dtable = oracle.literal_backward(p, q, k, v, table, dout)
    rng = np.random.default_rng(1)
    args = [q, k, v, table]
    grads = [dq, dk, dv, dtable]

    def central(i, u, eps):
        plus, minus = list(args), list(args)
        plus[i] = args[i] + eps * u
        minus[i] = args[i] - eps * u
        return (_loss(p, *plus, dout) - _loss(p, *minus, dout)) / (2 * eps)

    for i in range(4):
        for _ in range(2):
            u = rng.choice([-1.0, 1.0], size=args[i].shape)  # steps of 2^-12, 2^-11: exact
            # Richardson: the eps^2 error term of the central difference cancels
            fd = (4 * central(i, u, 2.0 ** -12) - central(i, u, 2.0 ** -11)) / 3
            an = float((grads[i] * u).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, i, fd, an)


def test_single_global_window_matches_torch_autograd():
    """Shift 0 and one window spanning the grid: plain dense attention with an
    additive bias read from the table, differentiated by torch in fp64."""
    p = _prob("global", 1, 2, 4, (1, 3, 4), (1, 3, 4), (1, 3, 4), (0, 0, 0))
    q, k, v, table, dout = _inputs(p, seed=3)
    N, H, d = 12, p.heads, p.head_dim
    tq, tk, tv = (torch.tensor(a.reshape(N, H, d), requires_grad=True) for a in (q, k, v))
    tt = torch.tensor(table, requires_grad=True)
    ys, xs = np.meshgrid(np.arange(3), np.arange(4), indexing="ij")
    ys, xs = ys.ravel(), xs.ravel()
    iy = torch.tensor(ys[:, None] - ys[None, :] + 2)
    ix = torch.tensor(xs[:, None] - xs[None, :] + 3)
    bias = tt[0, iy, ix, :].permute(2, 0, 1)  # [H, N, N]
    logits = torch.einsum("nhe,mhe->hnm", tq, tk) / np.sqrt(d) + bias
    o = torch.einsum("hnm,mhe->nhe", torch.softmax(logits, dim=-1), tv)
    (o * torch.tensor(dout.reshape(N, H, d))).sum().backward()
    dq, dk, dv, dtable = oracle.literal_backward(p, q, k, v, table, dout)
    np.testing.assert_allclose(dq.reshape(N, H, d), tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk.reshape(N, H, d), tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv.reshape(N, H, d), tv.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dtable, tt.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", list(CASES))
def test_table_gradient_sums_to_zero_per_head(name):
    """Each query's dS row sums to zero (sum_m P (dP - D) = D - D), so the table
    gradient of every head sums to zero."""
    p = CASES[name]
    *_, dtable = oracle.literal_backward(p, *_inputs(p, seed=5))
    sums = dtable.reshape(-1, p.heads).sum(axis=0)
    assert np.abs(sums).max() <= 1e-12 * max(1.0, np.abs(dtable).max())


def test_window_subsets_partition_the_gradients():
    p = CASES["ragged_2d"]
    args = _inputs(p, seed=7)
    full = oracle.literal_backward(p, *args)
    nW = p.batch * int(np.prod([p.padded[a] // p.window[a] for a in range(3)]))
    halves = [list(range(0, nW, 2)), list(range(1, nW, 2))]
    parts = [oracle.literal_backward(p, *args, windows=w) for w in halves]
    # token -> window (batch item b's windows follow batch item b - 1's)
    win = oracle.token_windows(p)
    per_b = nW // p.batch
    for i in range(3):
        for b in range(p.batch):
            for part, w in zip(parts, halves):
                mine = np.isin(win + b * per_b, w)
                np.testing.assert_array_equal(part[i][b][mine], full[i][b][mine])
                assert not part[i][b][~mine].any()
    np.testing.assert_allclose(parts[0][3] + parts[1][3], full[3], rtol=0, atol=1e-12)
