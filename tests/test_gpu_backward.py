"""GPU parity of the backward pass (swa_backward) against the fp64 oracle.

Gradients dq, dk, dv and the bias-table gradient are compared element by
element with the oracle's per-window backward, with the forward's metric:
max|G_gpu - G_ref| / max|G_ref| <= 1e-2 for bf16 and <= 1e-5 for fp32.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, host_f32, rel_err
from oracle_pool import pooled_backward_errors
from shifted_window_attention_cyclic_amd import SwaError, WindowAttention
from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, Problem, make_inputs
from test_gpu_parity import EDGE, LARGE, SMALL

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _dout(p, seed=11):
    g = torch.Generator().manual_seed(seed)
    dt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    return torch.randn((p.batch,) + tuple(p.extent) + (p.heads, p.head_dim), generator=g).to(dt)


def _run(p, x, dout):
    att = WindowAttention(p)
    d = {n: t.cuda() for n, t in x.items()}
    grads = att.backward(d["q"], d["k"], d["v"], d["table"], dout.cuda())
    torch.cuda.synchronize()
    att.close()
    return grads


def _takes_backward(p):
    att = WindowAttention(p)
    ok = att.info.backward_workspace_bytes > 0
    att.close()
    return ok


CASES = {**SMALL, **EDGE, **LARGE,
         # the big-window kernels with two batch items and a padded, masked latitude
         "b2_n288_3d_pad": Problem("b2n288", "bf16", 2, 3, 64, (2, 20, 24), (2, 24, 24), (2, 12, 12), (1, 6, 6),
                                   seed=31),
         # 16 x 20 windows (320 tokens, 5 blocks of 4 query waves with no idle slot;
         # a width of 20 splits diagonal runs at window rows), latitude padded 30 -> 32
         "n320_w20_pad": Problem("n320", "bf16", 1, 2, 64, (1, 30, 40), (1, 32, 40), (1, 16, 20), (0, 8, 10),
                                 seed=32),
         # the narrowest width whose diagonal runs split at row starts only (8), and a
         # narrower one (5), whose runs split wherever the table entry changes
         "n192_w8": Problem("n192w8", "bf16", 1, 2, 64, (1, 48, 24), (1, 48, 24), (1, 24, 8), (0, 12, 4), seed=33),
         "n200_w5": Problem("n200w5", "bf16", 1, 2, 64, (1, 40, 20), (1, 40, 20), (1, 40, 5), (0, 20, 2), seed=34),
         # 32-wide heads in 160-token windows (the persistent key kernel's 32-wide
         # variant: 5 query blocks, key groups of 4, 4 and 2 tiles), masked latitude
         "n160_d32": Problem("n160d32", "bf16", 1, 4, 32, (1, 40, 48), (1, 40, 48), (1, 10, 16), (0, 5, 8),
                             seed=35)}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_small_grid(name):
    p = CASES[name]
    if not _takes_backward(p):
        pytest.skip("the backward kernels do not take this window")
    say(f"[backward] {name} dtype={p.dtype} grid={p.extent} pad={p.padded} win={p.window} "
        f"shift={p.shift} heads={p.heads}x{p.head_dim}")
    x = make_inputs(p)
    dout = _dout(p)
    got = _run(p, x, dout)
    ref = oracle.literal_backward(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                  host_f32(x["table"]), host_f32(dout))
    for gname, g_gpu, g_ref in zip(("dq", "dk", "dv", "dtable"), got, ref):
        err = rel_err(host_f32(g_gpu), g_ref)
        say(f"  {gname}: rel err {err:.3e}")
        assert err <= TOL[p.dtype], gname
        assert torch.isfinite(g_gpu.float()).all(), gname


@pytest.mark.parametrize("name", ["c3_bf16_540x1080", "c4_bf16_181x360_pad190", "c5_bf16_4x180x360_3d",
                                  "c6_bf16_180x360_pad184_d128"])
def test_backward_full_size_every_window(name):
    """The workload at its full size: dq, dk, dv of every token and the table
    gradient (a sum over every window and batch item) against the oracle's
    per-window backward over all windows, split across host processes."""
    p = WORKLOADS[name]
    x = make_inputs(p)
    dout = _dout(p)
    got = _run(p, x, dout)
    say(f"[backward full] {name}: {p.windows} windows")
    host = {n: host_f32(x[n]) for n in ("q", "k", "v", "table")}
    host["dout"] = host_f32(dout)
    errs = pooled_backward_errors(p, host, [host_f32(g) for g in got])
    for gname in ("dq", "dk", "dv", "dtable"):
        say(f"  {gname}: rel err {errs[gname]:.3e}")
        assert errs[gname] <= TOL["bf16"], gname
    for g in got:
        assert torch.isfinite(g.float()).all()


def test_backward_full_size_table_gradient():
    """180x360 at full size: the table gradient (a sum over every window) and
    all token gradients against the oracle over all 450 windows."""
    p = WORKLOADS["c2_bf16_180x360"]
    x = make_inputs(p)
    dout = _dout(p)
    got = _run(p, x, dout)
    ref = oracle.literal_backward(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                  host_f32(x["table"]), host_f32(dout))
    for gname, g_gpu, g_ref in zip(("dq", "dk", "dv", "dtable"), got, ref):
        err = rel_err(host_f32(g_gpu), g_ref)
        say(f"  {gname}: rel err {err:.3e}")
        assert err <= TOL["bf16"], gname


def test_backward_is_bitwise_reproducible():
    """Every sum, the table gradient's included, runs in a fixed order."""
    p = WORKLOADS["c4_bf16_181x360_pad190"]
    x = make_inputs(p)
    dout = _dout(p)
    a = _run(p, x, dout)
    b = _run(p, x, dout)
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


@pytest.mark.parametrize("name", ["b2_n288_3d_pad", "n200_w5"])
def test_backward_big_windows_bitwise_reproducible(name):
    """The persistent big-window key kernel sums the table gradient per pair
    over windows, then per entry, each in a fixed order: two runs agree bit for
    bit (b2_n288_3d_pad: more runs of windows than windows, one window per
    workgroup; n200_w5: 7 query blocks, a last key group of 2 tiles)."""
    p = CASES[name]
    att = WindowAttention(p)
    assert att.info.backward_workgroups > 0
    att.close()
    x = make_inputs(p)
    dout = _dout(p)
    a = _run(p, x, dout)
    b = _run(p, x, dout)
    for gname, ga, gb in zip(("dq", "dk", "dv", "dtable"), a, b):
        assert torch.equal(ga, gb), gname


@pytest.mark.parametrize("name", ["c7_bf16_180x384_pad192_d128_w32"])
def test_backward_big_windows_full_size_sampled(name):
    """The 32x32-window kernels at full size (each window takes the fp64 oracle
    over a minute): every token's gradients in a few sampled windows (first,
    last, latitude wrap)."""
    p = WORKLOADS[name]
    x = make_inputs(p)
    dout = _dout(p)
    dq, dk, dv, dtable = _run(p, x, dout)
    nw = p.windows // p.batch
    wins = sorted({0, nw // 2 + 1, nw - 1})
    say(f"[backward big {name}] windows {wins}")
    ref = oracle.literal_backward(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                  host_f32(x["table"]), host_f32(dout), windows=wins)
    mine = np.isin(oracle.token_windows(p), wins)[None]
    for gname, g_gpu, g_ref in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        err = rel_err(host_f32(g_gpu)[mine], g_ref[mine])
        say(f"  {gname}: rel err {err:.3e} over {int(mine.sum())} tokens")
        assert err <= TOL["bf16"], gname
    for g in (dq, dk, dv, dtable):
        assert torch.isfinite(g.float()).all()


@pytest.mark.parametrize("name,schedule", [("c3_bf16_540x1080", 1), ("c6_bf16_180x360_pad184_d128", 1),
                                           ("c5_bf16_4x180x360_3d", 2), ("c7_bf16_180x384_pad192_d128_w32", 2),
                                           ("c1_f32_16x32", 1)])
def test_backward_schedule_reported(name, schedule):
    att = WindowAttention(WORKLOADS[name])
    assert att.info.backward_schedule == schedule
    assert att.info.backward_workspace_bytes > 0
    # bf16 schedule 1 runs persistent workgroups, a whole number per XCD; so
    # does the big-window key kernel for 2x12x12 windows (288 tokens, 64-wide
    # heads): heads * 5 key groups * runs of windows, about one per CU.  The fp32
    # kernel and 32x32 windows take one workgroup per unit or block.
    p = WORKLOADS[name]
    wg = att.info.backward_workgroups
    if schedule == 1 and p.dtype == "bf16":
        assert wg > 0 and wg % 8 == 0
    elif name == "c5_bf16_4x180x360_3d":
        assert wg == p.heads * 5 * (256 // (p.heads * 5))
    else:
        assert wg == 0
    att.close()


def test_backward_rejects_windows_it_does_not_take():
    # fp32 keeps whole windows in LDS: 16 x 16 windows do not fit
    p = Problem("f32big", "f32", 1, 2, 32, (1, 32, 32), (1, 32, 32), (1, 16, 16), (0, 8, 8), seed=3)
    att = WindowAttention(p)
    assert att.info.backward_workspace_bytes == 0
    assert att.info.backward_schedule == 0
    x = {n: t.cuda() for n, t in make_inputs(p).items()}
    with pytest.raises(SwaError):
        att.backward(x["q"], x["k"], x["v"], x["table"], torch.zeros_like(x["q"]))
    att.close()
