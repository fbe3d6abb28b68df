"""swa_backward_noalloc (the backward pass through the library's fixed device
scratch, for callers that cannot allocate) against swa_backward (caller
workspace), both through the C ABI, on two calls in a row where the second
problem is smaller than the first.

dq, dk, dv must match bit for bit (the same kernels compute every unit), and
so must the table gradient of the single-workgroup schedule (its chunk sums
run in swa_backward's order).  The big-window schedule's table gradient is
held to the bf16 tolerance: through the scratch its per-pair sums cover
shorter runs of windows (passes sized to the scratch), which changes the
order of the fp32 additions.  Each pair also checks the no-allocation result against
the fp64 oracle on the smaller problem.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, host_f32, rel_err
from shifted_window_attention_cyclic_amd import WindowAttention, swa_backward, swa_backward_noalloc
from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, Problem, make_inputs, small_variant

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _dout(p, seed=13):
    g = torch.Generator().manual_seed(seed)
    dt = torch.float32 if p.dtype == "f32" else torch.bfloat16
    return torch.randn(p.io_shape, generator=g).to(dt)


def _both(p):
    """(workspace result, no-allocation result, inputs, dout) for problem p."""
    x = make_inputs(p)
    dout = _dout(p)
    d = {n: t.cuda() for n, t in x.items()}
    do = dout.cuda()
    att = WindowAttention(p)
    info = att.info
    assert info.backward_workspace_bytes > 0
    ref = att.backward(d["q"], d["k"], d["v"], d["table"], do)
    got = [torch.full_like(t, float("nan")) for t in ref]  # every element must be written
    swa_backward_noalloc(att.handle, d["q"], d["k"], d["v"], d["table"], do, *got)
    torch.cuda.synchronize()
    schedule = info.backward_schedule
    att.close()
    return ref, got, x, dout, schedule


def _compare(name, ref, got, schedule):
    for gname, a, b in zip(("dq", "dk", "dv"), ref[:3], got[:3]):
        assert torch.equal(a, b), (name, gname)
    if schedule == 1:
        assert torch.equal(ref[3], got[3]), (name, "dtable")
    else:
        err = rel_err(host_f32(got[3]), host_f32(ref[3]))
        say(f"  {name} dtable vs swa_backward: rel err {err:.3e}")
        assert err <= TOL["bf16"], (name, "dtable")


PAIRS = {
    # 4,050 windows: the table shares of 540x1080 (69 MB) take three passes of the
    # 32 MiB scratch; then a small ragged grid in one pass
    "single_workgroup": (WORKLOADS["c3_bf16_540x1080"],
                         small_variant(WORKLOADS["c4_bf16_181x360_pad190"], 31, 40)),
    # 2x12x12 windows (big-window kernels, per-query statistics in the scratch too):
    # 900 windows of 12 heads (93 MB, three passes), then a small padded 3-D grid
    "big_windows": (WORKLOADS["c5_bf16_4x180x360_3d"],
                    Problem("b2n288", "bf16", 2, 3, 64, (2, 20, 24), (2, 24, 24), (2, 12, 12), (1, 6, 6),
                            seed=31)),
    # fp32: the 16x32 grid, then a smaller 3-D padded one
    "f32": (WORKLOADS["c1_f32_16x32"],
            Problem("f32d64", "f32", 1, 2, 32, (3, 10, 16), (4, 12, 16), (2, 4, 8), (1, 2, 4), seed=5)),
}


@pytest.mark.parametrize("pair", list(PAIRS))
def test_noalloc_backward_matches_workspace_backward(pair):
    first, second = PAIRS[pair]
    assert second.tokens < first.tokens
    for p in (first, second):
        say(f"[noalloc] {pair}: {p.name} grid={p.extent} pad={p.padded} win={p.window} heads={p.heads}x{p.head_dim}")
        ref, got, x, dout, schedule = _both(p)
        _compare(p.name, ref, got, schedule)
    # the second (smaller) call against the oracle as well
    want = oracle.literal_backward(second, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                   host_f32(x["table"]), host_f32(dout))
    for gname, g, r in zip(("dq", "dk", "dv", "dtable"), got, want):
        err = rel_err(host_f32(g), r)
        say(f"  {second.name} {gname} vs oracle: rel err {err:.3e}")
        assert err <= TOL[second.dtype], gname


def test_noalloc_backward_refuses_what_swa_backward_refuses():
    # fp32 keeps whole windows in LDS: 16 x 16 windows do not fit either entry
    p = Problem("f32big", "f32", 1, 2, 32, (1, 32, 32), (1, 32, 32), (1, 16, 16), (0, 8, 8), seed=3)
    att = WindowAttention(p)
    x = {n: t.cuda() for n, t in make_inputs(p).items()}
    grads = [torch.empty_like(x[n]) for n in ("q", "k", "v", "table")]
    with pytest.raises(Exception):
        swa_backward_noalloc(att.handle, x["q"], x["k"], x["v"], x["table"], torch.zeros_like(x["q"]), *grads)
    att.close()
