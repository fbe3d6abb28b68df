"""GPU checks of the forward pass's softmax statistics (swa_forward_lse) and of
the backward pass that reuses them (swa_backward_lse).

The log-sum-exp of each real query is compared with the oracle's literal
form, absolute error <= 1e-2 for bf16 (the kernels sum bf16-rounded softmax
terms) and <= 1e-5 for fp32; the output beside it must equal swa_forward's
bit for bit.  The gradients of swa_backward_lse are compared with the
oracle's backward with the forward's metric (max|G - G_ref| / max|G_ref|).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, host_f32, rel_err
from oracle_pool import pooled_backward_errors
from shifted_window_attention_cyclic_amd import SwaError, WindowAttention
from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, Problem, make_inputs
from test_gpu_backward import CASES, _dout
from test_gpu_parity import EDGE, LARGE, SMALL

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)


def _device(x):
    return {n: t.cuda() for n, t in x.items()}


@pytest.mark.parametrize("name", list(SMALL) + list(EDGE) + list(LARGE))
def test_forward_lse_matches_oracle(name):
    p = SMALL.get(name) or EDGE.get(name) or LARGE[name]
    say(f"[lse] {name} dtype={p.dtype} grid={p.extent} pad={p.padded} win={p.window} heads={p.heads}x{p.head_dim}")
    x = make_inputs(p)
    d = _device(x)
    att = WindowAttention(p)
    ref_out = att.forward(d["q"], d["k"], d["v"], d["table"])
    out, lse = att.forward_lse(d["q"], d["k"], d["v"], d["table"])
    torch.cuda.synchronize()
    say(f"  schedule {att.info.schedule}")
    att.close()
    assert torch.equal(out, ref_out)
    want = oracle.literal_lse(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["table"]))
    err = float(np.abs(lse.cpu().double().numpy() - want).max())
    say(f"  lse max abs err {err:.3e}")
    assert err <= LSE_TOL[p.dtype]


@pytest.mark.parametrize("schedule", ["stream", "block", "keyblock"])
def test_forward_lse_every_schedule(schedule):
    p = SMALL["c3s"]
    x = make_inputs(p)
    d = _device(x)
    att = WindowAttention(p, "fused", schedule)
    out, lse = att.forward_lse(d["q"], d["k"], d["v"], d["table"])
    torch.cuda.synchronize()
    att.close()
    want = oracle.literal_lse(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["table"]))
    err = float(np.abs(lse.cpu().double().numpy() - want).max())
    say(f"[lse {schedule}] max abs err {err:.3e}")
    assert err <= LSE_TOL["bf16"]


def test_forward_lse_refuses_the_staged_variant():
    p = SMALL["c3s"]
    d = _device(make_inputs(p))
    att = WindowAttention(p, "staged")
    with pytest.raises(SwaError):
        att.forward_lse(d["q"], d["k"], d["v"], d["table"])
    att.close()


def _backward_both(p, x, dout):
    d = _device(x)
    att = WindowAttention(p)
    out, lse = att.forward_lse(d["q"], d["k"], d["v"], d["table"])
    g_lse = att.backward_lse(d["q"], d["k"], d["v"], d["table"], out, lse, dout.cuda())
    g_ref = att.backward(d["q"], d["k"], d["v"], d["table"], dout.cuda())
    torch.cuda.synchronize()
    sched = att.info.backward_schedule
    att.close()
    return g_lse, g_ref, sched


@pytest.mark.parametrize("name", list(CASES))
def test_backward_lse_matches_oracle(name):
    p = CASES[name]
    att = WindowAttention(p)
    takes = att.info.backward_workspace_bytes > 0
    att.close()
    if not takes:
        pytest.skip("the backward kernels do not take this window")
    say(f"[backward lse] {name} dtype={p.dtype} grid={p.extent} win={p.window} heads={p.heads}x{p.head_dim}")
    x = make_inputs(p)
    dout = _dout(p)
    g_lse, g_ref, sched = _backward_both(p, x, dout)
    say(f"  backward schedule {sched}")
    if sched == 1:
        # the single-workgroup and fp32 kernels form their own statistics: bitwise equal
        for a, b in zip(g_lse, g_ref):
            assert torch.equal(a, b)
        return
    ref = oracle.literal_backward(p, host_f32(x["q"]), host_f32(x["k"]), host_f32(x["v"]),
                                  host_f32(x["table"]), host_f32(dout))
    for gname, g_gpu, g_want in zip(("dq", "dk", "dv", "dtable"), g_lse, ref):
        err = rel_err(host_f32(g_gpu), g_want)
        say(f"  {gname}: rel err {err:.3e}")
        assert err <= TOL[p.dtype], gname
        assert torch.isfinite(g_gpu.float()).all(), gname


def test_backward_lse_full_size_every_window():
    """4x180x360 with 2x12x12 windows at full size: the gradients from the
    forward's statistics against the oracle's backward over every window."""
    p = WORKLOADS["c5_bf16_4x180x360_3d"]
    x = make_inputs(p)
    dout = _dout(p)
    g_lse, _, sched = _backward_both(p, x, dout)
    assert sched == 2
    host = {n: host_f32(x[n]) for n in ("q", "k", "v", "table")}
    host["dout"] = host_f32(dout)
    errs = pooled_backward_errors(p, host, [host_f32(g) for g in g_lse])
    for gname in ("dq", "dk", "dv", "dtable"):
        say(f"  {gname}: rel err {errs[gname]:.3e}")
        assert errs[gname] <= TOL["bf16"], gname


def test_backward_lse_large_model_sampled():
    """The 32x32 windows of the Large model at full size: gradients from the
    forward's statistics against swa_backward's (themselves checked against
    the oracle on sampled windows), and the table gradient finite."""
    p = WORKLOADS["c7_bf16_180x384_pad192_d128_w32"]
    x = make_inputs(p)
    dout = _dout(p)
    g_lse, g_ref, sched = _backward_both(p, x, dout)
    assert sched == 2
    for gname, a, b in zip(("dq", "dk", "dv", "dtable"), g_lse, g_ref):
        err = rel_err(host_f32(a), host_f32(b))
        say(f"  {gname}: rel diff to swa_backward {err:.3e}")
        assert err <= TOL["bf16"], gname
        assert torch.isfinite(a.float()).all(), gname
