"""GPU parity of the HIP library against the fp64 oracle (MI355X only).

Everything goes through the C ABI (libswa.so via the ctypes binding).
Floating-point outputs are compared with the relative max-abs error
max|O_gpu - O_ref| / max|O_ref|: <= 1e-5 for fp32, <= 1e-2 for bf16.
Window routes (gather/scatter) and masks are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, device_inputs, host_f32, oracle_at, oracle_full, rel_err, sample_tokens
from shifted_window_attention_cyclic_amd import WindowAttention
from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, Problem, make_inputs, small_variant

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run(p, d, variant="fused", schedule="auto"):
    att = WindowAttention(p, variant, schedule)
    out = att.forward(d["q"], d["k"], d["v"], d["table"])
    torch.cuda.synchronize()
    att.close()
    return out


SMALL = {
    "c1": WORKLOADS["c1_f32_16x32"],
    "c2s": small_variant(WORKLOADS["c2_bf16_180x360"], 36, 48),
    "c3s": small_variant(WORKLOADS["c3_bf16_540x1080"], 36, 48),
    "c4s": WORKLOADS["c4_bf16_181x360_pad190"].with_(name="c4s", extent=(1, 31, 40), padded=(1, 40, 40)),
    "c5s": small_variant(WORKLOADS["c5_bf16_4x180x360_3d"], 24, 36),
    "c6s": small_variant(WORKLOADS["c6_bf16_180x360_pad184_d128"], 36, 48),
}


def _edge(name, dtype, batch, heads, d, extent, padded, window, shift, cyclic=(0, 0, 1), seed=5):
    return Problem(name, dtype, batch, heads, d, extent, padded, window, shift, cyclic, seed=seed)


EDGE = {
    "n35_ragged_tiles": _edge("n35", "bf16", 2, 3, 64, (1, 13, 21), (1, 15, 21), (1, 5, 7), (0, 2, 3)),
    "global_window_shift0": _edge("global", "bf16", 1, 2, 64, (1, 12, 12), (1, 12, 12), (1, 12, 12), (0, 0, 0)),
    "all_axes_masked": _edge("masked", "bf16", 1, 4, 32, (1, 24, 24), (1, 24, 24), (1, 8, 8), (0, 4, 4), (0, 0, 0)),
    "lat_cyclic_too": _edge("latcyc", "bf16", 1, 4, 32, (1, 24, 24), (1, 24, 24), (1, 8, 8), (0, 4, 4), (0, 1, 1)),
    "shift_not_half": _edge("s3", "bf16", 1, 2, 64, (1, 20, 30), (1, 20, 30), (1, 10, 10), (0, 3, 7)),
    "d32_n288_3d": _edge("d32n288", "bf16", 1, 3, 32, (4, 24, 24), (4, 24, 24), (2, 12, 12), (1, 6, 6)),
    # 32-wide heads, an even head count: 7-tile windows, width 10 (no 4-key bias runs), latitude padded
    "d32_n100_pad": _edge("d32p100", "bf16", 2, 4, 32, (1, 17, 30), (1, 20, 30), (1, 10, 10), (0, 5, 5)),
    # and an odd head count
    "d32_odd_heads": _edge("d32odd", "bf16", 1, 5, 32, (1, 24, 36), (1, 24, 36), (1, 12, 12), (0, 6, 6)),
    "n512_3d_pad": _edge("n512", "bf16", 1, 2, 64, (3, 16, 32), (4, 16, 32), (2, 16, 16), (1, 8, 8)),
    "time_pad": _edge("tpad", "bf16", 2, 2, 64, (3, 12, 24), (4, 12, 24), (2, 6, 6), (1, 3, 3)),
    "f32_d64_3d_pad": _edge("f32d64", "f32", 2, 2, 64, (3, 10, 16), (4, 12, 16), (2, 4, 8), (1, 2, 4)),
    "f32_n288": _edge("f32n288", "f32", 1, 2, 32, (2, 12, 12), (2, 12, 12), (2, 12, 12), (1, 6, 6)),
    # 128-wide heads: 5 tiles with a window width that is no multiple of 4 (general
    # streaming variant), 9 tiles (per-unit schedule: the streaming ring does not
    # fit the LDS) and 18 tiles in 3-D
    "d128_n80_ragged": _edge("d128n80", "bf16", 2, 3, 128, (1, 19, 30), (1, 24, 30), (1, 8, 10), (0, 4, 5)),
    "d128_n144": _edge("d128n144", "bf16", 1, 2, 128, (1, 24, 36), (1, 24, 36), (1, 12, 12), (0, 6, 6)),
    "d128_n288_3d": _edge("d128n288", "bf16", 1, 2, 128, (2, 12, 24), (2, 12, 24), (2, 12, 12), (1, 6, 6)),
}


# windows of more than 512 tokens: only the key-blocked schedule takes them
LARGE = {
    # TERRA Table V's Large-model window (32 x 32, 128-wide heads), latitude padded 40 -> 64
    "n1024_d128_pad": _edge("n1024", "bf16", 1, 2, 128, (1, 40, 64), (1, 64, 64), (1, 32, 32), (0, 16, 16)),
    "n1024_d64": _edge("n1024d64", "bf16", 1, 3, 64, (1, 64, 64), (1, 64, 64), (1, 32, 32), (0, 16, 16)),
    # 540 keys (a ragged last key block), 3 query blocks, window width 27 (no 4-key bias runs)
    "n540_ragged": _edge("n540", "bf16", 1, 2, 64, (1, 36, 54), (1, 40, 54), (1, 20, 27), (0, 10, 13)),
    # 3-D, time padded 5 -> 6 and masked, 32-wide heads
    "n768_3d_d32": _edge("n768", "bf16", 1, 3, 32, (5, 16, 32), (6, 16, 32), (3, 16, 16), (1, 8, 8)),
}


@pytest.mark.parametrize("name", list(SMALL) + list(EDGE) + list(LARGE))
@pytest.mark.parametrize("variant,schedule", [("fused", "auto"), ("staged", "auto"), ("fused", "block"),
                                              ("fused", "keyblock")])
def test_parity_small_full_grid(name, variant, schedule):
    p = SMALL.get(name) or EDGE.get(name) or LARGE[name]
    if schedule == "block" and p.window_tokens > 512:
        pytest.skip("the per-unit schedule takes windows of at most 512 tokens")
    say(f"[parity] {name} {variant} {schedule} dtype={p.dtype} B={p.batch} grid={p.extent} pad={p.padded} "
        f"win={p.window} shift={p.shift} heads={p.heads}x{p.head_dim} seed={p.seed}")
    x, d = device_inputs(p)
    out = run(p, d, variant, schedule)
    ref = oracle_full(p, x)
    err = rel_err(host_f32(out), ref)
    say(f"  rel err {err:.3e}")
    assert err <= TOL[p.dtype]
    assert torch.isfinite(out.float()).all()


FULL = ["c2_bf16_180x360", "c3_bf16_540x1080", "c4_bf16_181x360_pad190", "c5_bf16_4x180x360_3d",
        "c6_bf16_180x360_pad184_d128", "c7_bf16_180x384_pad192_d128_w32"]


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size_sampled(name):
    """The workload at its full size, in the launch configuration the benchmark
    times; the oracle evaluates a sample that covers every window edge class."""
    p = WORKLOADS[name]
    say(f"[full] {name} seed={p.seed}")
    x, d = device_inputs(p)
    out = run(p, d, "fused")
    idx = sample_tokens(p, count=512)
    ref = oracle_at(p, x, idx)
    got = host_f32(out).reshape(p.tokens, p.heads, p.head_dim)[idx]
    err = rel_err(got, ref)
    say(f"  {len(idx)} tokens, rel err {err:.3e}")
    assert err <= TOL[p.dtype]
    assert torch.isfinite(out.float()).all()
    # the staged variant runs the same attention arithmetic on window-major copies
    out2 = run(p, d, "staged")
    assert torch.equal(out, out2)
    del out2
    if p.window_tokens <= 512:
        # the per-window-block schedule computes the same sums in the same order
        out3 = run(p, d, "fused", "block")
        assert torch.equal(out, out3)
        del out3
        # the key-blocked schedule sums in blocks of 32 keys: within tolerance of the oracle
        out4 = run(p, d, "fused", "keyblock")
        got4 = host_f32(out4).reshape(p.tokens, p.heads, p.head_dim)[idx]
        err4 = rel_err(got4, ref)
        say(f"  key-blocked schedule: rel err {err4:.3e}")
        assert err4 <= TOL[p.dtype]


@pytest.mark.parametrize("name", ["c2_bf16_180x360", "c3_bf16_540x1080", "c4_bf16_181x360_pad190",
                                  "c5_bf16_4x180x360_3d", "c6_bf16_180x360_pad184_d128"])
def test_parity_full_grid_every_token(name):
    """The workload at its full size, in the launch configuration the benchmark
    times: every real token and head against the oracle's direct form (C,
    OpenMP over the host cores)."""
    p = WORKLOADS[name]
    say(f"[full grid] {name} seed={p.seed}")
    x, d = device_inputs(p)
    out = run(p, d, "fused")
    del d
    ref = oracle_full(p, x)
    err = rel_err(host_f32(out), ref)
    say(f"  {p.tokens} tokens x {p.heads} heads, rel err {err:.3e}")
    assert err <= TOL[p.dtype]
    assert torch.isfinite(out.float()).all()


def test_batch_past_2gib_keeps_the_streaming_schedule():
    """540x1080 with a batch of 4 (2.39 GB per tensor): the streaming schedule
    still takes it (its O stores address each batch item from that item's
    start), sampled tokens of every batch item match the oracle, and every
    token of the last batch item does."""
    p = WORKLOADS["c3b4_bf16_540x1080"]
    x, d = device_inputs(p)
    att = WindowAttention(p)
    assert att.info.schedule == 1  # SWA_SCHEDULE_STREAM
    out = att.forward(d["q"], d["k"], d["v"], d["table"])
    torch.cuda.synchronize()
    att.close()
    del d
    per = p.tokens // p.batch
    idx = np.concatenate([sample_tokens(p.with_(batch=1), count=128) + b * per for b in range(p.batch)])
    ref = oracle_at(p, x, idx)
    got = host_f32(out).reshape(p.tokens, p.heads, p.head_dim)[idx]
    err = rel_err(got, ref)
    say(f"[batch 4] {idx.size} sampled tokens, rel err {err:.3e}")
    assert err <= TOL["bf16"]
    last = np.arange((p.batch - 1) * per, p.batch * per)
    ref = oracle_at(p, x, last)
    err = rel_err(host_f32(out).reshape(p.tokens, p.heads, p.head_dim)[last], ref)
    say(f"  last batch item, every token: rel err {err:.3e}")
    assert err <= TOL["bf16"]
    assert torch.isfinite(out.float()).all()


def test_fp32_full_workload_matches_oracle_everywhere():
    p = WORKLOADS["c1_f32_16x32"]
    x, d = device_inputs(p)
    for variant in ("fused", "staged"):
        out = run(p, d, variant)
        assert rel_err(host_f32(out), oracle_full(p, x)) <= 1e-5


@pytest.mark.parametrize("name", list(SMALL) + ["n35_ragged_tiles", "n512_3d_pad", "time_pad"])
def test_gather_scatter_bit_exact(name):
    p = SMALL.get(name) or EDGE[name]
    say(f"[route] {name}")
    x, d = device_inputs(p)
    att = WindowAttention(p)
    wm = att.gather(d["q"])
    torch.cuda.synchronize()
    want = oracle.literal_windows(p, host_f32(x["q"]))  # [B, nW, N, h, d], pad slots zero
    assert np.array_equal(host_f32(wm).astype(np.float64), want.reshape(wm.shape))
    back = att.scatter(wm)
    torch.cuda.synchronize()
    assert torch.equal(back, d["q"])
    # scatter of the oracle's window tensor gives the oracle's un-windowed tensor
    src = torch.from_numpy(want.reshape(wm.shape)).to(d["q"].dtype).cuda()
    back2 = att.scatter(src)
    torch.cuda.synchronize()
    assert np.array_equal(host_f32(back2).astype(np.float64),
                          oracle.literal_unwindows(p, want))
    att.close()


def _check_windows(p, att, windows):
    vis = oracle.literal_visibility(p)  # [nW per batch item, N, N]
    nW = vis.shape[0]
    for w in windows:
        got = att.visibility(int(w)).cpu().numpy().astype(bool)
        assert np.array_equal(got, vis[int(w) % nW]), (p.name, w)


@pytest.mark.parametrize("name", list(SMALL) + ["n35_ragged_tiles", "all_axes_masked", "lat_cyclic_too",
                                                "time_pad", "shift_not_half"])
def test_visibility_all_windows_bit_exact(name):
    p = SMALL.get(name) or EDGE[name]
    att = WindowAttention(p)
    _check_windows(p, att, range(att.info.windows))
    att.close()


@pytest.mark.parametrize("name", FULL)
def test_visibility_full_size_edge_windows(name):
    p = WORKLOADS[name]
    att = WindowAttention(p)
    nw = [p.padded[a] // p.window[a] for a in range(3)]
    per = nw[0] * nw[1] * nw[2]
    picks = set()
    for t in {0, nw[0] - 1}:
        for y in {0, 1, nw[1] // 2, nw[1] - 2, nw[1] - 1}:
            for xx in {0, 1, nw[2] // 2, nw[2] - 1}:
                picks.add((t * nw[1] + y) * nw[2] + xx)
    picks |= {per * (p.batch - 1) + w for w in list(picks)}
    _check_windows(p, att, sorted(picks))
    att.close()


def test_determinism_bitwise():
    p = WORKLOADS["c4_bf16_181x360_pad190"]
    x, d = device_inputs(p)
    a = run(p, d)
    b = run(p, d)
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["c1", "c4s", "c5s"])
def test_per_window_independence(name):
    """Perturb every token of one shifted window: all other outputs stay bit-identical."""
    p = SMALL[name]
    x, d = device_inputs(p)
    base = run(p, d)
    att = WindowAttention(p)
    wm_mask = torch.zeros(att.window_major_shape, dtype=p.dtype == "f32" and torch.float32 or torch.bfloat16,
                          device="cuda")
    widx = att.info.windows // 2 + 1
    wm_mask[widx] = 1.0
    inside = att.scatter(wm_mask)  # 1 on the tokens of that window, 0 elsewhere
    torch.cuda.synchronize()
    att.close()
    d2 = dict(d)
    for n in ("q", "k", "v"):
        d2[n] = d[n] + 2.0 * inside
    pert = run(p, d2)
    sel = inside[..., 0, 0] > 0
    assert sel.any()
    assert torch.equal(pert[~sel], base[~sel])
    assert not torch.equal(pert[sel], base[sel])


def test_mask_isolates_wrapped_rows_on_gpu():
    """Ragged grid: latitude rows 0..4 share a rolled window with pad rows only
    (and rows 175..180 of the window before); changing K/V of every other row
    leaves rows 0..4 bit-identical, and vice versa."""
    p = WORKLOADS["c4_bf16_181x360_pad190"].with_(batch=1, heads=2, extent=(1, 181, 40), padded=(1, 190, 40))
    x, d = device_inputs(p)
    base = run(p, d)
    d2 = dict(d)
    d2["k"] = d["k"].clone()
    d2["v"] = d["v"].clone()
    d2["k"][:, :, 5:] *= -2
    d2["v"][:, :, 5:] += 1
    pert = run(p, d2)
    assert torch.equal(pert[:, :, :5], base[:, :, :5])
    d3 = dict(d)
    d3["v"] = d["v"].clone()
    d3["v"][:, :, :5] += 1
    pert3 = run(p, d3)
    assert torch.equal(pert3[:, :, 5:], base[:, :, 5:])
    assert not torch.equal(pert3[:, :, :5], base[:, :, :5])


@pytest.mark.parametrize("r", [1, 5, 7])
def test_longitude_translation_equivariance_bitwise(r):
    p = SMALL["c3s"]
    x, d = device_inputs(p)
    base = run(p, d)
    p2 = p.with_(shift=(0, p.shift[1], (p.shift[2] + r) % p.window[2]))
    d2 = {n: (torch.roll(t, shifts=r, dims=3) if n != "table" else t) for n, t in d.items()}
    moved = run(p2, d2)
    assert torch.equal(moved, torch.roll(base, shifts=r, dims=3))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unit_window_returns_v_exactly(dtype):
    p = _edge("unit", dtype, 2, 3, 32, (2, 6, 10), (2, 6, 10), (1, 1, 1), (0, 0, 0))
    x, d = device_inputs(p)
    out = run(p, d)
    assert torch.equal(out, d["v"])


def test_constant_v_gives_constant_output():
    p = SMALL["c5s"]
    x, d = device_inputs(p)
    d["v"] = torch.full_like(d["v"], 0.8125)
    out = run(p, d)
    assert (out.float() - 0.8125).abs().max().item() <= 0.8125 * 2 ** -8


def test_outputs_stay_inside_their_buffer():
    """Canary: guard elements after `out` are never written."""
    p = SMALL["c4s"]
    x, d = device_inputs(p)
    n = int(np.prod(p.io_shape))
    buf = torch.full((n + 4096,), -7.0, dtype=torch.bfloat16, device="cuda")
    att = WindowAttention(p)
    att.forward(d["q"], d["k"], d["v"], d["table"], out=buf[:n].view(p.io_shape))
    torch.cuda.synchronize()
    att.close()
    assert (buf[n:] == -7.0).all()
    assert rel_err(host_f32(buf[:n].view(p.io_shape)), oracle_full(p, x)) <= TOL["bf16"]


def test_explicit_scale():
    p = SMALL["c2s"].with_(scale=0.05)
    x, d = device_inputs(p)
    out = run(p, d)
    assert rel_err(host_f32(out), oracle_full(p, x)) <= TOL["bf16"]


def test_larger_logits_still_match():
    """Q and K at std 3 make logits up to ~100 base units: softmax must subtract the max."""
    p = SMALL["c3s"]
    x = make_inputs(p, qkv_std=3.0)
    d = {n: t.cuda() for n, t in x.items()}
    out = run(p, d)
    assert rel_err(host_f32(out), oracle_full(p, x)) <= TOL["bf16"]


@pytest.mark.gpu
def test_auto_schedule_choice():
    """AUTO takes the streaming schedule for windows of up to 9 query tiles that
    fit its LDS ring, else the per-(window, head) schedule for windows of up to
    512 tokens that fit its LDS, else the key-blocked one."""
    want = {"c2_bf16_180x360": 1, "c3_bf16_540x1080": 1, "c4_bf16_181x360_pad190": 1,
            "c5_bf16_4x180x360_3d": 2, "c6_bf16_180x360_pad184_d128": 1, "c7_bf16_180x384_pad192_d128_w32": 3}
    small = {"d128_n80_ragged": 1, "d128_n144": 2, "d128_n288_3d": 2, "n1024_d128_pad": 3, "n540_ragged": 3}
    for name, schedule in small.items():
        att = WindowAttention(EDGE.get(name) or LARGE[name])
        assert att.info.schedule == schedule, name
        att.close()
    for name, schedule in want.items():
        att = WindowAttention(WORKLOADS[name])
        assert att.info.schedule == schedule, name
        assert att.info.workgroups >= 8, name
        att.close()


def test_streaming_workgroups_per_cu():
    """The persistent streaming schedule launches one workgroup per CU, and two
    for the 32-wide 9-tile variant, whose LDS is half a CU's and whose registers
    are held to what two 12-wave workgroups allow: a change that raises its
    register count past that halves its occupancy, and this fails."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_cu = {"c2_bf16_180x360": 2, "c3_bf16_540x1080": 1, "c4_bf16_181x360_pad190": 1,
              "c6_bf16_180x360_pad184_d128": 1}
    for name, n in per_cu.items():
        att = WindowAttention(WORKLOADS[name])
        assert att.info.workgroups == n * cus // 8 * 8, (name, att.info.workgroups, cus)
        att.close()
