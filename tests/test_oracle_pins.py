"""Pins of the fp64 oracle to facts outside itself (CPU only).

The pages print no worked example, so the oracle is pinned by
  * hand-derived window geometry (tests/golden/segments.json),
  * closed forms (uniform weights, a linear bias table, constant V, unit windows),
  * a library routine on the special case that reduces to it (one window with
    shift 0 is global attention: torch's scaled_dot_product_attention),
  * brute force over hand-derived key sets on tiny grids,
  * invariants (longitude translation equivariance, per-window independence,
    mask isolation), and
  * agreement of its two separately written forms (direct C, literal numpy).
Each is chosen so that a plausible slip in the oracle (wrong roll direction,
mask on the cyclic axis, pad placed at the start, bias sign, scale, missing
max subtraction, wrong window-local coordinate) fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, Problem, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "segments.json")


def P(extent, padded, window, shift, heads=2, head_dim=8, batch=1, cyclic=(0, 0, 1), seed=7,
      scale=None):
    return Problem("t", "f32", batch, heads, head_dim, tuple(extent), tuple(padded),
                   tuple(window), tuple(shift), tuple(cyclic), scale=scale, seed=seed)


def f64(x):
    return x.double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)


def run_direct(oracle_lib, p, x, query_index=None):
    out, _ = oracle_lib.direct_forward(p, f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["table"]),
                                       query_index=query_index)
    return out


def run_literal(oracle_lib, p, x):
    return oracle_lib.literal_forward(p, f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["table"]))


def golden_axes():
    with open(GOLDEN) as f:
        return {a["name"]: a for a in json.load(f)["axes"]}


def expand(first, last, extent):
    out, c = [first], first
    while c != last:
        c = (c + 1) % extent
        out.append(c)
    return out


def axis_problem(ax, axis):
    """A problem whose `axis` is the golden axis and whose other axes are trivial."""
    ext, pad, win, sh, cyc = [1, 1, 1], [1, 1, 1], [1, 1, 1], [0, 0, 0], [0, 0, 1]
    ext[axis], pad[axis], win[axis], sh[axis] = ax["extent"], ax["padded"], ax["window"], ax["shift"]
    cyc[axis] = ax["cyclic"]
    return P(ext, pad, win, sh, cyclic=cyc)


def axis_of(ax):
    return 2 if ax["cyclic"] else (0 if ax["name"].startswith("tiny_time") else 1)


# --------------------------------------------------------------------------- geometry


@pytest.mark.parametrize("name", list(golden_axes()))
def test_segments_match_hand_derivation(oracle_lib, name):
    ax = golden_axes()[name]
    a = axis_of(ax)
    p = axis_problem(ax, a)
    E = ax["extent"]
    if "segments" in ax:
        seg_of = {c: seg for seg in ax["segments"] for c in seg}
    else:
        seg_of = {int(c): expand(f, l, E) for c, (f, l) in ax["segments_of"].items()}
    for c, seg in seg_of.items():
        qc = [0, 0, 0]
        qc[a] = c
        got = []
        for c2 in range(ax["padded"]):
            kc = [0, 0, 0]
            kc[a] = c2
            if oracle_lib.visible(p, qc, kc):
                got.append(c2)
        assert sorted(got) == sorted(seg), (name, c)
    for c, l in ax["local"].items():
        assert oracle_lib.local_coord(p, a, int(c)) == l, (name, c)


@pytest.mark.parametrize("name", ["tiny_lat_pad", "tiny_lon_cyclic", "tiny_time"])
def test_literal_visibility_matches_hand_derivation(oracle_lib, name):
    ax = golden_axes()[name]
    a = axis_of(ax)
    p = axis_problem(ax, a)
    vis = oracle_lib.literal_visibility(p)  # [nW, N, N], windows along axis a
    w, s, Pd = ax["window"], ax["shift"], ax["padded"]
    seg_of = {c: set(seg) for seg in ax["segments"] for c in seg}
    for win in range(Pd // w):
        for n in range(w):
            src_n = (win * w + n + s) % Pd
            for m in range(w):
                src_m = (win * w + m + s) % Pd
                want = src_n in seg_of and src_m in seg_of[src_n]
                assert bool(vis[win, n, m]) == want, (name, win, n, m)


def test_pad_is_at_the_end_and_never_a_key(oracle_lib):
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2))
    for y in range(7):
        assert not oracle_lib.visible(p, (0, y, 0), (0, 7, 0))
    assert oracle_lib.visible(p, (0, 6, 0), (0, 6, 0))


# --------------------------------------------------------------------------- two forms


TINY = [
    P((1, 8, 12), (1, 8, 12), (1, 4, 4), (0, 2, 2)),
    P((1, 8, 12), (1, 8, 12), (1, 4, 4), (0, 0, 0)),
    P((1, 7, 12), (1, 8, 12), (1, 4, 4), (0, 2, 2), batch=2),
    P((1, 13, 15), (1, 15, 15), (1, 5, 5), (0, 3, 1), heads=3, head_dim=4),
    P((1, 6, 9), (1, 6, 9), (1, 6, 3), (0, 5, 2)),
    P((4, 6, 8), (4, 6, 8), (2, 3, 4), (1, 1, 2)),
    P((3, 5, 8), (4, 6, 8), (2, 3, 4), (1, 1, 3), heads=1, head_dim=16),
    P((1, 8, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), cyclic=(0, 1, 1)),
    P((1, 8, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), cyclic=(0, 0, 0)),
]


@pytest.mark.parametrize("i", range(len(TINY)))
def test_literal_equals_direct(oracle_lib, i):
    p = TINY[i]
    x = make_inputs(p, seed=100 + i)
    d = run_direct(oracle_lib, p, x)
    l = run_literal(oracle_lib, p, x)
    assert np.abs(d - l).max() <= 1e-12 * max(1.0, np.abs(l).max())


def test_query_subset_equals_full(oracle_lib):
    p = TINY[5]
    x = make_inputs(p, seed=3)
    full = run_direct(oracle_lib, p, x).reshape(p.tokens, p.heads, p.head_dim)
    idx = np.array([0, 5, 17, p.tokens - 1, 40])
    sub = run_direct(oracle_lib, p, x, query_index=idx)
    assert np.array_equal(sub, full[idx])


# --------------------------------------------------------------------------- library routine


@pytest.mark.parametrize("shape", [((1, 6, 8), (1, 6, 8)), ((2, 3, 4), (2, 3, 4))])
def test_single_window_shift0_is_global_attention(oracle_lib, shape):
    extent, window = shape
    p = P(extent, extent, window, (0, 0, 0), heads=3, head_dim=16, batch=2)
    x = make_inputs(p, seed=11)
    x["table"] = torch.randn(p.table_shape, generator=torch.Generator().manual_seed(5),
                             dtype=torch.float32)
    got = run_direct(oracle_lib, p, x)
    lit = run_literal(oracle_lib, p, x)
    # global attention over all T*H*W tokens with the relative bias of raw coordinate
    # differences, via torch's fused routine in float64 on the CPU
    T, H, W = extent
    coords = torch.stack(torch.meshgrid(torch.arange(T), torch.arange(H), torch.arange(W),
                                        indexing="ij"), -1).reshape(-1, 3)
    rel = coords[:, None, :] - coords[None, :, :] + torch.tensor(window) - 1
    tab = x["table"].double()
    bias = tab[rel[..., 0], rel[..., 1], rel[..., 2]].permute(2, 0, 1)  # [h, n, m]
    n = T * H * W

    def heads_first(a):
        return a.double().reshape(p.batch, n, p.heads, p.head_dim).permute(0, 2, 1, 3)

    ref = torch.nn.functional.scaled_dot_product_attention(
        heads_first(x["q"]), heads_first(x["k"]), heads_first(x["v"]), attn_mask=bias[None],
        scale=1.0 / math.sqrt(p.head_dim))
    ref = ref.permute(0, 2, 1, 3).reshape(got.shape).numpy()
    assert np.abs(got - ref).max() < 1e-12
    assert np.abs(lit - ref).max() < 1e-12


def test_explicit_scale_is_used(oracle_lib):
    p = P((1, 4, 4), (1, 4, 4), (1, 4, 4), (0, 0, 0), heads=1, head_dim=8, scale=0.37)
    x = make_inputs(p, seed=12)
    x["table"].zero_()
    got = run_direct(oracle_lib, p, x)
    q, k, v = (x[n].double().reshape(1, 16, 8) for n in ("q", "k", "v"))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.37)
    assert np.abs(got.reshape(1, 16, 8) - ref.numpy()).max() < 1e-12


# --------------------------------------------------------------------------- closed forms


def test_uniform_weights_give_segment_means_ragged(oracle_lib):
    """Q = 0 and a zero table make every visible key weigh the same: the output
    is the mean of V over the key set, whose size the hand derivation fixes
    (ragged 181 -> 190 latitude, window 10x10, shift 5; longitude 360)."""
    base = WORKLOADS["c4_bf16_181x360_pad190"]
    p = base.with_(dtype="f32", heads=2, head_dim=4, batch=1)
    x = make_inputs(p, seed=21)
    x["q"].zero_()
    x["table"].zero_()
    ax = golden_axes()
    lat = ax["ragged_lat_181_pad190_w10_s5"]["segments_of"]
    lon = ax["lon_360_w10_s5"]["segments_of"]
    cases = [(0, 0), (4, 359), (180, 200), (100, 5), (175, 0)]
    idx = np.array([y * 360 + xx for y, xx in cases])
    got = run_direct(oracle_lib, p, x, query_index=idx)
    v = x["v"].double().numpy()[0, 0]
    for i, (y, xx) in enumerate(cases):
        ys = expand(*lat[str(y)], 181)
        xs = expand(*lon[str(xx)], 360)
        want = v[np.ix_(ys, xs)].reshape(len(ys) * len(xs), 2, 4).mean(axis=0)
        assert np.abs(got[i] - want).max() < 1e-14, (y, xx, len(ys) * len(xs))
    assert [len(expand(*lat[str(y)], 181)) * 10 for y, _ in cases] == [50, 50, 60, 100, 60]


def test_uniform_weights_3d(oracle_lib):
    """Time axis masked: T = 4, window 2, shift 1 splits time into {0}, {1,2}, {3}."""
    p = P((4, 4, 8), (4, 4, 8), (2, 4, 4), (1, 2, 2), heads=1, head_dim=4)
    x = make_inputs(p, seed=22)
    x["q"].zero_()
    x["table"].zero_()
    got = run_direct(oracle_lib, p, x)
    v = x["v"].double().numpy()[0]
    tseg = {0: [0], 1: [1, 2], 2: [1, 2], 3: [3]}
    yseg = {0: [0, 1], 1: [0, 1], 2: [2, 3], 3: [2, 3]}
    xseg = {c: ([2, 3, 4, 5] if 2 <= c <= 5 else [6, 7, 0, 1]) for c in range(8)}
    for t in range(4):
        for y in range(4):
            for xx in range(8):
                want = v[np.ix_(tseg[t], yseg[y], xseg[xx])].reshape(-1, 1, 4).mean(axis=0)
                assert np.abs(got[0, t, y, xx] - want).max() < 1e-14


def test_linear_bias_table_closed_form(oracle_lib):
    """With Q = 0 and table[dy, dx] = a*(dy - (w_y-1)) + b*(dx - (w_x-1)), the logit of
    key j for query i is a*(l_y(i)-l_y(j)) + b*(l_x(i)-l_x(j)); the query part cancels
    in the softmax, so weights are proportional to exp(-a*l_y(j) - b*l_x(j)), with the
    hand-derived window-local coordinates.  Fixes the bias sign (query minus key), the
    use of rolled-window positions, and that the bias is not scaled."""
    ax = golden_axes()
    lat, lon = ax["tiny_lat_pad"], ax["tiny_lon_cyclic"]
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), heads=1, head_dim=4)
    x = make_inputs(p, seed=23)
    x["q"].zero_()
    a, b = 0.7, -0.45
    dy = torch.arange(7, dtype=torch.float64)[:, None] - 3
    dx = torch.arange(7, dtype=torch.float64)[None, :] - 3
    x["table"] = (a * dy + b * dx)[None, :, :, None].float()  # exact in fp32? close enough:
    tab = x["table"].double().numpy()
    got = run_direct(oracle_lib, p, x)
    v = x["v"].double().numpy()[0, 0]
    seg_y = {c: seg for seg in lat["segments"] for c in seg}
    seg_x = {c: seg for seg in lon["segments"] for c in seg}
    ly = {int(k): val for k, val in lat["local"].items()}
    lx = {int(k): val for k, val in lon["local"].items()}
    for y in range(7):
        for xx in range(8):
            keys = [(y2, x2) for y2 in seg_y[y] for x2 in seg_x[xx]]
            logits = np.array([tab[0, ly[y] - ly[y2] + 3, lx[xx] - lx[x2] + 3, 0]
                               for y2, x2 in keys])
            w = np.exp(logits - logits.max())
            w /= w.sum()
            want = sum(wi * v[y2, x2] for wi, (y2, x2) in zip(w, keys))
            assert np.abs(got[0, 0, y, xx] - want).max() < 1e-13
            # the same weights follow from the key part alone
            w2 = np.exp([-a * ly[y2] - b * lx[x2] for y2, x2 in keys])
            assert np.abs(w - w2 / w2.sum()).max() < 1e-6


def test_constant_values(oracle_lib):
    p = TINY[6]
    x = make_inputs(p, seed=24)
    x["v"].fill_(0.8125)
    got = run_direct(oracle_lib, p, x)
    assert np.abs(got - 0.8125).max() < 1e-15


def test_unit_window_returns_v(oracle_lib):
    p = P((2, 5, 6), (2, 5, 6), (1, 1, 1), (0, 0, 0), heads=2, head_dim=8)
    x = make_inputs(p, seed=25)
    got = run_direct(oracle_lib, p, x)
    assert np.array_equal(got, f64(x["v"]))


# --------------------------------------------------------------------------- brute force


def test_brute_force_over_hand_segments(oracle_lib):
    """Random Q/K/V/table on the tiny padded grid, every query computed with plain
    Python arithmetic over the hand-derived key set."""
    ax = golden_axes()
    lat, lon = ax["tiny_lat_pad"], ax["tiny_lon_cyclic"]
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), heads=2, head_dim=3)
    x = make_inputs(p, seed=26)
    got = run_direct(oracle_lib, p, x)
    q, k, v, tab = (f64(x[n]) for n in ("q", "k", "v", "table"))
    seg_y = {c: seg for seg in lat["segments"] for c in seg}
    seg_x = {c: seg for seg in lon["segments"] for c in seg}
    ly = {int(kk): val for kk, val in lat["local"].items()}
    lx = {int(kk): val for kk, val in lon["local"].items()}
    sc = 1.0 / math.sqrt(3)
    for y in range(7):
        for xx in range(8):
            for h in range(2):
                keys = [(y2, x2) for y2 in seg_y[y] for x2 in seg_x[xx]]
                logits = []
                for y2, x2 in keys:
                    dot = sum(q[0, 0, y, xx, h, e] * k[0, 0, y2, x2, h, e] for e in range(3))
                    logits.append(dot * sc + tab[0, ly[y] - ly[y2] + 3, lx[xx] - lx[x2] + 3, h])
                m = max(logits)
                ws = [math.exp(l - m) for l in logits]
                tot = sum(ws)
                for e in range(3):
                    want = sum(w * v[0, 0, y2, x2, h, e] for w, (y2, x2) in zip(ws, keys)) / tot
                    assert abs(got[0, 0, y, xx, h, e] - want) < 1e-13


# --------------------------------------------------------------------------- invariants


@pytest.mark.parametrize("r", [1, 3, 6])
def test_longitude_translation_equivariance(oracle_lib, r):
    p = P((1, 7, 12), (1, 8, 12), (1, 4, 4), (0, 2, 1), heads=2, head_dim=8)
    x = make_inputs(p, seed=27)
    base = run_direct(oracle_lib, p, x)
    p2 = p.with_(shift=(0, 2, (1 + r) % 4))
    x2 = dict(x)
    for n in ("q", "k", "v"):
        x2[n] = torch.roll(x[n], shifts=r, dims=3)
    moved = run_direct(oracle_lib, p2, x2)
    # the direct form sums keys in grid order, which the roll changes: equal to rounding
    assert np.abs(moved - np.roll(base, r, axis=3)).max() < 1e-14


def test_per_window_independence(oracle_lib):
    """Perturbing every input token of one shifted window (latitude block [2,6),
    longitude block [6,8)+[0,2) of the tiny grid) leaves all other outputs bit-identical."""
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), heads=2, head_dim=4)
    x = make_inputs(p, seed=28)
    base = run_direct(oracle_lib, p, x)
    ys, xs = [2, 3, 4, 5], [6, 7, 0, 1]
    x2 = {n: t.clone() for n, t in x.items()}
    for n in ("q", "k", "v"):
        x2[n][0, 0, np.ix_(ys, xs)[0], np.ix_(ys, xs)[1]] += 3.0
    pert = run_direct(oracle_lib, p, x2)
    inside = np.zeros((7, 8), bool)
    inside[np.ix_(ys, xs)] = True
    assert np.array_equal(pert[0, 0][~inside], base[0, 0][~inside])
    assert not np.array_equal(pert[0, 0][inside], base[0, 0][inside])


def test_mask_isolates_regions_of_one_rolled_window(oracle_lib):
    """The last rolled latitude window of the ragged grid holds pad rows and the
    wrapped rows 0..4.  Changing K/V of rows 175..180 (another region of the
    neighbouring window) and of every other row must not move rows 0..4; changing
    rows 0..4 must."""
    p = P((1, 181, 20), (1, 190, 20), (1, 10, 10), (0, 5, 5), heads=1, head_dim=4)
    x = make_inputs(p, seed=29)
    base = run_direct(oracle_lib, p, x)
    x2 = {n: t.clone() for n, t in x.items()}
    x2["k"][0, 0, 5:] *= -2.0
    x2["v"][0, 0, 5:] += 1.0
    pert = run_direct(oracle_lib, p, x2)
    assert np.array_equal(pert[0, 0, :5], base[0, 0, :5])
    x3 = {n: t.clone() for n, t in x.items()}
    x3["v"][0, 0, :5] += 1.0
    pert3 = run_direct(oracle_lib, p, x3)
    assert np.array_equal(pert3[0, 0, 5:], base[0, 0, 5:])
    assert not np.array_equal(pert3[0, 0, :5], base[0, 0, :5])


def test_masked_latitude_does_not_wrap_but_longitude_does(oracle_lib):
    p = P((1, 8, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2))
    assert not oracle_lib.visible(p, (0, 0, 3), (0, 7, 3))  # lat rows 0 and 7: no wrap
    assert oracle_lib.visible(p, (0, 3, 0), (0, 3, 7))  # lon cols 0 and 7: wrap


def test_workload_shapes_are_valid_tilings(oracle_lib):
    for p in WORKLOADS.values():
        assert oracle_lib.check(p) == 0, p.name


# --------------------------------------------------------------------------- roll direction and pad values


def _roll_plus_attention(p, x):
    """Brute force with the OTHER roll direction, written here from the steps:
    pad at the end, roll by +s (rolled[c'] = padded[(c' - s) mod P]), cut into
    windows, mask pairs across the wrap (now the first s rolled rows of a
    masked axis) and pad keys, bias by the position inside the window."""
    B, (T, H, W), (Pt, Ph, Pw) = p.batch, p.extent, p.padded
    w, s = np.array(p.window), np.array(p.shift)
    scale = 1.0 / math.sqrt(p.head_dim)
    q, k, v, tab = (f64(x[n]) for n in ("q", "k", "v", "table"))
    out = np.zeros_like(q)
    for b in range(B):
        # per rolled coordinate: source (or None for pad), wrapped flags, window, local
        info = {}
        for ct in range(Pt):
            for cy in range(Ph):
                for cx in range(Pw):
                    cr = np.array([ct, cy, cx])
                    src = (cr - s) % np.array([Pt, Ph, Pw])
                    real = src[0] < T and src[1] < H and src[2] < W
                    wrapped = tuple(bool(cr[a] < s[a]) and not p.cyclic[a] for a in range(3))
                    info[(ct, cy, cx)] = (tuple(src) if real else None, wrapped, tuple(cr // w), cr % w)
        for crq, (srcq, wq, winq, lq) in info.items():
            if srcq is None:
                continue
            keys = [(srck, lk) for crk, (srck, wk, wink, lk) in info.items()
                    if wink == winq and wk == wq and srck is not None]
            for h in range(p.heads):
                qi = q[(b,) + srcq + (h,)]
                lg = np.array([scale * qi @ k[(b,) + sk + (h,)]
                               + tab[tuple(lq - lk + w - 1) + (h,)] for sk, lk in keys])
                e = np.exp(lg - lg.max())
                out[(b,) + srcq + (h,)] = sum(ei * v[(b,) + sk + (h,)] for ei, (sk, _) in zip(e / e.sum(), keys))
    return out


def test_roll_direction_is_immaterial_at_half_window_shift(oracle_lib):
    """With s = w/2 and the padded extent a multiple of w, rolling by +s or -s
    gives the same windows, masks and window-local positions, so the same output."""
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), heads=2, head_dim=4)
    x = make_inputs(p, seed=31)
    assert np.abs(_roll_plus_attention(p, x) - run_direct(oracle_lib, p, x)).max() < 1e-12


def test_roll_direction_matters_off_half_window(oracle_lib):
    """The same brute force with s != w/2 must NOT match: the test above can fail."""
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 1, 1), heads=1, head_dim=4)
    x = make_inputs(p, seed=32)
    assert np.abs(_roll_plus_attention(p, x) - run_direct(oracle_lib, p, x)).max() > 1e-3


def test_pad_values_do_not_matter(oracle_lib, monkeypatch):
    """Pad tokens get weight exactly 0: filling the pad slots of the literal form
    with large random values instead of zeros leaves every real output unchanged."""
    from oracle import literal

    p = P((1, 13, 8), (1, 16, 8), (1, 4, 4), (0, 2, 2), heads=2, head_dim=4)
    x = make_inputs(p, seed=33)
    base = run_literal(oracle_lib, p, x)
    orig = literal._pad
    rng = np.random.default_rng(5)

    def noisy_pad(prob, a):
        out = orig(prob, a)
        T, H, W = prob.extent
        noise = rng.normal(0.0, 50.0, out.shape)
        noise[:, :T, :H, :W] = 0.0
        return out + noise

    monkeypatch.setattr(literal, "_pad", noisy_pad)
    noisy = run_literal(oracle_lib, p, x)
    assert np.array_equal(noisy, base)


# --------------------------------------------------------------------------- log-sum-exp


def test_lse_single_window_shift0_is_logsumexp(oracle_lib):
    """One window with shift 0 is global attention: the log-sum-exp of a query is
    torch's logsumexp over all its logits (scaled products plus the bias of the
    raw coordinate differences), in float64 on the CPU."""
    p = P((2, 3, 4), (2, 3, 4), (2, 3, 4), (0, 0, 0), heads=3, head_dim=16, batch=2)
    x = make_inputs(p, seed=41)
    x["table"] = torch.randn(p.table_shape, generator=torch.Generator().manual_seed(6), dtype=torch.float32)
    got = oracle_lib.literal_lse(p, f64(x["q"]), f64(x["k"]), f64(x["table"]))
    T, H, W = p.extent
    coords = torch.stack(torch.meshgrid(torch.arange(T), torch.arange(H), torch.arange(W),
                                        indexing="ij"), -1).reshape(-1, 3)
    rel = coords[:, None, :] - coords[None, :, :] + torch.tensor(p.window) - 1
    bias = x["table"].double()[rel[..., 0], rel[..., 1], rel[..., 2]].permute(2, 0, 1)  # [h, n, m]
    n = T * H * W
    q = x["q"].double().reshape(p.batch, n, p.heads, p.head_dim).permute(0, 2, 1, 3)
    k = x["k"].double().reshape(p.batch, n, p.heads, p.head_dim).permute(0, 2, 1, 3)
    logits = q @ k.transpose(-1, -2) / math.sqrt(p.head_dim) + bias[None]
    ref = torch.logsumexp(logits, dim=-1).permute(0, 2, 1).reshape(got.shape).numpy()
    assert np.abs(got - ref).max() < 1e-12


def test_lse_brute_force_over_hand_segments(oracle_lib):
    """The tiny padded grid: each query's log-sum-exp by plain Python arithmetic
    over its hand-derived key set."""
    ax = golden_axes()
    lat, lon = ax["tiny_lat_pad"], ax["tiny_lon_cyclic"]
    p = P((1, 7, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), heads=2, head_dim=3)
    x = make_inputs(p, seed=27)
    got = oracle_lib.literal_lse(p, f64(x["q"]), f64(x["k"]), f64(x["table"]))
    q, k, tab = (f64(x[n]) for n in ("q", "k", "table"))
    seg_y = {c: seg for seg in lat["segments"] for c in seg}
    seg_x = {c: seg for seg in lon["segments"] for c in seg}
    ly = {int(kk): val for kk, val in lat["local"].items()}
    lx = {int(kk): val for kk, val in lon["local"].items()}
    sc = 1.0 / math.sqrt(3)
    for y in range(7):
        for xx in range(8):
            for h in range(2):
                logits = []
                for y2 in seg_y[y]:
                    for x2 in seg_x[xx]:
                        dot = sum(q[0, 0, y, xx, h, e] * k[0, 0, y2, x2, h, e] for e in range(3))
                        logits.append(dot * sc + tab[0, ly[y] - ly[y2] + 3, lx[xx] - lx[x2] + 3, h])
                m = max(logits)
                want = m + math.log(sum(math.exp(l - m) for l in logits))
                assert abs(got[0, 0, y, xx, h] - want) < 1e-13


def test_lse_uniform_logits_count_the_key_set(oracle_lib):
    """Q = 0 and a constant table c make every logit c: the log-sum-exp is
    c + log(size of the key set), the sizes fixed by the hand derivation
    (ragged 181 -> 190 latitude, window 10x10, shift 5; longitude 360)."""
    base = WORKLOADS["c4_bf16_181x360_pad190"]
    p = base.with_(dtype="f32", heads=2, head_dim=4, batch=1)
    x = make_inputs(p, seed=28)
    x["q"].zero_()
    x["table"].fill_(0.25)
    got = oracle_lib.literal_lse(p, f64(x["q"]), f64(x["k"]), f64(x["table"]))
    ax = golden_axes()
    lat = ax["ragged_lat_181_pad190_w10_s5"]["segments_of"]
    lon = ax["lon_360_w10_s5"]["segments_of"]
    for y, xx in [(0, 0), (4, 359), (180, 200), (100, 5), (175, 0)]:
        size = len(expand(*lat[str(y)], 181)) * len(expand(*lon[str(xx)], 360))
        assert np.abs(got[0, 0, y, xx] - (0.25 + math.log(size))).max() < 1e-13


def test_lse_gives_the_forward_weights(oracle_lib):
    """exp(logit - lse) are the weights of the forward output: with V the one-hot
    code of each key, the literal forward returns them, and they sum to 1."""
    p = P((1, 6, 8), (1, 8, 8), (1, 4, 4), (0, 2, 2), heads=2, head_dim=5, cyclic=(0, 0, 1))
    x = make_inputs(p, seed=29)
    lse = oracle_lib.literal_lse(p, f64(x["q"]), f64(x["k"]), f64(x["table"]))
    out = run_literal(oracle_lib, p, x)
    # a ones vector for V makes the forward return the weight sum (1 for every real query)
    x1 = dict(x)
    x1["v"] = torch.ones_like(x["v"])
    ones = run_literal(oracle_lib, p, x1)
    assert np.abs(ones - 1.0).max() < 1e-12
    # and the output equals sum_k exp(logit - lse) v_k over the visible keys, by brute force
    # through the literal form's own windows for one query
    import oracle as O
    qw, kw, vw = (O.literal_windows(p, f64(x[n])) for n in ("q", "k", "v"))
    bias = O.literal_bias(p, f64(x["table"]))
    vis = O.literal_visibility(p)
    lw = O.literal_windows(p, lse[..., None])[..., 0]  # [B, nW, N, h]
    b, w, n, h = 0, 1, 5, 1
    logit = (qw[b, w, n, h] @ kw[b, w, :, h].T) / math.sqrt(5) + bias[h, n]
    wts = np.where(vis[w, n], np.exp(logit - lw[b, w, n, h]), 0.0)
    assert abs(wts.sum() - 1.0) < 1e-12
    o = wts @ vw[b, w, :, h]
    ow = O.literal_windows(p, out)
    assert np.abs(o - ow[b, w, n, h]).max() < 1e-12
