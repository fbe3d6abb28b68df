"""The oracle's per-window backward over every window of a full-size grid,
split across worker processes (test infrastructure).

``oracle.literal_backward`` is plain numpy and takes about 0.1 s per 12x12
window with 8 heads, so the 4,050 windows of a 540x1080 grid take minutes on
one core.  Its gradients are per-window (every real token lies in exactly one
window) and its table gradient is a sum of per-window shares, so disjoint
window subsets can run in separate processes and be combined exactly as the
single call would, up to the order of the fp64 table sums.

The workers are spawned (not forked) and import only numpy and the oracle:
they never touch the GPU.  Inputs and the GPU's gradients reach them through
memory-mapped files; each worker returns, per gradient, the largest absolute
difference and the largest reference magnitude over its tokens, plus its share
of the table gradient.
"""
import multiprocessing as mp
import os
import tempfile
from concurrent.futures import ProcessPoolExecutor
from types import SimpleNamespace

import numpy as np

NAMES = ("q", "k", "v", "dout", "dq", "dk", "dv")
FIELDS = ("batch", "heads", "head_dim", "extent", "padded", "window", "shift", "cyclic", "scale", "windows")


def _plain(prob):
    """The problem's fields as a plain namespace (the workers then import no
    part of the library's package)."""
    return SimpleNamespace(**{f: getattr(prob, f, None) for f in FIELDS})


def _worker(args):
    import oracle

    prob, files, shape, table, windows = args
    a = {n: np.memmap(files[n], dtype=np.float32, mode="r", shape=shape) for n in NAMES}
    ref = oracle.literal_backward(prob, a["q"], a["k"], a["v"], table, a["dout"], windows=windows)
    mine = np.isin(oracle.token_windows(prob), [w % (prob.windows // prob.batch) for w in windows])
    bsel = sorted({w // (prob.windows // prob.batch) for w in windows})
    diff, mag = [], []
    for name, r in zip(("dq", "dk", "dv"), ref[:3]):
        d = m = 0.0
        for b in bsel:
            rb = r[b][mine]
            gb = np.asarray(a[name][b][mine], dtype=np.float64)
            d = max(d, float(np.abs(gb - rb).max(initial=0.0)))
            m = max(m, float(np.abs(rb).max(initial=0.0)))
        diff.append(d)
        mag.append(m)
    return diff, mag, ref[3]


def pooled_backward_errors(prob, host, grads_gpu, workers=None):
    """Relative max-abs errors of the GPU's dq, dk, dv (every token) and its
    table gradient against the oracle's literal backward over all windows.

    host: dict of fp32 numpy arrays q, k, v, dout, table; grads_gpu: fp32
    numpy arrays dq, dk, dv, dtable.  Windows are split into one contiguous
    range per batch item and worker (each range stays inside one batch item).
    """
    workers = workers or min(16, os.cpu_count() or 1)
    shape = tuple(host["q"].shape)
    tmpdir = "/dev/shm" if os.path.isdir("/dev/shm") else None
    files = {}
    try:
        for name, arr in list(host.items()) + list(zip(("dq", "dk", "dv"), grads_gpu[:3])):
            if name == "table":
                continue
            fd, path = tempfile.mkstemp(prefix=f"swa_{name}_", suffix=".f32", dir=tmpdir)
            os.close(fd)
            mm = np.memmap(path, dtype=np.float32, mode="w+", shape=shape)
            mm[...] = arr
            mm.flush()
            del mm
            files[name] = path
        per_b = prob.windows // prob.batch
        jobs = []
        for b in range(prob.batch):
            nj = max(1, workers // prob.batch)
            for j in range(nj):
                w0, w1 = b * per_b + per_b * j // nj, b * per_b + per_b * (j + 1) // nj
                if w1 > w0:
                    jobs.append((_plain(prob), files, shape, host["table"], list(range(w0, w1))))
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            results = list(ex.map(_worker, jobs))
    finally:
        for path in files.values():
            os.unlink(path)
    errs = {}
    for i, name in enumerate(("dq", "dk", "dv")):
        errs[name] = max(r[0][i] for r in results) / max(max(r[1][i] for r in results), 1e-30)
    dtable_ref = sum(r[2] for r in results)
    dt = np.asarray(grads_gpu[3], dtype=np.float64)
    errs["dtable"] = float(np.abs(dt - dtable_ref).max() / max(np.abs(dtable_ref).max(), 1e-30))
    return errs
