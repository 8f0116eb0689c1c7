"""Row-parallel oracle checks for the large workloads (test infrastructure).

The oracle itself is unchanged: each worker builds an oracle problem for a
range of queries and runs the same per-row checks as the serial tests (routed
heads bit for bit, then parity.check_row on the selection and its scores).
Workers are started fresh ("spawn") and import neither torch nor the HIP
library, so they never touch the GPU; the keys are sent to each worker once.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle as O
from parity import RTOL, check_row, tolerance

_KEYS = {}


def _init(K, k_scale, B, kdt, kbar):
    # one BLAS thread per worker: the pool already spreads rows over the cores
    from threadpoolctl import threadpool_limits
    _KEYS["limits"] = threadpool_limits(1)
    _KEYS.update(K=K, k_scale=k_scale, B=B, kdt=kdt, kbar=kbar)


def _misa_rows(job):
    """Check rows [r0, r0 + len) of a MISA output; returns (rows, ill-posed
    head sets, worst error / tolerance)."""
    r0, q, w, pos, heads_gpu, A, k, idx, sc = job
    P = O.Problem(q, w, _KEYS["K"], pos, _KEYS["B"], _KEYS["kdt"], _KEYS["k_scale"], kbar=_KEYS["kbar"])
    heads_o, r_o = O.route(P, A)
    ill, worst = 0, 0.0
    rtol = RTOL[_KEYS["kdt"]]
    for t in range(P.T):
        g = sorted(int(h) for h in heads_gpu[t])
        o = sorted(int(h) for h in heads_o[t])
        if g != o:
            srt = np.sort(r_o[t])[::-1]
            scale = max(1e-300, np.abs(r_o[t]).max())
            margin = srt[A - 1] - srt[A] if A < P.H else np.inf
            assert margin <= 1e-12 * scale, f"row {r0 + t}: heads {g} != oracle {o} (margin {margin:.3e})"
            ill += 1
        n = P.n(t)
        keys = np.arange(n)
        hs = heads_o[t]
        sel, _ = O.first_k(O.routed_scores(P, t, hs, keys), keys, k)
        worst = max(worst, check_row(
            idx[t], sc[t], k, n, "ascending", sel,
            lambda s, t=t, hs=hs: O.routed_scores(P, t, hs, s),
            lambda s, t=t, hs=hs: tolerance(P, t, hs, s, rtol), label=f"row {r0 + t}"))
    return P.T, ill, worst


def check_misa_all_rows(inp, B, A, k, heads, idx, sc, chunk=128, workers=None):
    """Every row of a MISA output (heads [T, A], idx / sc [T, k], host arrays)
    against the oracle, in parallel over host cores. Returns (rows checked,
    ill-posed head sets, worst error / tolerance)."""
    kdt = O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16
    T = len(inp["pos"])
    jobs = [(r0, inp["q"][r0:r0 + chunk], inp["w"][r0:r0 + chunk], inp["pos"][r0:r0 + chunk],
             heads[r0:r0 + chunk], A, k, idx[r0:r0 + chunk], sc[r0:r0 + chunk]) for r0 in range(0, T, chunk)]
    # heaviest rows (longest prefixes) first, so the pool drains evenly
    jobs.sort(key=lambda j: -int(np.max(j[3])))
    n = workers or min(16, os.cpu_count() or 1)
    ctx = mp.get_context("spawn")
    rows = ill = 0
    worst = 0.0
    with ctx.Pool(n, initializer=_init, initargs=(inp["K"], inp["k_scale"], B, kdt, inp.get("kbar"))) as pool:
        for r, i, wv in pool.imap_unordered(_misa_rows, jobs):
            rows += r
            ill += i
            worst = max(worst, wv)
    return rows, ill, worst
