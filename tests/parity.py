"""Comparison of the HIP library's outputs with the CPU oracle.

Rules (floating point decides selections, so sets are compared up to the
score tolerance, everything integer is compared exactly):
  * routed head sets: identical, except for queries whose oracle margin between
    the A-th and (A+1)-th router score is at float64 rounding level;
  * scores: |gpu - oracle| <= rtol * Ibar + 2^-16 * Jhat at every returned key,
    with Ibar = sum_h |w| ReLU(z) and Jhat = sum_h |w| sum_i |q_i k_i| over the
    scoring heads (rtol = 2e-3 for bf16 keys, 1.5e-2 for fp8 keys);
  * top-k sets: same size, valid, unique, ascending, visible; a key chosen by
    the GPU but not by the oracle (or the reverse) must be within tolerance of
    the keys it displaced;
  * padding: idx = -1 and score = -inf after the k_t valid entries.
"""
from __future__ import annotations

import numpy as np

import oracle as O

RTOL = {O.KDT_BF16: 2e-3, O.KDT_FP8: 1.5e-2}


def rtol_of(inp):
    """bf16 tolerance only when neither keys nor queries are fp8."""
    fp8 = inp["k_scale"] is not None or inp.get("q_scale") is not None
    return RTOL[O.KDT_FP8 if fp8 else O.KDT_BF16]
ABS = 2.0 ** -16


def to_gpu(inp, device="cuda"):
    """(q, w, K, k_scale, pos) device tensors; fp8 queries come as uint8 codes
    (their scales: q_scale_gpu)."""
    import torch
    if inp.get("q_scale") is not None:
        q = torch.from_numpy(inp["q"]).to(device)
    else:
        q = torch.from_numpy(inp["q"].view(np.int16)).to(device)
    w = torch.from_numpy(inp["w"]).to(device)
    if inp["k_scale"] is not None:
        K = torch.from_numpy(inp["K"]).to(device)
        ks = torch.from_numpy(inp["k_scale"]).to(device)
    else:
        K = torch.from_numpy(inp["K"].view(np.int16)).to(device)
        ks = None
    pos = torch.from_numpy(inp["pos"].astype(np.int32)).to(device)
    return q, w, K, ks, pos


def q_scale_gpu(inp, device="cuda"):
    import torch
    qs = inp.get("q_scale")
    return None if qs is None else torch.from_numpy(qs).to(device)


def oracle_problem(inp, B, rows=None):
    """Oracle problem of an input dict; an optional inp["kbar"] (float32 cached
    block means) and inp["q_scale"] (fp8 queries) are passed through."""
    kdt = O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16
    kbar = inp.get("kbar")
    qs = inp.get("q_scale")
    qdt = O.QDT_FP8 if qs is not None else O.QDT_BF16
    if rows is None:
        return O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B, kdt, inp["k_scale"], kbar=kbar,
                         q_dtype=qdt, q_scale=qs)
    rows = np.asarray(rows)
    return O.Problem(inp["q"][rows], inp["w"][rows], inp["K"], inp["pos"][rows], B, kdt, inp["k_scale"],
                     kbar=kbar, q_dtype=qdt, q_scale=None if qs is None else qs[rows])


def kdtype(inp):
    return O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16


def check_heads(P, A, heads_gpu, r_gpu=None, rows=None):
    """Routed head sets must be identical; returns the number of ill-posed
    queries (oracle margin at float64 rounding) where a difference is allowed."""
    heads_o, r_o = O.route(P, A)
    ill = 0
    for t in range(P.T):
        g = sorted(int(h) for h in heads_gpu[t])
        o = sorted(int(h) for h in heads_o[t])
        assert list(heads_gpu[t]) == g, f"row {t}: heads not ascending {heads_gpu[t]}"
        if g != o:
            srt = np.sort(r_o[t])[::-1]
            scale = max(1e-300, np.abs(r_o[t]).max())
            margin = srt[A - 1] - srt[A] if A < P.H else np.inf
            assert margin <= 1e-12 * scale, (
                f"row {t}: heads {g} != oracle {o} with margin {margin:.3e} (scale {scale:.3e})")
            ill += 1
        if r_gpu is not None:
            # r is returned as float32 of a float64 value
            assert np.allclose(r_gpu[t], r_o[t].astype(np.float32), rtol=2e-7, atol=1e-30), \
                f"row {t}: r differs"
    return heads_o, ill


def tolerance(P, t, heads, keys, rtol):
    ibar, jhat = O.magnitude_terms(P, t, heads, keys)
    return rtol * ibar + ABS * jhat


def check_row(idx_g, sc_g, k, n_vis, order, oracle_sel, score_fn, tol_fn,
              sure_pool=None, maybe_pool=None, label=""):
    """Check one output row.

    oracle_sel: the oracle's selected indices; score_fn(keys) -> oracle scores;
    tol_fn(keys) -> tolerances. sure_pool / maybe_pool (sets) describe keys that
    must / may be in the GPU's candidate pool when the pool itself is decided by
    a floating-point comparison (MISA-dagger, HISA); None means the pool is the
    whole visible prefix.
    """
    idx_g = np.asarray(idx_g)
    sc_g = np.asarray(sc_g)
    valid = idx_g >= 0
    kt_g = int(valid.sum())
    kt_o = len(oracle_sel)
    assert valid[:kt_g].all() and not valid[kt_g:].any(), f"{label}: padding not at the end"
    assert np.all(idx_g[kt_g:] == -1) and np.all(np.isneginf(sc_g[kt_g:])), f"{label}: bad padding"
    g = idx_g[:kt_g].astype(np.int64)
    if maybe_pool:
        assert abs(kt_g - kt_o) <= len(maybe_pool), f"{label}: count {kt_g} vs {kt_o}"
    else:
        assert kt_g == kt_o, f"{label}: {kt_g} selected, oracle {kt_o}"
    if order == "ascending":
        assert np.all(np.diff(g) > 0), f"{label}: indices not strictly ascending"
    assert len(np.unique(g)) == kt_g, f"{label}: duplicate indices"
    assert (g >= 0).all() and (g < n_vis).all(), f"{label}: index outside the visible prefix"
    if kt_g == 0:
        return 0.0
    o_at_g = score_fn(g)
    tol_g = tol_fn(g)
    err = np.abs(sc_g[:kt_g].astype(np.float64) - o_at_g)
    bad = err > tol_g
    assert not bad.any(), (f"{label}: score error {err[bad][:4]} > tol {tol_g[bad][:4]} "
                           f"at keys {g[bad][:4]}")
    oset = set(int(s) for s in oracle_sel)
    gset = set(int(s) for s in g)
    extra = np.array(sorted(gset - oset), dtype=np.int64)     # GPU took, oracle did not
    missing = np.array(sorted(oset - gset), dtype=np.int64)   # oracle took, GPU did not
    if sure_pool is not None or maybe_pool is not None:
        allowed = (sure_pool or set()) | (maybe_pool or set())
        for s in extra:
            assert int(s) in allowed, f"{label}: key {s} outside every admissible candidate pool"
        if maybe_pool:
            missing = np.array([s for s in missing if int(s) not in maybe_pool], dtype=np.int64)
    if len(extra) and len(missing):
        lo = (score_fn(extra) + tol_fn(extra)).min()
        hi = (score_fn(missing) - tol_fn(missing)).max()
        assert lo >= hi, (f"{label}: GPU kept {extra[:4]} over oracle's {missing[:4]} "
                          f"beyond tolerance ({lo:.6g} < {hi:.6g})")
    elif len(missing) and not maybe_pool:
        raise AssertionError(f"{label}: oracle keys {missing[:4]} missing")
    rel = err / np.maximum(np.abs(o_at_g), 1e-30)
    return float(np.max(err / np.maximum(tol_g, 1e-300)))


def pool_bands(scores, chosen, tol):
    """Split keys into sure-in / maybe for a selection decided on float scores:
    a chosen key is sure when no unchosen key can reach it within tolerance
    (and vice versa)."""
    chosen = np.asarray(chosen, dtype=np.int64)
    mask = np.zeros(len(scores), dtype=bool)
    mask[chosen] = True
    if mask.all() or not mask.any():
        return set(int(s) for s in chosen), set()
    lo_in = scores - tol
    hi_out = scores + tol
    best_out = hi_out[~mask].max()
    worst_in = lo_in[mask].min()
    sure = set(int(s) for s in np.nonzero(mask & (lo_in > best_out))[0])
    maybe = set(int(s) for s in np.nonzero(mask & ~(lo_in > best_out))[0])
    maybe |= set(int(s) for s in np.nonzero(~mask & (hi_out >= worst_in))[0])
    return sure, maybe
