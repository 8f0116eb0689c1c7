"""Pins for the oracle's companion terms and block statistics (no GPU).

  * magnitude_terms (Ibar = sum_h |w| ReLU(z), Jhat = sum_h |w| sum_i |q_i k_i|),
    which set every score tolerance of the GPU parity checks, against an exact
    rational brute force written out term by term;
  * full_block_means and block_means (the means of the whole array's blocks,
    and a query's own blocks with its partial last block and cached means)
    against explicit loops in exact arithmetic, including B not dividing L,
    B > L and B = 1;
  * the generator's planted needles: the dense indexer of the oracle ranks
    every needle into its top-k at the tiny-decode and the 128K workloads (the
    needle-in-a-haystack stand-in must be findable by the method it stands in
    for; HISA write-up, "Needle-in-a-Haystack").

Each pin is a function taking the oracle function it checks, so that the
planted-slip tests at the end can hand it plausible mistakes (|z| in place of
ReLU(z), a dropped |w|, sum|q| * sum|k| in place of sum|q_i k_i|, an
off-by-one tail block) and see it fail.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth


def _frac(vals):
    return np.vectorize(lambda v: Fraction(float(v)), otypes=[object])(np.asarray(vals, dtype=np.float64))


def _exact_keys(inp):
    """Key values as Fractions, decoded with torch's casts (not the oracle's)."""
    if inp["k_scale"] is None:
        kv = torch.from_numpy(inp["K"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        return _frac(kv)
    codes = torch.from_numpy(inp["K"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = _frac(inp["k_scale"].astype(np.float64))
    return _frac(codes) * sc[:, None]


def _exact_q(inp):
    qv = torch.from_numpy(inp["q"].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    return _frac(qv)


def _problem(inp, B=4):
    kdt = O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16
    return O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B, kdt, inp["k_scale"],
                     kbar=inp.get("kbar"))


# ------------------------------------------------------------------ magnitude terms

def _pin_magnitudes(fn, inp, heads_per_query, exact_values):
    """Ibar and Jhat of fn against term-by-term rational sums."""
    P = _problem(inp)
    q, K = _exact_q(inp), _exact_keys(inp)
    w = _frac(inp["w"].astype(np.float64))
    for t in range(P.T):
        heads = heads_per_query[t]
        keys = np.arange(P.L)
        ibar, jhat = fn(P, t, heads, keys)
        for s in keys:
            ib, jh = Fraction(0), Fraction(0)
            for h in heads:
                z = Fraction(0)
                ab = Fraction(0)
                for i in range(P.d):
                    prod = q[t, h, i] * K[s, i]
                    z += prod
                    ab += abs(prod)
                ib += abs(w[t, h]) * (z if z > 0 else Fraction(0))
                jh += abs(w[t, h]) * ab
            if exact_values:
                assert ibar[s] == float(ib) and jhat[s] == float(jh), (t, s)
            else:
                assert abs(Fraction(float(ibar[s])) - ib) <= Fraction(1, 10 ** 12) * (ib + jh), (t, s)
                assert abs(Fraction(float(jhat[s])) - jh) <= Fraction(1, 10 ** 12) * jh, (t, s)
            assert ibar[s] <= jhat[s] * (1 + 1e-12)   # |ReLU(z)| <= sum |q_i k_i|


def _mag_inputs(seed, kdt, int_grid):
    inp = synth.random_small(seed, T=3, L=12, H=5, d=8, k_dtype=kdt, int_grid=int_grid)
    # negative weights in every query (a dropped |w| shows)
    inp["w"][:, 0] = -np.abs(inp["w"][:, 0]) - np.float32(0.25)
    return inp


_HEADS = [[0, 2, 4], [1, 0], [0, 1, 2, 3, 4]]


@pytest.mark.parametrize("seed", range(3))
def test_magnitude_terms_exact_on_dyadic_grid(seed):
    """Dyadic inputs: every sum is exact in float64, so Ibar and Jhat must equal
    the rational values bit for bit."""
    _pin_magnitudes(O.magnitude_terms, _mag_inputs(seed, O.KDT_BF16, True), _HEADS, exact_values=True)


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
@pytest.mark.parametrize("seed", range(2))
def test_magnitude_terms_exact_random(seed, kdt):
    _pin_magnitudes(O.magnitude_terms, _mag_inputs(10 + seed, kdt, False), _HEADS, exact_values=False)


# ------------------------------------------------------------------ block means

def _pin_full_block_means(fn, inp, B):
    """fn(K values, B) against the rational mean of each block of the whole
    array: blocks [b*B, min((b+1)*B, L)), the last one possibly partial."""
    K = _exact_keys(inp)
    L, d = K.shape
    vals = O.dequant_keys(inp["K"], O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16, inp["k_scale"])
    got = fn(vals, B)
    nb = (L + B - 1) // B
    assert got.shape == (nb, d), got.shape
    for b in range(nb):
        s0, s1 = b * B, min(b * B + B, L)
        for i in range(d):
            exact = sum((K[s, i] for s in range(s0, s1)), Fraction(0)) / (s1 - s0)
            # float64 sum of a few bf16 / fp8*scale values is exact; one rounding in the division
            assert abs(Fraction(float(got[b, i])) - exact) <= abs(exact) * Fraction(1, 2 ** 52), (b, i)


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
@pytest.mark.parametrize("L,B", [(23, 5), (24, 8), (7, 32), (9, 1), (16, 16), (17, 16)])
def test_full_block_means_explicit(kdt, L, B):
    inp = synth.random_small(3, T=1, L=L, H=2, d=6, k_dtype=kdt)
    _pin_full_block_means(O.full_block_means, inp, B)


def _pin_query_block_means(fn, inp, B):
    """fn(P, t): means of query t's visible blocks; the last block covers
    [(M_t - 1) B, n_t) only, and cached rows stand in for complete earlier blocks."""
    P = _problem(inp, B)
    K = _exact_keys(inp)
    kbar = inp.get("kbar")
    for t in range(P.T):
        n = P.n(t)
        got = fn(P, t)
        M = (n + B - 1) // B
        assert got.shape == (M, P.d), (t, got.shape)
        for b in range(M):
            s0, s1 = b * B, min(b * B + B, n)
            for i in range(P.d):
                if kbar is not None and b < M - 1:
                    exact = Fraction(float(kbar[b, i]))
                else:
                    exact = sum((K[s, i] for s in range(s0, s1)), Fraction(0)) / (s1 - s0)
                assert abs(Fraction(float(got[b, i])) - exact) <= abs(exact) * Fraction(1, 2 ** 52), (t, b, i)


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
@pytest.mark.parametrize("B", [1, 4, 6, 40])
@pytest.mark.parametrize("cached", [False, True])
def test_query_block_means_explicit(kdt, B, cached):
    inp = synth.random_small(4, T=4, L=30, H=2, d=5, k_dtype=kdt)
    inp["pos"] = np.array([29, 12, 0, 5], dtype=np.int32)
    if cached:
        nb = (30 + B - 1) // B
        inp["kbar"] = np.random.default_rng(1).standard_normal((nb, 5)).astype(np.float32)
    _pin_query_block_means(O.block_means, inp, B)


# ------------------------------------------------------------------ needles

def _needle_recall(P, needles, k):
    res = O.dense_topk(P, k)
    hit = tot = 0
    for t, (idx, _) in enumerate(res):
        chosen = set(int(s) for s in idx)
        for s in needles[t]:
            tot += 1
            hit += int(s) in chosen
    return hit, tot


def test_needles_found_by_dense_oracle_tiny_decode():
    wl = synth.CONFIGS["c1_tiny_decode"]
    inp = synth.make_inputs(wl, seed=0)
    hit, tot = _needle_recall(_problem(inp, wl.B), inp["needles"], wl.k)
    assert tot == wl.T * wl.needles
    assert hit == tot


@pytest.mark.slow
def test_needles_found_by_dense_oracle_128k_rows():
    wl = synth.CONFIGS["c4_hier_decode_128k"]
    inp = synth.make_inputs(wl, seed=0)
    rows = [0, wl.T - 1]
    sub = dict(inp, q=inp["q"][rows], w=inp["w"][rows], pos=inp["pos"][rows])
    hit, tot = _needle_recall(_problem(sub, wl.B), [inp["needles"][t] for t in rows], wl.k)
    assert tot == len(rows) * wl.needles
    assert hit == tot


# ------------------------------------------------------------------ planted slips

def _slip_abs_z(P, t, heads, keys):
    ib, jh = O.magnitude_terms(P, t, heads, keys)
    z = P.q[t, list(heads)] @ P.K[np.asarray(keys)].T
    return (np.abs(P.w[t, list(heads)])[:, None] * np.abs(z)).sum(axis=0), jh


def _slip_signed_w(P, t, heads, keys):
    heads = list(heads)
    kk = P.K[np.asarray(keys)]
    z = P.q[t, heads] @ kk.T
    w = P.w[t, heads][:, None]
    return (w * np.maximum(z, 0.0)).sum(axis=0), (w * (np.abs(P.q[t, heads]) @ np.abs(kk).T)).sum(axis=0)


def _slip_product_of_sums(P, t, heads, keys):
    heads = list(heads)
    kk = P.K[np.asarray(keys)]
    ib, _ = O.magnitude_terms(P, t, heads, keys)
    wa = np.abs(P.w[t, heads])[:, None]
    return ib, (wa * np.abs(P.q[t, heads]).sum(axis=1)[:, None] * np.abs(kk).sum(axis=1)[None, :]).sum(axis=0)


def _slip_all_heads(P, t, heads, keys):
    return O.magnitude_terms(P, t, range(P.H), keys)


@pytest.mark.parametrize("slip", [_slip_abs_z, _slip_signed_w, _slip_product_of_sums, _slip_all_heads])
def test_magnitude_pin_catches_slips(slip):
    with pytest.raises(AssertionError):
        _pin_magnitudes(slip, _mag_inputs(0, O.KDT_BF16, False), _HEADS, exact_values=False)


def _slip_divide_by_B(vals, B):
    L = vals.shape[0]
    return np.stack([vals[s0:s0 + B].sum(axis=0) / B for s0 in range(0, L, B)])


def _slip_drop_partial(vals, B):
    L = vals.shape[0]
    return np.stack([vals[s0:s0 + B].mean(axis=0) for s0 in range(0, L - B + 1, B)])


def _slip_one_extra_key(vals, B):
    L = vals.shape[0]
    return np.stack([vals[s0:min(s0 + B + 1, L)].mean(axis=0) for s0 in range(0, L, B)])


@pytest.mark.parametrize("slip", [_slip_divide_by_B, _slip_drop_partial, _slip_one_extra_key])
def test_block_mean_pin_catches_slips(slip):
    inp = synth.random_small(3, T=1, L=23, H=2, d=6)
    with pytest.raises(AssertionError):
        _pin_full_block_means(slip, inp, 5)


def _slip_query_full_tail(P, t):
    """The query's last block taken over the whole block, past its position."""
    out = O.block_means(P, t)
    n = P.n(t)
    M = out.shape[0]
    if M and n % P.B:
        s0 = (M - 1) * P.B
        out[M - 1] = P.K[s0:min(s0 + P.B, P.L)].mean(axis=0)
    return out


def _slip_query_ignore_cache(P, t):
    Q = O.Problem.__new__(O.Problem)
    Q.__dict__.update(P.__dict__)
    Q.kbar = None
    return O.block_means(Q, t)


def test_query_block_mean_pin_catches_slips():
    inp = synth.random_small(4, T=4, L=30, H=2, d=5)
    inp["pos"] = np.array([29, 12, 0, 5], dtype=np.int32)
    with pytest.raises(AssertionError):
        _pin_query_block_means(_slip_query_full_tail, inp, 4)
    inp["kbar"] = np.random.default_rng(1).standard_normal((8, 5)).astype(np.float32)
    with pytest.raises(AssertionError):
        _pin_query_block_means(_slip_query_ignore_cache, inp, 4)
