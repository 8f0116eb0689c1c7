"""Pins for the oracle with fp8 queries (no GPU).

Queries may come as OCP E4M3FN codes with one fp32 scale per (query, head);
the value of q[t,h,i] is code * q_scale[t,h] and every definition is unchanged.
Pinned by: the decoder against torch's cast times the scale (exact in
float64); exact rational brute force of routing, scores and selections on tiny
inputs; the invariants A = H => dense, k' >= n => dense, m*B >= n => dense;
scaling laws of q_scale (x2 doubles every score exactly, a sign flip of a
head's scale is the same as negating its codes); needle recall of the dense
indexer at the 128K shape with fp8 queries.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth


def _P(inp, B):
    kdt = O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16
    return O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B, kdt, inp["k_scale"],
                     q_dtype=O.QDT_FP8, q_scale=inp["q_scale"])


def test_fp8_query_decode_is_code_times_scale():
    inp = synth.random_small(1, T=3, L=5, H=4, d=16, q_fp8=True)
    inp["q_scale"][0, 1] = -inp["q_scale"][0, 1]          # a negative scale flips the sign
    got = O.dequant_queries(inp["q"], O.QDT_FP8, inp["q_scale"])
    codes = torch.from_numpy(inp["q"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = codes * inp["q_scale"].astype(np.float64)[:, :, None]
    assert np.array_equal(got, ref)
    assert np.array_equal(got[0, 1], -codes[0, 1] * abs(float(inp["q_scale"][0, 1])))
    # the generator's codes reproduce q to E4M3 precision (relative 2^-4 of the row's range)
    q32 = np.random.default_rng(np.random.SeedSequence([1, 3, 5, 4, 16, 0])).standard_normal((3, 4, 16), dtype=np.float32).astype(np.float64)
    assert np.all(np.abs(got[1:] - q32[1:]) <= 2.0 ** -4 * np.abs(q32[1:]).max(axis=2, keepdims=True) + 1e-12)


def _frac(v):
    return np.vectorize(lambda x: Fraction(float(x)), otypes=[object])(np.asarray(v, dtype=np.float64))


def _rank_select(vals, k):
    n = len(vals)
    return [i for i in range(n)
            if sum(1 for j in range(n) if vals[j] > vals[i] or (vals[j] == vals[i] and j < i)) < k]


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("B", [1, 3, 4])
def test_exact_brute_force_fp8_queries(seed, B):
    """Routing, MISA, dense and HISA on tiny fp8-query inputs against exact
    rational arithmetic (values from torch's decoders, not the oracle's)."""
    inp = synth.random_small(200 + seed, T=3, L=16, H=4, d=8, k_dtype=synth.KDT_FP8, q_fp8=True)
    inp["q_scale"][1, 2] *= np.float32(-1.0)
    P = _P(inp, B)
    codes_q = torch.from_numpy(inp["q"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes_k = torch.from_numpy(inp["K"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    q = _frac(codes_q) * _frac(inp["q_scale"])[:, :, None]
    K = _frac(codes_k) * _frac(inp["k_scale"])[:, None]
    w = _frac(inp["w"])
    A, k, m = 2, 4, 2
    heads, r = O.route(P, A)
    dot = lambda a, b: sum((x * y for x, y in zip(a, b)), Fraction(0))
    for t in range(P.T):
        n = P.n(t)
        blocks = [(b0, min(b0 + B, n)) for b0 in range(0, n, B)]
        means = [[sum((K[s, i] for s in range(b0, b1)), Fraction(0)) / (b1 - b0) for i in range(P.d)]
                 for b0, b1 in blocks]
        rx = [w[t, h] * max([Fraction(0)] + [dot(q[t, h], mb) for mb in means]) for h in range(P.H)]
        assert np.allclose([float(v) for v in rx], r[t], rtol=1e-13, atol=1e-300)
        srt = sorted(rx, reverse=True)
        if srt[A - 1] - srt[A] > Fraction(1, 10 ** 9):
            assert sorted(_rank_select(rx, A)) == list(heads[t])
        score = lambda s, hs: sum((w[t, h] * max(Fraction(0), dot(q[t, h], K[s])) for h in hs), Fraction(0))
        ir = [score(s, heads[t]) for s in range(n)]
        ia = [score(s, range(P.H)) for s in range(n)]
        got = O.routed_scores(P, t, heads[t], np.arange(n))
        assert np.allclose(got, [float(v) for v in ir], rtol=1e-13, atol=1e-300)
        if n > k:
            srt = sorted(ir, reverse=True)
            if srt[k - 1] - srt[k] > Fraction(1, 10 ** 9):
                assert sorted(O.misa_topk(P, A, k, heads=heads)[0][t][0]) == sorted(_rank_select(ir, k))
            srt = sorted(ia, reverse=True)
            if srt[k - 1] - srt[k] > Fraction(1, 10 ** 9):
                assert sorted(O.dense_topk(P, k)[t][0]) == sorted(_rank_select(ia, k))
        beta = [sum((w[t, h] * max(Fraction(0), dot(q[t, h], mb)) for h in range(P.H)), Fraction(0)) for mb in means]
        assert np.allclose(O.hisa_block_scores(P, t), [float(v) for v in beta], rtol=1e-13, atol=1e-300)


def _medium(seed):
    inp = synth.random_small(seed, T=6, L=600, H=16, d=32, k_dtype=synth.KDT_FP8, q_fp8=True)
    inp["pos"][0] = 0
    inp["pos"][1] = 599
    return inp


def _same(a, b):
    for (i1, s1), (i2, s2) in zip(a, b):
        assert list(i1) == list(i2)
        assert np.array_equal(s1, s2)


def test_fp8_query_invariants():
    inp = _medium(11)
    P = _P(inp, 64)
    res, heads = O.misa_topk(P, P.H, 40)
    assert (heads == np.arange(P.H)).all()
    for (i1, s1), (i2, s2) in zip(res, O.dense_topk(P, 40)):         # A = H: dense (the two sum
        assert list(i1) == list(i2)                                   # the heads in different orders)
        assert np.allclose(s1, s2, rtol=1e-12, atol=1e-12)
    _same(O.misa_hier_topk(P, 4, 600, 40)[0], O.dense_topk(P, 40))    # k' >= n: dense
    _same(O.hisa_topk(P, 10, 40)[0], O.dense_topk(P, 40))             # m B >= n: dense


def test_fp8_query_scale_laws():
    inp = _medium(12)
    P = _P(inp, 64)
    base, heads = O.misa_topk(P, 4, 50)
    two = dict(inp, q_scale=(inp["q_scale"] * np.float32(2.0)).astype(np.float32))
    P2 = _P(two, 64)
    res2, heads2 = O.misa_topk(P2, 4, 50)
    assert np.array_equal(heads, heads2)
    for (i1, s1), (i2, s2) in zip(base, res2):
        assert list(i1) == list(i2)
        assert np.array_equal(s1 * 2.0, s2)
    # a negative scale on a head is the same as negating that head's codes
    neg = dict(inp, q_scale=inp["q_scale"].copy(), q=inp["q"].copy())
    neg["q_scale"][:, 3] *= np.float32(-1.0)
    flip = dict(inp, q=inp["q"].copy())
    flip["q"][:, 3] ^= np.uint8(0x80)
    assert np.array_equal(_P(neg, 64).q, _P(flip, 64).q)


@pytest.mark.slow
def test_needles_found_by_dense_oracle_with_fp8_queries():
    wl = synth.CONFIGS["c4_hier_decode_128k"]
    inp = synth.make_inputs(wl, seed=0, q_fp8=True)
    rows = [0, wl.T - 1]
    sub = dict(inp, q=inp["q"][rows], w=inp["w"][rows], pos=inp["pos"][rows], q_scale=inp["q_scale"][rows])
    P = _P(sub, wl.B)
    res = O.dense_topk(P, wl.k)
    for i, t in enumerate(rows):
        chosen = set(int(s) for s in res[i][0])
        assert all(int(s) in chosen for s in inp["needles"][t])
