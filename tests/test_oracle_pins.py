"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * the bf16 / E4M3FN decoders against torch's own casts (library routines);
  * a hand-derived worked example (tests/golden/hand_example.json);
  * exhaustive rank counting in exact rational arithmetic on tiny inputs, which
    characterises "first k under (-score, index)" without sorting;
  * invariants the method must satisfy: A = H gives the dense indexer, k' >= n
    gives the dense indexer, m*B >= n gives the dense indexer, k' = k gives the
    MISA set, B = 1 and B >= n closed forms of the router, causality, ReLU
    non-negativity, exact scaling in w, block-mean linearity;
  * a special case that reduces to numpy's stable argsort.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ decoders

def test_decode_bf16_matches_torch_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    # signed zeros decode with their sign
    assert np.signbit(O.decode_bf16(np.array([0x8000], dtype=np.uint16)))[0]


def test_decode_e4m3fn_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert got[1] == 2.0 ** -9          # smallest subnormal
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_fp8_dequant_is_code_times_scale():
    codes = synth.encode_e4m3fn(np.array([[2.0, -0.5], [448.0, 0.0]], dtype=np.float32))
    vals = O.dequant_keys(codes, O.KDT_FP8, np.array([0.25, 3.0], dtype=np.float32))
    assert np.array_equal(vals, np.array([[0.5, -0.125], [1344.0, 0.0]]))


# ------------------------------------------------------------------ worked example

def _hand_problem(fp8=False):
    g = json.load(open(os.path.join(HERE, "golden", "hand_example.json")))
    q = synth.encode_bf16(np.array(g["q"], dtype=np.float32))
    w = np.array(g["w"], dtype=np.float32)
    pos = np.array(g["pos"], dtype=np.int32)
    if fp8:
        K = synth.encode_e4m3fn(np.array(g["fp8_codes_as_values"], dtype=np.float32))
        P = O.Problem(q, w, K, pos, g["B"], O.KDT_FP8, np.array(g["fp8_scale"], dtype=np.float32))
    else:
        K = synth.encode_bf16(np.array(g["K"], dtype=np.float32))
        P = O.Problem(q, w, K, pos, g["B"])
    return P, g["expect"]


def _check_results(res, expect):
    assert len(res) == len(expect)
    for (idx, sc), e in zip(res, expect):
        assert list(idx) == e["idx"]
        assert list(sc) == [float(v) for v in e["scores"]]
        assert not np.any(np.signbit(sc) & (sc == 0))   # no -0.0 leaks out


@pytest.mark.parametrize("fp8", [False, True])
def test_hand_example(fp8):
    P, E = _hand_problem(fp8)
    heads, r = O.route(P, 1)
    assert heads.tolist() == E["route_A1_heads"]
    assert r.tolist() == E["route_r"]
    assert not np.any(np.signbit(r) & (r == 0))
    heads2, _ = O.route(P, 2)
    assert heads2.tolist() == E["route_A2_heads"]
    for t in range(P.T):
        assert O.dense_scores(P, t, np.arange(P.n(t))).tolist() == E["dense_scores"][t]
        assert O.hisa_block_scores(P, t).tolist() == E["hisa_beta"][t]
    _check_results(O.misa_topk(P, 1, 2)[0], E["misa_A1_k2"])
    _check_results(O.misa_topk(P, 1, 4)[0], E["misa_A1_k4"])
    _check_results(O.misa_topk(P, 1, 2, heads=np.zeros((P.T, 1), dtype=np.int64))[0],
                   E["routed_head0_k2"])
    _check_results(O.dense_topk(P, 2), E["dense_k2"])
    _check_results(O.dense_topk(P, 3), E["dense_k3"])
    _check_results(O.misa_hier_topk(P, 1, 2, 1)[0], E["hier_A1_kp2_k1"])
    _check_results(O.misa_hier_topk(P, 1, 3, 2)[0], E["hier_A1_kp3_k2"])
    res, blocks = O.hisa_topk(P, 1, 2)
    assert [list(b) for b in blocks] == E["hisa_m1_blocks"]
    _check_results(res, E["hisa_m1_k2"])


# ------------------------------------------------------------------ exact brute force

def _frac_bf16(bits):
    # widening bf16 -> fp32 by a 16-bit shift is exact; Fraction(float) is exact
    f = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.vectorize(lambda v: Fraction(float(v)), otypes=[object])(f)


def _rank_select(vals, k):
    """Brute force: item i is chosen iff fewer than k items beat it, where j
    beats i when vals[j] > vals[i] or (equal and j < i).  No sorting."""
    n = len(vals)
    chosen = []
    for i in range(n):
        beaten = sum(1 for j in range(n) if vals[j] > vals[i] or (vals[j] == vals[i] and j < i))
        if beaten < k:
            chosen.append(i)
    return chosen


class Exact:
    """Exact rational evaluation of the definitions on tiny inputs."""

    def __init__(self, inp, B):
        self.q = _frac_bf16(inp["q"])
        self.w = np.vectorize(lambda v: Fraction(float(v)), otypes=[object])(inp["w"])
        self.K = _frac_bf16(inp["K"])
        self.pos = inp["pos"]
        self.B = B
        self.T, self.H, self.d = self.q.shape
        self.L = self.K.shape[0]

    def n(self, t):
        return int(min(max(int(self.pos[t]) + 1, 0), self.L))

    def dot(self, a, b):
        return sum((x * y for x, y in zip(a, b)), Fraction(0))

    def score(self, t, s, heads):
        return sum((self.w[t, h] * max(Fraction(0), self.dot(self.q[t, h], self.K[s])) for h in heads),
                   Fraction(0))

    def kbar(self, t):
        n, out = self.n(t), []
        for b0 in range(0, n, self.B):
            b1 = min(b0 + self.B, n)
            out.append([sum((self.K[s, i] for s in range(b0, b1)), Fraction(0)) / (b1 - b0)
                        for i in range(self.d)])
        return out

    def kmax(self, t):
        n, out = self.n(t), []
        for b0 in range(0, n, self.B):
            b1 = min(b0 + self.B, n)
            out.append([max(self.K[s, i] for s in range(b0, b1)) for i in range(self.d)])
        return out

    def beta_max(self, t):
        return [sum((self.w[t, h] * max(Fraction(0), self.dot(self.q[t, h], c)) for h in range(self.H)),
                    Fraction(0)) for c in self.kmax(t)]

    def r(self, t):
        kb = self.kbar(t)
        return [self.w[t, h] * max([Fraction(0)] + [self.dot(self.q[t, h], c) for c in kb])
                for h in range(self.H)]

    def beta(self, t, heads=None):
        heads = range(self.H) if heads is None else heads
        return [sum((self.w[t, h] * max(Fraction(0), self.dot(self.q[t, h], c)) for h in heads),
                    Fraction(0)) for c in self.kbar(t)]


def _tiny(seed, int_grid, T=3, L=20, H=4, d=8, positions="random"):
    return synth.random_small(seed, T=T, L=L, H=H, d=d, int_grid=int_grid, positions=positions)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("B", [1, 2, 4])
def test_exact_brute_force_int_grid(seed, B):
    """Dyadic inputs with power-of-two block counts keep every oracle value
    exact in float64, so sets, ties and values must match the exact brute
    force bit for bit (exact ties are common on this grid)."""
    inp = _tiny(seed, True)
    # prefix lengths 20, 10, 6: every block (tails included) holds 1, 2 or 4 keys
    inp["pos"] = np.array([19, 9, 5], dtype=np.int32)
    P = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B)
    X = Exact(inp, B)
    A, k, kp, m = 2, 3, 5, 2
    heads, r = O.route(P, A)
    for t in range(X.T):
        rx = X.r(t)
        assert [float(v) for v in rx] == list(r[t])
        assert sorted(_rank_select(rx, A)) == list(heads[t])
        n = X.n(t)
        ir = [X.score(t, s, heads[t]) for s in range(n)]
        ia = [X.score(t, s, range(X.H)) for s in range(n)]
        # MISA
        (gi, gs), = [O.misa_topk(P, A, k, heads=heads)[0][t]]
        assert sorted(gi) == sorted(_rank_select(ir, k))
        assert [float(ir[s]) for s in gi] == list(gs)
        # dense
        di, ds = O.dense_topk(P, k)[t]
        assert sorted(di) == sorted(_rank_select(ia, k))
        # MISA-dagger
        cand = _rank_select(ir, kp)
        final = [cand[j] for j in _rank_select([ia[s] for s in cand], k)]
        hi, _ = O.misa_hier_topk(P, A, kp, k, heads=heads)[0][t]
        assert sorted(hi) == sorted(final)
        # HISA
        bx = X.beta(t)
        blocks = _rank_select(bx, m)
        cand = [s for b in blocks for s in range(b * B, min((b + 1) * B, n))]
        final = [cand[j] for j in _rank_select([ia[s] for s in cand], k)]
        (si, _), bl = O.hisa_topk(P, m, k)[0][t], O.hisa_topk(P, m, k)[1][t]
        assert list(bl) == blocks
        assert sorted(si) == sorted(final)
        # HISA with max-pooled representatives
        blocks = _rank_select(X.beta_max(t), m)
        cand = [s for b in blocks for s in range(b * B, min((b + 1) * B, n))]
        final = [cand[j] for j in _rank_select([ia[s] for s in cand], k)]
        res, xbl = O.hisa_topk(P, m, k, pool="max")
        assert [float(v) for v in X.beta_max(t)] == list(O.hisa_block_scores(P, t, "max"))
        assert list(xbl[t]) == blocks
        assert sorted(res[t][0]) == sorted(final)
        # MISA inside HISA: the routed heads in both stages
        blocks = _rank_select(X.beta(t, heads[t]), m)
        cand = [s for b in blocks for s in range(b * B, min((b + 1) * B, n))]
        final = [cand[j] for j in _rank_select([ir[s] for s in cand], k)]
        res, mbl, _ = O.misa_hisa_topk(P, A, m, k, heads=heads)
        mi, ms = res[t]
        assert list(mbl[t]) == blocks
        assert sorted(mi) == sorted(final)
        assert [float(ir[s]) for s in mi] == list(ms)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("B", [3, 5, 32])
def test_exact_brute_force_random_values(seed, B):
    """Gaussian bf16 inputs: values agree with the exact ones to float64
    rounding, and selections agree wherever the exact margin at the cut is
    not itself at rounding level."""
    inp = _tiny(100 + seed, False, L=24)
    P = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B)
    X = Exact(inp, B)
    A, k = 2, 5
    heads, r = O.route(P, A)
    for t in range(X.T):
        rx = X.r(t)
        assert np.allclose([float(v) for v in rx], r[t], rtol=1e-13, atol=1e-15)
        srt = sorted(rx, reverse=True)
        if srt[A - 1] - srt[A] > Fraction(1, 10 ** 9):
            assert sorted(_rank_select(rx, A)) == list(heads[t])
        n = X.n(t)
        ir = [X.score(t, s, heads[t]) for s in range(n)]
        ref = np.array([float(v) for v in ir])
        got = O.routed_scores(P, t, heads[t], np.arange(n))
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-14)
        if n > k:
            srt = sorted(ir, reverse=True)
            if srt[k - 1] - srt[k] > Fraction(1, 10 ** 9):
                gi, _ = O.misa_topk(P, A, k, heads=heads)[0][t]
                assert sorted(gi) == sorted(_rank_select(ir, k))


# ------------------------------------------------------------------ invariants

def _medium(seed, k_dtype=O.KDT_BF16, T=6, L=700, H=16, d=32, positions="random"):
    inp = synth.random_small(seed, T=T, L=L, H=H, d=d, k_dtype=k_dtype, positions=positions)
    inp["pos"][0] = 0          # a single visible key
    inp["pos"][1] = L - 1      # the whole array
    return inp


def _P(inp, B):
    return O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B,
                     O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16, inp["k_scale"])


def _same(a, b):
    for (i1, s1), (i2, s2) in zip(a, b):
        assert list(i1) == list(i2)
        assert np.array_equal(s1, s2)


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
def test_A_equals_H_is_dense(kdt):
    inp = _medium(1, kdt)
    P = _P(inp, 64)
    res, heads = O.misa_topk(P, P.H, 50)
    assert (heads == np.arange(P.H)).all()
    dense = O.dense_topk(P, 50)
    for (i1, s1), (i2, s2) in zip(res, dense):
        assert list(i1) == list(i2)
        assert np.allclose(s1, s2, rtol=1e-12, atol=1e-12)


def test_kprime_covering_prefix_is_dense():
    inp = _medium(2)
    P = _P(inp, 64)
    res = O.misa_hier_topk(P, 4, P.L, 40)[0]
    _same(res, O.dense_topk(P, 40))


def test_kprime_equal_k_gives_misa_set():
    inp = _medium(3)
    P = _P(inp, 64)
    hier = O.misa_hier_topk(P, 4, 40, 40)[0]
    misa = O.misa_topk(P, 4, 40)[0]
    for (i1, _), (i2, _) in zip(hier, misa):
        assert sorted(i1) == sorted(i2)


def test_hisa_covering_prefix_is_dense():
    inp = _medium(4)
    for B, m in [(64, 11), (100, 7), (700, 1)]:
        P = _P(inp, B)
        _same(O.hisa_topk(P, m, 33)[0], O.dense_topk(P, 33))


def test_hisa_token_blocks_is_dense():
    """B = 1 makes every block one token and beta the dense score, so keeping
    m >= k blocks reproduces the dense top-k."""
    inp = _medium(5, L=300)
    P = _P(inp, 1)
    _same(O.hisa_topk(P, 40, 25)[0], O.dense_topk(P, 25))


def test_misa_hisa_all_heads_is_hisa():
    """A = H routes every head, so both stages use all heads: HISA."""
    inp = _medium(7)
    for B, m in [(64, 3), (37, 5)]:
        P = _P(inp, B)
        res, blocks, heads = O.misa_hisa_topk(P, P.H, m, 30)
        assert (heads == np.arange(P.H)).all()
        ref, ref_blocks = O.hisa_topk(P, m, 30)
        for t in range(P.T):
            assert list(blocks[t]) == list(ref_blocks[t])
            assert list(res[t][0]) == list(ref[t][0])
            assert np.allclose(res[t][1], ref[t][1], rtol=1e-12, atol=1e-12)


def test_misa_hisa_covering_prefix_is_misa():
    """m * B >= n_t keeps every block, so the refine stage is MISA itself."""
    inp = _medium(8)
    for B, m in [(64, 11), (700, 1)]:
        P = _P(inp, B)
        res, _, heads = O.misa_hisa_topk(P, 4, m, 33)
        _same(res, O.misa_topk(P, 4, 33, heads=heads)[0])


def test_misa_hisa_token_blocks_is_misa():
    """B = 1 makes beta_R the routed token score, so m >= k blocks give MISA's top-k."""
    inp = _medium(9, L=300)
    P = _P(inp, 1)
    res, _, heads = O.misa_hisa_topk(P, 3, 40, 25)
    _same(res, O.misa_topk(P, 3, 25, heads=heads)[0])


def test_router_block_size_one_closed_form():
    inp = _medium(6, L=200)
    P = _P(inp, 1)
    _, r = O.route(P, 3)
    for t in range(P.T):
        z = O.head_logits(P, t, range(P.H), np.arange(P.n(t)))
        assert np.allclose(r[t], P.w[t] * np.maximum(z, 0).max(axis=1), rtol=1e-13, atol=1e-15)


def test_router_single_block_closed_form():
    inp = _medium(7, L=200)
    P = _P(inp, 4096)
    _, r = O.route(P, 3)
    for t in range(P.T):
        mean = P.K[: P.n(t)].mean(axis=0)
        assert np.allclose(r[t], P.w[t] * np.maximum(P.q[t] @ mean, 0), rtol=1e-12, atol=1e-15)


def test_block_mean_linearity():
    """q . Kbar_b equals the mean over the block of the per-key logits z."""
    inp = _medium(8)
    for B in [7, 64, 128]:
        P = _P(inp, B)
        for t in range(P.T):
            n = P.n(t)
            z = O.head_logits(P, t, range(P.H), np.arange(n))
            rho = O.block_logits(P, t)
            for b, (s0, s1) in enumerate(O.block_ranges(n, B)):
                assert np.allclose(rho[:, b], z[:, s0:s1].mean(axis=1), rtol=1e-11, atol=1e-12)


def test_causality():
    """Changing keys after pos[t] leaves query t's routing, scores and
    selections unchanged; no selected index lies beyond pos[t]."""
    inp = _medium(9)
    t = 2
    K2 = inp["K"].copy()
    K2[inp["pos"][t] + 1:] = synth.encode_bf16(np.full((1, K2.shape[1]), 7.0, dtype=np.float32))

    def one(K):
        return O.Problem(inp["q"][t:t + 1], inp["w"][t:t + 1], K, inp["pos"][t:t + 1], 64)

    a, b = O.misa_topk(one(inp["K"]), 4, 30), O.misa_topk(one(K2), 4, 30)
    assert (a[1] == b[1]).all()
    _same(a[0], b[0])
    _same(O.hisa_topk(one(inp["K"]), 3, 30)[0], O.hisa_topk(one(K2), 3, 30)[0])
    _same(O.misa_hier_topk(one(inp["K"]), 4, 60, 30)[0], O.misa_hier_topk(one(K2), 4, 60, 30)[0])
    P1 = _P(inp, 64)
    for t2, (idx, _) in enumerate(O.misa_topk(P1, 4, 10 ** 6)[0]):
        assert idx.max(initial=-1) <= inp["pos"][t2] and len(idx) == P1.n(t2)


def test_relu_nonnegativity_and_zero_keys():
    inp = _medium(10)
    inp["w"] = np.abs(inp["w"])
    inp["K"][5] = 0                     # a zero key scores exactly zero
    P = _P(inp, 64)
    for t in range(P.T):
        keys = np.arange(P.n(t))
        sc = O.dense_scores(P, t, keys)
        assert (sc >= 0).all()
        if P.n(t) > 5:
            assert sc[5] == 0.0 and not np.signbit(sc[5])


def test_weight_doubling_scales_exactly():
    inp = _medium(11)
    P1 = _P(inp, 64)
    P2 = _P(dict(inp, w=inp["w"] * np.float32(2)), 64)
    h1, r1 = O.route(P1, 4)
    h2, r2 = O.route(P2, 4)
    assert (h1 == h2).all() and np.array_equal(r2, 2 * r1)
    for (i1, s1), (i2, s2) in zip(O.misa_topk(P1, 4, 25)[0], O.misa_topk(P2, 4, 25)[0]):
        assert list(i1) == list(i2) and np.array_equal(s2, 2 * s1)


def test_single_head_unit_weight_is_stable_argsort():
    """H = 1, w = 1: the selection is numpy's stable argsort of -ReLU(z)."""
    inp = synth.random_small(12, T=4, L=300, H=1, d=16)
    inp["w"][:] = 1.0
    P = _P(inp, 16)
    res, _ = O.misa_topk(P, 1, 37)
    for t, (idx, sc) in enumerate(res):
        z = O.head_logits(P, t, [0], np.arange(P.n(t)))[0]
        ref = np.argsort(-np.maximum(z, 0), kind="stable")[:37]
        assert list(idx) == list(ref)


def test_hisa_candidate_fraction_closed_form():
    """With full blocks, HISA scores exactly m*B of the L prefix tokens:
    64*128/131072 = 6.25 % at a 128K context (the pages report about 6 %)."""
    inp = synth.random_small(13, T=2, L=4096, H=2, d=8, positions="decode")
    P = _P(inp, 128)
    _, blocks = O.hisa_topk(P, 2, 10)
    for t, bl in enumerate(blocks):
        sizes = [min((b + 1) * 128, P.n(t)) - b * 128 for b in bl]
        assert len(bl) == 2
        assert sum(sizes) <= 2 * 128
    assert 64 * 128 / 131072 == 0.0625


def test_rows_shorter_than_k_take_everything():
    inp = _medium(14)
    inp["pos"][:] = np.array([0, 3, 9, 20, 31, 2])
    P = _P(inp, 8)
    for t, (idx, sc) in enumerate(O.misa_topk(P, 3, 32)[0]):
        assert sorted(idx) == list(range(P.n(t)))


# ------------------------------------------------------- cached block means

def _exact_block_means_f32(P):
    """Means of every block of the whole key array, from an explicit loop; on a
    dyadic grid with power-of-two blocks they are exact in float32."""
    M = -(-P.L // P.B)
    out = np.zeros((M, P.d), dtype=np.float32)
    for b in range(M):
        s0, s1 = b * P.B, min((b + 1) * P.B, P.L)
        acc = np.zeros(P.d)
        for s in range(s0, s1):
            acc += P.K[s]
        out[b] = acc / (s1 - s0)
        assert np.array_equal(out[b].astype(np.float64), acc / (s1 - s0))  # exact in fp32
    return out


@pytest.mark.parametrize("B", [2, 4, 8])
def test_cached_exact_means_change_nothing(B):
    """Cached means equal to the pooled ones give the same routes, block scores
    and selections, bit for bit."""
    inp = synth.random_small(11, T=5, L=60, H=6, d=16, int_grid=True, positions="random")
    P = _P(inp, B)
    kbar = _exact_block_means_f32(P)
    Pc = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B, O.KDT_BF16, None, kbar=kbar)
    h1, r1 = O.route(P, 3)
    h2, r2 = O.route(Pc, 3)
    assert np.array_equal(h1, h2) and np.array_equal(r1, r2)
    for t in range(P.T):
        assert np.array_equal(O.hisa_block_scores(P, t), O.hisa_block_scores(Pc, t))
    _same(O.misa_topk(P, 3, 9)[0], O.misa_topk(Pc, 3, 9)[0])
    _same(O.hisa_topk(P, 2, 9)[0], O.hisa_topk(Pc, 2, 9)[0])


def test_cached_means_closed_form():
    """With arbitrary cached rows, r(t,h) = w * max(0, max over the complete
    earlier blocks of q.kbar_b, q.mean(last block)) -- written out per head
    here -- and the cached row of the query's own last block is never read."""
    inp = synth.random_small(12, T=6, L=90, H=5, d=8, positions="random")
    B = 16
    P = _P(inp, B)
    M = -(-P.L // B)
    rng = np.random.default_rng(3)
    kbar = rng.standard_normal((M, P.d)).astype(np.float32)
    Pc = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B, O.KDT_BF16, None, kbar=kbar)
    _, r = O.route(Pc, 2)
    for t in range(P.T):
        n = P.n(t)
        Mt = -(-n // B)
        for h in range(P.H):
            best = 0.0
            for b in range(Mt - 1):
                best = max(best, float(np.dot(P.q[t, h], kbar[b].astype(np.float64))))
            if Mt > 0:
                s0 = (Mt - 1) * B
                tail = P.K[s0:n].sum(axis=0) / (n - s0)
                best = max(best, float(np.dot(P.q[t, h], tail)))
            assert np.isclose(r[t, h], P.w[t, h] * best, rtol=1e-12, atol=1e-14)
        # poisoning the row of the query's own last block changes nothing
        if Mt > 0:
            k2 = kbar.copy()
            k2[Mt - 1] = 1e6
            P2 = O.Problem(inp["q"][t:t + 1], inp["w"][t:t + 1], inp["K"], inp["pos"][t:t + 1], B,
                           O.KDT_BF16, None, kbar=k2)
            assert np.array_equal(O.route(P2, 2)[1][0], r[t])


def test_hisa_max_pool_reductions():
    """Max pooling reduces to mean pooling where the two representatives agree:
    blocks of one key (B = 1), and blocks whose keys are all equal; elsewhere
    the max-pooled representative dominates the mean in every dimension."""
    inp = _tiny(7, False, T=4, L=40, H=4, d=16)
    P1 = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], 1)
    a, b = O.hisa_topk(P1, 5, 6), O.hisa_topk(P1, 5, 6, pool="max")
    for t in range(P1.T):
        assert list(a[1][t]) == list(b[1][t])
        assert list(a[0][t][0]) == list(b[0][t][0])
    B = 4
    K = inp["K"].copy()
    for b0 in range(0, K.shape[0], B):
        K[b0:b0 + B] = K[b0]  # every block holds one key B times
    PB = O.Problem(inp["q"], inp["w"], K, inp["pos"], B)
    for t in range(PB.T):
        assert np.array_equal(O.hisa_block_scores(PB, t), O.hisa_block_scores(PB, t, "max"))
    P4 = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B)
    for t in range(P4.T):
        assert np.all(O.block_maxima(P4, t) >= O.block_means(P4, t))


def test_hisa_max_pool_keeps_a_needle_block():
    """Hand-built case (d = 2, one head, w = 1, q = (1, 0)): block 0 holds keys
    (4, 0) and (-4, 0), whose mean (0, 0) scores 0 while its maximum (4, 0)
    scores 4; block 1 holds (1, 0) twice and scores 1 either way.  With m = 1
    mean pooling keeps block 1 and misses the key that scores 4; max pooling
    keeps block 0 and finds it."""
    bf = lambda v: np.array(v, dtype=np.float32).view(np.uint32) >> 16
    q = bf([[[1.0, 0.0]]]).astype(np.uint16)
    K = bf([[4.0, 0.0], [-4.0, 0.0], [1.0, 0.0], [1.0, 0.0]]).astype(np.uint16)
    P = O.Problem(q, np.ones((1, 1), np.float32), K, np.array([3], np.int32), 2)
    assert list(O.hisa_block_scores(P, 0)) == [0.0, 1.0]
    assert list(O.hisa_block_scores(P, 0, "max")) == [4.0, 1.0]
    (mi, ms), = O.hisa_topk(P, 1, 1)[0]
    (xi, xs), = O.hisa_topk(P, 1, 1, pool="max")[0]
    assert (list(mi), list(ms)) == ([2], [1.0])
    assert (list(xi), list(xs)) == ([0], [4.0])
