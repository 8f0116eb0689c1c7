"""Exact selection on the GPU: every top-k, top-k' and top-m the library takes
is the first k items under (-score, index) of the scores it computed itself.

The scores are fetched from the library in the same launch configuration as
the selection (k >= n returns a whole score row: every visible key, ascending,
with its score), and the selection is then recomputed on the host with a
stable sort, so index sets must agree bit for bit; this pins the selection
kernels without any floating-point tolerance (the scores themselves are
checked against the oracle elsewhere).

Integer-grid inputs make every fp32 score exact, so there the selection must
also equal the oracle's (heavy exact ties, ties at zero across the cut from a
negative weight, a single huge outlier that crowds every other key into one
histogram bin).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import to_gpu

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _np(t):
    return t.cpu().numpy()


def _first_k(scores, idx, k):
    """First min(k, n) of the items under (-score, index); -0.0 == +0.0."""
    s = np.asarray(scores, dtype=np.float32).astype(np.float64) + 0.0
    order = np.lexsort((np.asarray(idx), -s))[: min(k, len(idx))]
    return np.asarray(idx)[order]


def _full_rows(idx, sc, n):
    """(indices, scores) of a take-everything call, checked to be the whole prefix."""
    rows = []
    for t in range(idx.shape[0]):
        assert np.array_equal(idx[t, : n[t]], np.arange(n[t])), f"row {t}: not the whole prefix"
        assert np.all(idx[t, n[t]:] == -1)
        rows.append(sc[t, : n[t]])
    return rows


def _assert_selection(sel_idx, sel_sc, full, k, label):
    for t, row in enumerate(full):
        kt = min(k, len(row))
        got = sel_idx[t, :kt].astype(np.int64)
        want = np.sort(_first_k(row, np.arange(len(row)), k))
        assert np.array_equal(got, want), f"{label} row {t}: selection differs from first-k of its scores"
        assert np.all(sel_idx[t, kt:] == -1), f"{label} row {t}: padding"
        assert np.array_equal(sel_sc[t, :kt].view(np.uint32), row[got].view(np.uint32)), \
            f"{label} row {t}: returned scores differ from the scored row"


def _n(inp, L):
    return np.minimum(np.maximum(inp["pos"].astype(np.int64) + 1, 0), L)


def _misa_exact(inp, B, A, k, heads=None):
    q, w, K, ks, pos = to_gpu(inp)
    L = K.shape[0]
    hd = None if heads is None else torch.from_numpy(np.ascontiguousarray(heads, dtype=np.int32)).cuda()
    fi, fs = S.score_topk(q, w, K, pos, B, A, L, ks, heads=hd)
    si, ss = S.score_topk(q, w, K, pos, B, A, k, ks, heads=hd)
    full = _full_rows(_np(fi), _np(fs), _n(inp, L))
    _assert_selection(_np(si), _np(ss), full, k, "misa")
    return full, _np(si)


@pytest.mark.parametrize("name", ["c1_tiny_decode", "c2_decode_batch", "c4_hier_decode_128k",
                                  "c5_glm5_hisa_128k"])
def test_misa_selection_is_first_k_of_its_scores(name):
    wl = synth.CONFIGS[name]
    _misa_exact(synth.make_inputs(wl, seed=0), wl.B, wl.A, wl.k)


def test_misa_selection_exact_c3_every_row():
    """Causal prefill T = L = 16384: the top-2048 of every row against a host
    sort of the same row's scores (rows of 1 .. 16384 keys)."""
    wl = synth.CONFIGS["c3_causal_prefill"]
    inp = synth.make_inputs(wl, seed=0)
    q, w, K, ks, pos = to_gpu(inp)
    L = wl.L
    fi, fs = S.score_topk(q, w, K, pos, wl.B, wl.A, L, ks)
    si, ss = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks)
    torch.cuda.synchronize()
    n = _n(inp, L)
    step = 1024
    for r0 in range(0, wl.T, step):
        rows = slice(r0, min(wl.T, r0 + step))
        fsc = _np(fs[rows])
        fidx = _np(fi[rows])
        nr = n[rows]
        col = np.arange(L)[None, :]
        vis = col < nr[:, None]
        assert np.array_equal(np.where(vis, fidx, -1), np.where(vis, col, -1)), "full rows are not whole prefixes"
        assert np.all(fidx[~vis] == -1)
        # stable sort on -score puts ties in index order; invisible columns last
        key = np.where(vis, -(fsc.astype(np.float64) + 0.0), np.inf)
        order = np.argsort(key, axis=1, kind="stable")[:, : wl.k]
        want = np.sort(order, axis=1)
        kt = np.minimum(wl.k, nr)
        lead = np.arange(wl.k)[None, :] < kt[:, None]
        got = _np(si[rows])
        gsc = _np(ss[rows])
        assert np.array_equal(np.where(lead, got, -1), np.where(lead, want, -1)), \
            f"rows {r0}..: selection differs from first-k of the scores"
        assert np.all(got[~lead] == -1)
        picked = np.take_along_axis(fsc, np.where(lead, got, 0), axis=1)
        assert np.array_equal(np.where(lead, gsc, 0).view(np.uint32), np.where(lead, picked, 0).view(np.uint32))


def _hier_exact(inp, B, A, kprime, k):
    q, w, K, ks, pos = to_gpu(inp)
    L = K.shape[0]
    n = _n(inp, L)
    fi, fs = S.score_topk(q, w, K, pos, B, A, L, ks)          # routed scores, whole rows
    routed = _full_rows(_np(fi), _np(fs), n)
    kc = min(kprime, L)
    ci, cs = S.hier_topk(q, w, K, pos, B, A, kprime, kc, ks)   # every candidate, reranked score
    hi, hs = S.hier_topk(q, w, K, pos, B, A, kprime, k, ks)
    ci, cs, hi, hs = _np(ci), _np(cs), _np(hi), _np(hs)
    for t in range(len(routed)):
        cand = np.sort(_first_k(routed[t], np.arange(n[t]), kprime))
        nc = len(cand)
        assert np.array_equal(ci[t, :nc], cand), f"hier row {t}: candidate set differs from top-k' of routed scores"
        assert np.all(ci[t, nc:] == -1)
        final = np.sort(_first_k(cs[t, :nc], cand, k))
        kt = min(k, nc)
        assert np.array_equal(hi[t, :kt], final), f"hier row {t}: final set differs from top-k of reranked scores"
        pos_in = np.searchsorted(cand, hi[t, :kt])
        assert np.array_equal(hs[t, :kt].view(np.uint32), cs[t, pos_in].view(np.uint32))


@pytest.mark.parametrize("name", ["c1_tiny_decode", "c4_hier_decode_128k"])
def test_hier_selections_exact(name):
    wl = synth.CONFIGS[name]
    kp = wl.kprime if name.startswith("c4") else 1024
    _hier_exact(synth.make_inputs(wl, seed=0), wl.B, wl.A, kp, wl.k)


def test_hier_selections_exact_random():
    inp = synth.random_small(71, T=9, L=20000, H=64, k_dtype=synth.KDT_FP8, positions="random")
    inp["pos"][0] = 0
    _hier_exact(inp, 128, 8, 3000, 700)


def test_hier_selections_exact_random_bf16():
    # long rows with bf16 keys and 40 heads (rows short of k' are taken whole)
    inp = synth.random_small(72, T=7, L=21000, H=40, k_dtype=synth.KDT_BF16, positions="random")
    inp["pos"][0] = 0
    _hier_exact(inp, 64, 5, 2500, 300)


def _hisa_exact(inp, B, m, k, maxpool=False):
    q, w, K, ks, pos = to_gpu(inp)
    L = K.shape[0]
    n = _n(inp, L)
    beta = _np(S.hisa_block_scores(q, w, K, pos, B, ks))
    f = S.hisa_maxpool_topk if maxpool else S.hisa_topk
    # k >= m B: every token of the chosen blocks is returned, so the blocks show
    ai, acs = f(q, w, K, pos, B, m, m * B, ks)
    si, ss = f(q, w, K, pos, B, m, k, ks)
    ai, acs, si, ss = _np(ai), _np(acs), _np(si), _np(ss)
    for t in range(len(n)):
        M = -(-int(n[t]) // B)
        if not maxpool:
            assert np.all(np.isfinite(beta[t, :M])) and np.all(np.isneginf(beta[t, M:]))
            blocks = np.sort(_first_k(beta[t, :M], np.arange(M), m))
            toks = np.concatenate([np.arange(b * B, min(b * B + B, n[t])) for b in blocks]) if len(blocks) \
                else np.zeros(0, dtype=np.int64)
            assert np.array_equal(ai[t, : len(toks)], toks), f"hisa row {t}: blocks differ from top-m of beta"
            assert np.all(ai[t, len(toks):] == -1)
        # the refine's top-k among the candidates, against the candidates' own scores
        cand = ai[t][ai[t] >= 0]
        cs = acs[t, : len(cand)]
        final = np.sort(_first_k(cs, cand, k))
        kt = min(k, len(cand))
        assert np.array_equal(si[t, :kt], final), f"hisa row {t}: final selection"


@pytest.mark.parametrize("name", ["c1_tiny_decode", "c5_glm5_hisa_128k"])
def test_hisa_selections_exact(name):
    wl = synth.CONFIGS[name]
    m = wl.m if name.startswith("c5") else 8
    _hisa_exact(synth.make_inputs(wl, seed=0), wl.B, m, wl.k)


def test_hisa_selections_exact_random_and_maxpool():
    inp = synth.random_small(72, T=7, L=9000, H=32, k_dtype=synth.KDT_FP8, positions="random")
    _hisa_exact(inp, 64, 12, 300)
    _hisa_exact(inp, 64, 12, 300, maxpool=True)


def test_block_scores_against_oracle():
    inp = synth.random_small(73, T=11, L=3000, H=64, k_dtype=synth.KDT_BF16, positions="random")
    q, w, K, ks, pos = to_gpu(inp)
    beta = _np(S.hisa_block_scores(q, w, K, pos, 100, ks))
    P = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], 100)
    for t in range(P.T):
        b = O.hisa_block_scores(P, t)
        rho = O.block_logits(P, t)
        mag = (np.abs(P.w[t])[:, None] * np.maximum(rho, 0)).sum(axis=0)
        # formed in float64 on the GPU, rounded once to float32
        assert np.all(np.abs(beta[t, : len(b)] - b) <= 1e-6 * mag + 1e-30), t
        assert np.all(np.isneginf(beta[t, len(b):]))


# ----------------------------------------------------------------- exact scores: integer grid

def _grid(seed, T, L, H, fp8=False, positions="random"):
    inp = synth.random_small(seed, T=T, L=L, H=H, positions=positions, int_grid=True)
    if fp8:
        # grid values are E4M3 values; a power-of-two scale keeps every product exact
        vals = synth.bf16_bits_to_f32(inp["K"])
        inp["K"] = synth.encode_e4m3fn(vals * np.float32(4.0))
        inp["k_scale"] = np.full(L, 0.25, dtype=np.float32)
    return inp


def _oracle_exact(inp, B, heads, k):
    kdt = O.KDT_FP8 if inp["k_scale"] is not None else O.KDT_BF16
    P = O.Problem(inp["q"], inp["w"], inp["K"], inp["pos"], B, kdt, inp["k_scale"])
    res, _ = O.misa_topk(P, heads.shape[1], k, heads=heads)
    return P, res


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("L", [3000, 16384, 40000])
def test_int_grid_selection_equals_oracle(L, fp8):
    """Exact scores: indices and scores equal the oracle's bit for bit, in the
    row kernel (L <= 16384) and the split long-row path (L > 16384)."""
    T, H, A, k = 6, 16, 4, 700
    inp = _grid(80 + L % 97, T, L, H, fp8=fp8, positions="decode" if L > 16384 else "random")
    heads = np.stack([np.sort(np.random.default_rng(t).choice(H, A, replace=False)) for t in range(T)])
    P, res = _oracle_exact(inp, 128, heads, k)
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.score_topk(q, w, K, pos, 128, A, k, ks, heads=torch.from_numpy(heads.astype(np.int32)).cuda())
    idx, sc = _np(idx), _np(sc)
    for t in range(T):
        oi, os_ = res[t]
        kt = len(oi)
        order = np.argsort(oi)
        assert np.array_equal(idx[t, :kt], oi[order]), f"row {t}"
        assert np.array_equal(sc[t, :kt].astype(np.float64), os_[order]), f"row {t} scores"


@pytest.mark.parametrize("L", [5000, 16384, 50000])
def test_zero_ties_across_the_cut(L):
    """One routed head with a negative weight: every key with q.k <= 0 scores
    exactly 0, the largest value, so the cut falls inside a tie of thousands of
    keys and the lowest indices must win."""
    T, H, k = 4, 8, 1500
    inp = _grid(90 + L % 89, T, L, H, positions="decode")
    heads = np.full((T, 1), 3, dtype=np.int64)
    inp["w"][:, 3] = np.float32(-0.5)
    P, res = _oracle_exact(inp, 128, heads, k)
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.score_topk(q, w, K, pos, 128, 1, k, ks, heads=torch.from_numpy(heads.astype(np.int32)).cuda())
    idx, sc = _np(idx), _np(sc)
    for t in range(T):
        oi, os_ = res[t]
        assert np.all(os_[: k] == 0.0)  # the cut lies inside the zero tie
        assert np.array_equal(idx[t], np.sort(oi)), f"row {t}"
        assert np.all(sc[t] == 0.0) and not np.any(np.signbit(sc[t])), f"row {t}: -0.0 or nonzero"


@pytest.mark.parametrize("L", [9000, 16384, 60000])
def test_single_outlier_crowds_the_bins(L):
    """One key far above the rest: bins spread linearly between a row's
    extremes put every other key into the lowest bin, so the threshold is
    found among a crowded bin (row kernel: digit search over all items; long
    rows: a boundary list larger than the on-chip list)."""
    T, H, A, k = 3, 8, 8, 2000
    inp = _grid(95 + L % 83, T, L, H, positions="decode")
    inp["w"][:] = np.abs(inp["w"]) + np.float32(0.5)  # positive weights: the outlier wins
    big = synth.encode_bf16(np.full((1, 128), 64.0, dtype=np.float32))
    inp["K"][L // 3] = big[0]
    heads = np.tile(np.arange(A), (T, 1))
    P, res = _oracle_exact(inp, 128, heads, k)
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.score_topk(q, w, K, pos, 128, A, k, ks)   # A = H: the dense indexer
    idx, sc = _np(idx), _np(sc)
    for t in range(T):
        oi, os_ = res[t]
        assert L // 3 in set(oi.tolist())
        order = np.argsort(oi)
        assert np.array_equal(idx[t], oi[order]), f"row {t}"
        assert np.array_equal(sc[t].astype(np.float64), os_[order]), f"row {t} scores"
