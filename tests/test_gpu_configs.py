"""GPU parity at the five full workload sizes, in the launch configuration the
benchmark times (same entry points, same shapes).

Every configuration is checked on every row, the causal prefill (16384 x
16384) included: routed heads bit for bit, then each row's selection and
scores against the oracle's within the score tolerance.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import RTOL, check_heads, check_row, oracle_problem, to_gpu, tolerance
from test_gpu_parity import _check_misa, check_hier, check_hisa, check_misa_hisa

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _np(t):
    return t.cpu().numpy()


def _inputs(name, seed=0):
    wl = synth.CONFIGS[name]
    return wl, synth.make_inputs(wl, seed=seed)


@pytest.mark.parametrize("name", ["c1_tiny_decode", "c2_decode_batch"])
def test_decode_misa(name):
    wl, inp = _inputs(name)
    q, w, K, ks, pos = to_gpu(inp)
    heads, r = S.route(q, w, K, pos, wl.B, wl.A, ks, with_r=True)
    idx, sc = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks)
    P = oracle_problem(inp, wl.B)
    heads_o, ill = check_heads(P, wl.A, _np(heads), _np(r))
    assert ill == 0
    _check_misa(inp, wl.B, wl.A, wl.k, _np(idx), _np(sc), heads_o, label=name)


def test_c1_all_paths():
    wl, inp = _inputs("c1_tiny_decode")
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.hier_topk(q, w, K, pos, wl.B, wl.A, 1024, wl.k, ks)
    check_hier(inp, wl.B, wl.A, 1024, wl.k, _np(idx), _np(sc), label="c1 hier")
    idx, sc = S.hisa_topk(q, w, K, pos, wl.B, 8, wl.k, ks)
    check_hisa(inp, wl.B, 8, wl.k, _np(idx), _np(sc), label="c1 hisa")
    idx, sc = S.score_topk(q, w, K, pos, wl.B, wl.H, wl.k, ks)   # dense DSA
    P = oracle_problem(inp, wl.B)
    dense = O.dense_topk(P, wl.k)
    allh = list(range(P.H))
    for t in range(P.T):
        check_row(_np(idx)[t], _np(sc)[t], wl.k, P.n(t), "ascending", dense[t][0],
                  lambda s, t=t: O.dense_scores(P, t, s),
                  lambda s, t=t: tolerance(P, t, allh, s, RTOL[O.KDT_BF16]), label=f"c1 dense {t}")


def test_c3_prefill_every_row():
    """Causal prefill T = L = 16384: routed heads, selection and scores of every
    one of the 16,384 rows against the oracle (run row by row, in parallel over
    the host cores)."""
    from oracle_pool import check_misa_all_rows
    wl, inp = _inputs("c3_causal_prefill")
    q, w, K, ks, pos = to_gpu(inp)
    heads = S.route(q, w, K, pos, wl.B, wl.A, ks)
    idx, sc = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks)
    torch.cuda.synchronize()
    gi, gs = _np(idx), _np(sc)
    # every row: min(k, n_t) indices, ascending, inside the visible prefix, then padding
    n = np.minimum(np.maximum(inp["pos"].astype(np.int64) + 1, 0), wl.L)
    kt = np.minimum(wl.k, n)
    lead = np.arange(wl.k)[None, :] < kt[:, None]
    assert np.array_equal(gi >= 0, lead), "selection counts or padding position"
    assert np.all(gi[~lead] == -1) and np.all(np.isneginf(gs[~lead])), "padding values"
    both = lead[:, 1:] & lead[:, :-1]
    assert np.all(np.diff(gi, axis=1)[both] > 0), "indices not strictly ascending"
    rows, ill, worst = check_misa_all_rows(inp, wl.B, wl.A, wl.k, _np(heads), gi, gs)
    print(f"c3: {rows} rows checked, worst error / tolerance {worst:.3e}")
    assert rows == wl.T and ill == 0


def test_c4_hier_decode():
    wl, inp = _inputs("c4_hier_decode_128k")
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.hier_topk(q, w, K, pos, wl.B, wl.A, wl.kprime, wl.k, ks)
    check_hier(inp, wl.B, wl.A, wl.kprime, wl.k, _np(idx), _np(sc), label="c4 hier")
    idx, sc = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks)
    _check_misa(inp, wl.B, wl.A, wl.k, _np(idx), _np(sc), label="c4 misa")


def test_c5_glm5_misa_and_hisa():
    wl, inp = _inputs("c5_glm5_hisa_128k")
    q, w, K, ks, pos = to_gpu(inp)
    heads = S.route(q, w, K, pos, wl.B, wl.A, ks)
    P = oracle_problem(inp, wl.B)
    _, ill = check_heads(P, wl.A, _np(heads))
    assert ill == 0
    idx, sc = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks)
    _check_misa(inp, wl.B, wl.A, wl.k, _np(idx), _np(sc), label="c5 misa")
    idx, sc = S.hisa_topk(q, w, K, pos, wl.B, wl.m, wl.k, ks)
    check_hisa(inp, wl.B, wl.m, wl.k, _np(idx), _np(sc), label="c5 hisa")
    idx, sc = S.hisa_maxpool_topk(q, w, K, pos, wl.B, wl.m, wl.k, ks)
    check_hisa(inp, wl.B, wl.m, wl.k, _np(idx), _np(sc), label="c5 hisa max-pool", pool="max")
    heads_o, _ = O.route(P, wl.A)
    idx, sc = S.misa_hisa_topk(q, w, K, pos, wl.B, wl.A, wl.m, wl.k, ks)
    check_misa_hisa(inp, wl.B, wl.A, wl.m, wl.k, _np(idx), _np(sc), heads_o, label="c5 misa-hisa")
