"""The benchmark's selection-quality report (IoU with the dense top-k, recall of
planted needles; the synthetic stand-ins for the pages' IoU and
needle-in-a-haystack measurements) computed from the GPU's selections agrees
with the same report computed from the oracle's selections.

The GPU's sets may differ from the oracle's only by swaps inside the score
tolerance (the parity tests check that); the Jaccard distance 1 - IoU is a
metric, so the two reports' IoU may differ by at most the distances between
the GPU's and the oracle's sets of the method and of the dense indexer, and a
needle may be counted differently only if it is one of the swapped keys.
"""
import numpy as np
import pytest

import oracle as O
import synth
from bench import selection_quality
from parity import oracle_problem, to_gpu

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _sets(rows):
    return [set(int(s) for s in np.asarray(r) if s >= 0) for r in rows]


def _jd(a, b):
    return 1.0 - len(a & b) / max(1, len(a | b))


def _compare(gpu_sel, gpu_dense, o_sel, o_dense, needles, label):
    qg = selection_quality(gpu_sel, gpu_dense, needles)
    qo = selection_quality(o_sel, o_dense, needles)
    gs, gd, os_, od = _sets(gpu_sel), _sets(gpu_dense), _sets(o_sel), _sets(o_dense)
    T = len(gs)
    bound = sum(_jd(gs[t], os_[t]) + _jd(gd[t], od[t]) for t in range(T)) / T
    assert bound <= 0.01, f"{label}: GPU sets far from the oracle's ({bound:.4f})"
    assert abs(qg["iou_vs_dense_topk"] - qo["iou_vs_dense_topk"]) <= bound + 1e-12, (label, qg, qo)
    swapped = sum(len(set(needles[t]) & (gs[t] ^ os_[t])) for t in range(T))
    swapped_d = sum(len(set(needles[t]) & (gd[t] ^ od[t])) for t in range(T))
    nn = qg["needles"]
    assert nn == qo["needles"]
    if nn:
        assert abs(qg["needle_recall"] - qo["needle_recall"]) * nn <= swapped, (label, qg, qo)
        assert abs(qg["dense_needle_recall"] - qo["dense_needle_recall"]) * nn <= swapped_d, (label, qg, qo)
    return qg, qo


def _oracle_sets(P, path, wl, kprime=None, m=None):
    if path == "hier":
        res = O.misa_hier_topk(P, wl.A, kprime, wl.k)[0]
    elif path == "misa":
        res = O.misa_topk(P, wl.A, wl.k)[0]
    else:
        res = O.hisa_topk(P, m, wl.k)[0]
    return [r[0] for r in res], [r[0] for r in O.dense_topk(P, wl.k)]


def test_quality_tiny_decode_every_row():
    wl = synth.CONFIGS["c1_tiny_decode"]
    inp = synth.make_inputs(wl, seed=0)
    q, w, K, ks, pos = to_gpu(inp)
    dense = S.score_topk(q, w, K, pos, wl.B, wl.H, wl.k, ks)[0].cpu().numpy()
    P = oracle_problem(inp, wl.B)
    for path, call, kw in [("misa", lambda: S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks), {}),
                           ("hier", lambda: S.hier_topk(q, w, K, pos, wl.B, wl.A, 1024, wl.k, ks),
                            {"kprime": 1024}),
                           ("hisa", lambda: S.hisa_topk(q, w, K, pos, wl.B, 8, wl.k, ks), {"m": 8})]:
        sel = call()[0].cpu().numpy()
        o_sel, o_dense = _oracle_sets(P, path, wl, **kw)
        qg, qo = _compare(sel, dense, o_sel, o_dense, inp["needles"], f"c1 {path}")
        print(path, qg, qo)


def test_quality_128k_two_rows():
    wl = synth.CONFIGS["c4_hier_decode_128k"]
    inp = synth.make_inputs(wl, seed=0)
    q, w, K, ks, pos = to_gpu(inp)
    rows = [0, wl.T - 1]
    dense = S.score_topk(q, w, K, pos, wl.B, wl.H, wl.k, ks)[0].cpu().numpy()[rows]
    P = oracle_problem(inp, wl.B, rows=rows)
    needles = [inp["needles"][t] for t in rows]
    for path, call, kw in [("hier", lambda: S.hier_topk(q, w, K, pos, wl.B, wl.A, wl.kprime, wl.k, ks),
                            {"kprime": wl.kprime}),
                           ("misa", lambda: S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks), {})]:
        sel = call()[0].cpu().numpy()[rows]
        o_sel, o_dense = _oracle_sets(P, path, wl, **kw)
        qg, qo = _compare(sel, dense, o_sel, o_dense, needles, f"c4 {path}")
        print(path, qg, qo)
