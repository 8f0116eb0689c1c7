"""Entry points captured in HIP graphs: every replay must reproduce the eager
call bit for bit, also after other calls on other inputs ran in between (the
library clears its counters and histograms with kernels, never with memsets,
so a replayed graph starts from the same state as an eager call)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import to_gpu

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _inputs(seed, T, L, H, kdt, positions="random"):
    return to_gpu(synth.random_small(seed, T=T, L=L, H=H, k_dtype=kdt, positions=positions))


def _replays_match(call, other, n=3):
    ref = [t.clone() for t in call()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = call()
    for i in range(n):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {i} differs from the eager call"
        other()
        torch.cuda.synchronize()


def _ws(nbytes):
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda")


def test_graph_hier_long_rows():
    # rows longer than the one-workgroup selection: the split selection clears its
    # histogram inside the scoring launch
    T, L, H, B, A, kp, k = 8, 20000, 64, 128, 8, 3000, 500
    q, w, K, ks, pos = _inputs(51, T, L, H, O.KDT_FP8, positions="decode")
    q2, w2, K2, ks2, pos2 = _inputs(52, T, L, H, O.KDT_FP8, positions="random")
    p = S.make_problem(q, w, K, pos, B, ks)
    ws = _ws(S.workspace_bytes(p, S.OP_HIER_TOPK, A=A, kprime=kp, k=k))
    out = (torch.empty((T, k), dtype=torch.int32, device="cuda"),
           torch.empty((T, k), dtype=torch.float32, device="cuda"))
    _replays_match(lambda: S.hier_topk(q, w, K, pos, B, A, kp, k, ks, ws=ws, out=out),
                   lambda: S.hier_topk(q2, w2, K2, pos2, B, A, kp, k, ks2))


def test_graph_misa_many_queries():
    # the router's single-pass bf16 form with settling and selection
    T, L, H, B, A, k = 1100, 1100, 64, 16, 8, 64
    q, w, K, ks, pos = _inputs(53, T, L, H, O.KDT_BF16, positions="prefill")
    q2, w2, K2, ks2, pos2 = _inputs(54, T, L, H, O.KDT_BF16, positions="random")
    p = S.make_problem(q, w, K, pos, B, ks)
    ws = _ws(S.workspace_bytes(p, S.OP_SCORE_TOPK, A=A, k=k))
    out = (torch.empty((T, k), dtype=torch.int32, device="cuda"),
           torch.empty((T, k), dtype=torch.float32, device="cuda"))
    _replays_match(lambda: S.score_topk(q, w, K, pos, B, A, k, ks, ws=ws, out=out),
                   lambda: S.score_topk(q2, w2, K2, pos2, B, A, k, ks2))


def test_graph_hisa():
    T, L, H, B, m, k = 16, 6000, 32, 128, 8, 300
    q, w, K, ks, pos = _inputs(55, T, L, H, O.KDT_FP8, positions="decode")
    q2, w2, K2, ks2, pos2 = _inputs(56, T, L, H, O.KDT_FP8, positions="random")
    p = S.make_problem(q, w, K, pos, B, ks)
    ws = _ws(S.workspace_bytes(p, S.OP_HISA_TOPK, m=m, k=k))
    out = (torch.empty((T, k), dtype=torch.int32, device="cuda"),
           torch.empty((T, k), dtype=torch.float32, device="cuda"))
    _replays_match(lambda: S.hisa_topk(q, w, K, pos, B, m, k, ks, ws=ws, out=out),
                   lambda: S.hisa_topk(q2, w2, K2, pos2, B, m, k, ks2))


def test_graph_cached_means_with_update():
    # a decode step with cached block means: refresh the last block, then MISA-dagger
    T, L, H, B, A, kp, k = 8, 9000, 64, 128, 8, 2000, 300
    q, w, K, ks, pos = _inputs(57, T, L, H, O.KDT_FP8, positions="decode")
    kbar = S.block_means(K, B, ks)
    p = S.make_problem(q, w, K, pos, B, ks, kbar)
    ws = _ws(S.workspace_bytes(p, S.OP_HIER_TOPK, A=A, kprime=kp, k=k))
    out = (torch.empty((T, k), dtype=torch.int32, device="cuda"),
           torch.empty((T, k), dtype=torch.float32, device="cuda"))

    def step():
        S.block_means_update(K, B, kbar, kbar.shape[0] - 1, ks, ws=ws)
        return S.hier_topk(q, w, K, pos, B, A, kp, k, ks, ws=ws, out=out, kbar=kbar)

    q2, w2, K2, ks2, pos2 = _inputs(58, T, L, H, O.KDT_FP8, positions="random")
    _replays_match(step, lambda: S.hier_topk(q2, w2, K2, pos2, B, A, kp, k, ks2))


def test_graph_misa_hisa():
    T, L, H, B, A, m, k = 16, 6000, 32, 128, 8, 8, 300
    q, w, K, ks, pos = _inputs(59, T, L, H, O.KDT_FP8, positions="decode")
    q2, w2, K2, ks2, pos2 = _inputs(60, T, L, H, O.KDT_FP8, positions="random")
    p = S.make_problem(q, w, K, pos, B, ks)
    ws = _ws(S.workspace_bytes(p, S.OP_MISA_HISA_TOPK, A=A, m=m, k=k))
    out = (torch.empty((T, k), dtype=torch.int32, device="cuda"),
           torch.empty((T, k), dtype=torch.float32, device="cuda"))
    _replays_match(lambda: S.misa_hisa_topk(q, w, K, pos, B, A, m, k, ks, ws=ws, out=out),
                   lambda: S.misa_hisa_topk(q2, w2, K2, pos2, B, A, m, k, ks2))


def test_graph_hisa_maxpool():
    T, L, H, B, m, k = 16, 6000, 32, 128, 8, 300
    q, w, K, ks, pos = _inputs(61, T, L, H, O.KDT_FP8, positions="decode")
    q2, w2, K2, ks2, pos2 = _inputs(62, T, L, H, O.KDT_FP8, positions="random")
    p = S.make_problem(q, w, K, pos, B, ks)
    ws = _ws(S.workspace_bytes(p, S.OP_HISA_TOPK, m=m, k=k))
    out = (torch.empty((T, k), dtype=torch.int32, device="cuda"),
           torch.empty((T, k), dtype=torch.float32, device="cuda"))
    _replays_match(lambda: S.hisa_maxpool_topk(q, w, K, pos, B, m, k, ks, ws=ws, out=out),
                   lambda: S.hisa_maxpool_topk(q2, w2, K2, pos2, B, m, k, ks2))
