"""misa_hier_topk_noalloc (the entry point for callers that cannot allocate)
against misa_hier_topk with a caller workspace: identical outputs, bit for
bit, on two calls in a row that share the static scratch, the second with a
smaller problem; an oversized problem is rejected before anything runs."""
import numpy as np
import pytest
import torch

import synth
from parity import to_gpu

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _same(a, b):
    return torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_noalloc_matches_workspace_entry_point_twice():
    wl = synth.CONFIGS["c4_hier_decode_128k"]
    big = synth.make_inputs(wl, seed=0)
    small = synth.random_small(5, T=5, L=3000, H=64, k_dtype=synth.KDT_BF16, positions="random")
    small["pos"][0] = 0
    for inp, (A, kp, k) in [(big, (wl.A, wl.kprime, wl.k)), (small, (8, 500, 100))]:
        q, w, K, ks, pos = to_gpu(inp)
        ref = S.hier_topk(q, w, K, pos, 128, A, kp, k, ks)
        got = S.hier_topk_noalloc(q, w, K, pos, 128, A, kp, k, ks)
        torch.cuda.synchronize()
        assert _same(ref, got), f"T={q.shape[0]} L={K.shape[0]}"


def test_noalloc_rejects_a_problem_larger_than_the_scratch():
    inp = synth.random_small(6, T=40, L=200000, H=64, k_dtype=synth.KDT_FP8, positions="decode")
    q, w, K, ks, pos = to_gpu(inp)
    p = S.make_problem(q, w, K, pos, 128, ks)
    assert S.workspace_bytes(p, S.OP_HIER_TOPK, A=8, kprime=8192, k=2048) > S.STATIC_SCRATCH_BYTES
    idx = torch.full((40, 2048), 7, dtype=torch.int32, device="cuda")
    sc = torch.full((40, 2048), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(S.MisaError) as e:
        S.hier_topk_noalloc(q, w, K, pos, 128, 8, 8192, 2048, ks, out=(idx, sc))
    assert e.value.status == -3 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((idx == 7).all()) and bool((sc == 3.0).all())   # outputs untouched
