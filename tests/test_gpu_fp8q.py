"""GPU parity with fp8 queries: q as E4M3FN codes with a per-(query, head)
fp32 scale, fp8 keys, scored on the fp8 matrix cores (one 16x16x128 fp8 MFMA
per row tile and key group).

Routed head sets must match the oracle bit for bit (the router forms
code * scale exactly in float64); scores and selections must match within the
fp8 tolerance; selections must equal the first k of the library's own score
rows exactly. Cases cover negative query scales (the sign folded into the
codes), the dense path (scales applied inside the scoring kernel), explicit
head lists, the staged (few rows) and unstaged (256 rows) kernel forms, and
the full 128K workloads.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import check_heads, oracle_problem, q_scale_gpu, rtol_of, to_gpu, tolerance, check_row
from test_gpu_exact_selection import _assert_selection, _first_k, _full_rows, _n
from test_gpu_parity import _check_misa, check_hier, check_hisa, check_misa_hisa

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _np(t):
    return t.cpu().numpy()


def _case(seed, T, L, H, positions="random", neg=True):
    inp = synth.random_small(seed, T=T, L=L, H=H, k_dtype=synth.KDT_FP8, positions=positions, q_fp8=True)
    if positions == "random" and T >= 3:
        inp["pos"][0] = 0
        inp["pos"][1] = L - 1
    if neg:
        inp["q_scale"][:, ::5] *= np.float32(-1.0)   # negative query scales
        inp["k_scale"][::7] *= np.float32(-1.0)
    return inp


def _gpu(inp):
    q, w, K, ks, pos = to_gpu(inp)
    return q, w, K, ks, pos, q_scale_gpu(inp)


ROUTE_CASES = [(1, 5, 3000, 64, 8, 128), (2, 16, 20000, 32, 8, 128), (3, 9, 777, 48, 5, 37), (4, 32, 5000, 64, 8, 64)]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}A{c[4]}B{c[5]}")
def test_route_fp8q(case):
    seed, T, L, H, A, B = case
    inp = _case(seed, T, L, H)
    q, w, K, ks, pos, qs = _gpu(inp)
    heads, r = S.route(q, w, K, pos, B, A, ks, with_r=True, q_scale=qs)
    _, ill = check_heads(oracle_problem(inp, B), A, _np(heads), _np(r))
    assert ill == 0


MISA_CASES = [
    # seed, T, L, H, A, B, k, positions
    (11, 7, 3000, 64, 8, 128, 300, "random"),      # staged rows (few rows per workgroup)
    (12, 32, 9000, 64, 8, 128, 500, "decode"),     # 256 rows: unstaged form
    (13, 5, 20000, 32, 8, 128, 1000, "decode"),    # long rows
    (14, 9, 1500, 16, 16, 64, 100, "random"),      # A = H: dense, scales applied by the kernel
    (15, 12, 2000, 40, 3, 100, 77, "random"),
]


@pytest.mark.parametrize("case", MISA_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}A{c[4]}k{c[6]}{c[7]}")
def test_misa_fp8q(case):
    seed, T, L, H, A, B, k, positions = case
    inp = _case(seed, T, L, H, positions)
    q, w, K, ks, pos, qs = _gpu(inp)
    idx, sc = S.score_topk(q, w, K, pos, B, A, k, ks, q_scale=qs)
    worst = _check_misa(inp, B, A, k, _np(idx), _np(sc), label="fp8q misa")
    print(f"worst error / tolerance = {worst:.3e}")


def test_misa_fp8q_explicit_heads():
    inp = _case(16, 11, 2500, 64)
    rng = np.random.default_rng(0)
    A = 6
    hs = np.stack([rng.choice(64, A, replace=False) for _ in range(11)]).astype(np.int32)
    q, w, K, ks, pos, qs = _gpu(inp)
    idx, sc = S.score_topk(q, w, K, pos, 128, A, 120, ks, heads=torch.from_numpy(hs).cuda(), q_scale=qs)
    _check_misa(inp, 128, A, 120, _np(idx), _np(sc), hs, label="fp8q explicit heads")


HIER_CASES = [(21, 6, 3000, 64, 8, 128, 600, 100), (22, 8, 20000, 64, 8, 128, 4096, 512),
              (23, 5, 17500, 40, 6, 128, 20000, 500)]  # long rows, 40 heads, k' >= n


@pytest.mark.parametrize("case", HIER_CASES, ids=lambda c: f"T{c[1]}L{c[2]}kp{c[6]}k{c[7]}")
def test_hier_fp8q(case):
    seed, T, L, H, A, B, kp, k = case
    inp = _case(seed, T, L, H, "random" if L < 10000 else "decode")
    q, w, K, ks, pos, qs = _gpu(inp)
    idx, sc = S.hier_topk(q, w, K, pos, B, A, kp, k, ks, q_scale=qs)
    check_hier(inp, B, A, kp, k, _np(idx), _np(sc), label="fp8q hier")


HISA_CASES = [(31, 7, 3000, 64, 128, 5, 200), (32, 40, 9000, 32, 64, 16, 512), (33, 4, 40000, 32, 128, 64, 2048)]


@pytest.mark.parametrize("case", HISA_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}B{c[4]}m{c[5]}k{c[6]}")
def test_hisa_fp8q(case):
    seed, T, L, H, B, m, k = case
    inp = _case(seed, T, L, H, "random" if L < 10000 else "decode")
    q, w, K, ks, pos, qs = _gpu(inp)
    idx, sc = S.hisa_topk(q, w, K, pos, B, m, k, ks, q_scale=qs)
    check_hisa(inp, B, m, k, _np(idx), _np(sc), label="fp8q hisa")
    idx, sc = S.hisa_maxpool_topk(q, w, K, pos, B, m, k, ks, q_scale=qs)
    check_hisa(inp, B, m, k, _np(idx), _np(sc), label="fp8q hisa max-pool", pool="max")


def test_misa_hisa_fp8q():
    inp = _case(41, 9, 5000, 32)
    q, w, K, ks, pos, qs = _gpu(inp)
    heads = S.route(q, w, K, pos, 128, 8, ks, q_scale=qs)
    idx, sc = S.misa_hisa_topk(q, w, K, pos, 128, 8, 6, 300, ks, q_scale=qs)
    P = oracle_problem(inp, 128)
    heads_o, ill = check_heads(P, 8, _np(heads))
    assert ill == 0
    check_misa_hisa(inp, 128, 8, 6, 300, _np(idx), _np(sc), heads_o, label="fp8q misa-hisa")


@pytest.mark.parametrize("name", ["c4_hier_decode_128k", "c5_glm5_hisa_128k"])
def test_full_workloads_fp8q(name):
    wl = synth.CONFIGS[name]
    inp = synth.make_inputs(wl, seed=0, q_fp8=True)
    q, w, K, ks, pos, qs = _gpu(inp)
    heads = S.route(q, w, K, pos, wl.B, wl.A, ks, q_scale=qs)
    _, ill = check_heads(oracle_problem(inp, wl.B), wl.A, _np(heads))
    assert ill == 0
    idx, sc = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks, q_scale=qs)
    _check_misa(inp, wl.B, wl.A, wl.k, _np(idx), _np(sc), label=f"{name} fp8q misa")
    if name.startswith("c4"):
        idx, sc = S.hier_topk(q, w, K, pos, wl.B, wl.A, wl.kprime, wl.k, ks, q_scale=qs)
        check_hier(inp, wl.B, wl.A, wl.kprime, wl.k, _np(idx), _np(sc), label="c4 fp8q hier")
    else:
        idx, sc = S.hisa_topk(q, w, K, pos, wl.B, wl.m, wl.k, ks, q_scale=qs)
        check_hisa(inp, wl.B, wl.m, wl.k, _np(idx), _np(sc), label="c5 fp8q hisa")


@pytest.mark.parametrize("name", ["c4_hier_decode_128k", "c5_glm5_hisa_128k"])
def test_selection_exact_fp8q(name):
    """The selection is the first k of the library's own fp8-scored rows."""
    wl = synth.CONFIGS[name]
    inp = synth.make_inputs(wl, seed=0, q_fp8=True)
    q, w, K, ks, pos, qs = _gpu(inp)
    L = wl.L
    fi, fs = S.score_topk(q, w, K, pos, wl.B, wl.A, L, ks, q_scale=qs)
    si, ss = S.score_topk(q, w, K, pos, wl.B, wl.A, wl.k, ks, q_scale=qs)
    full = _full_rows(_np(fi), _np(fs), _n(inp, L))
    _assert_selection(_np(si), _np(ss), full, wl.k, f"{name} fp8q")


def test_fp8q_unsupported_requests():
    inp = _case(51, 4, 1000, 32)
    q, w, K, ks, pos, qs = _gpu(inp)
    Kb = torch.zeros((1000, 128), dtype=torch.int16, device="cuda")           # bf16 keys
    with pytest.raises(S.MisaError) as e:
        S.score_topk(q, w, Kb, pos, 128, 8, 50, None, q_scale=qs)
    assert e.value.status == -2
    big = _case(52, 40, 2000, 64, positions="prefill", neg=False)             # 40 x 8 rows > 256
    q2, w2, K2, ks2, pos2, qs2 = _gpu(big)
    with pytest.raises(S.MisaError) as e:
        S.score_topk(q2, w2, K2, pos2, 128, 8, 50, ks2, q_scale=qs2)
    assert e.value.status == -2
    # HISA takes any batch
    idx, sc = S.hisa_topk(q2, w2, K2, pos2, 128, 4, 50, ks2, q_scale=qs2)
    check_hisa(big, 128, 4, 50, _np(idx), _np(sc), label="fp8q hisa, many queries")


@pytest.mark.parametrize("source", ["pooled", "arbitrary"])
@pytest.mark.parametrize("L", [3000, 20000])
def test_fp8q_cached_block_means(source, L):
    """fp8 queries with cached block means: the head ranking launches no block-sum
    pass and pools each query's last block itself (float64, code * scale exact)."""
    inp = _case(71, 9, L, 64, positions="random" if L < 10000 else "decode")
    q, w, K, ks, pos, qs = _gpu(inp)
    B, A = 128, 8
    M = -(-L // B)
    if source == "pooled":
        kbar = S.block_means(K, B, ks)
    else:
        rows = np.random.default_rng(L).standard_normal((M, 128)).astype(np.float32) * 0.2
        kbar = torch.from_numpy(rows).cuda()
    inp = dict(inp, kbar=_np(kbar))
    P = oracle_problem(inp, B)
    heads, r = S.route(q, w, K, pos, B, A, ks, with_r=True, kbar=kbar, q_scale=qs)
    heads_o, ill = check_heads(P, A, _np(heads), _np(r))
    assert ill == 0
    idx, sc = S.score_topk(q, w, K, pos, B, A, 100, ks, kbar=kbar, q_scale=qs)
    _check_misa(inp, B, A, 100, _np(idx), _np(sc), heads_o, label="fp8q cached misa")
    idx, sc = S.hier_topk(q, w, K, pos, B, A, 600, 100, ks, kbar=kbar, q_scale=qs)
    check_hier(inp, B, A, 600, 100, _np(idx), _np(sc), label="fp8q cached hier")
    idx, sc = S.misa_hisa_topk(q, w, K, pos, B, A, 6, 100, ks, kbar=kbar, q_scale=qs)
    check_misa_hisa(inp, B, A, 6, 100, _np(idx), _np(sc), heads_o, label="fp8q cached misa-hisa")


def test_fp8q_cached_block_means_full_c4():
    """The cached-means MISA-dagger step at the full 128K decode shape with fp8
    queries: heads bit-exact, selections within the fp8 tolerance, and the same
    call without a workspace (static scratch) bit for bit."""
    wl = synth.CONFIGS["c4_hier_decode_128k"]
    inp = synth.make_inputs(wl, seed=1, q_fp8=True)
    q, w, K, ks, pos, qs = _gpu(inp)
    kbar = S.block_means(K, wl.B, ks)
    inp = dict(inp, kbar=_np(kbar))
    heads = S.route(q, w, K, pos, wl.B, wl.A, ks, kbar=kbar, q_scale=qs)
    heads_o, ill = check_heads(oracle_problem(inp, wl.B), wl.A, _np(heads))
    assert ill == 0
    idx, sc = S.hier_topk(q, w, K, pos, wl.B, wl.A, wl.kprime, wl.k, ks, kbar=kbar, q_scale=qs)
    check_hier(inp, wl.B, wl.A, wl.kprime, wl.k, _np(idx), _np(sc), label="c4 fp8q cached hier")
    i2, s2 = S.hier_topk_noalloc(q, w, K, pos, wl.B, wl.A, wl.kprime, wl.k, ks, kbar=kbar, q_scale=qs)
    assert torch.equal(idx, i2) and torch.equal(sc, s2)
