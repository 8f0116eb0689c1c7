"""GPU parity: the HIP library against the CPU oracle on seeded inputs.

Small sweeps cover several key tiles, query groups and ragged tails (T, L and B
not multiples of the tile sizes), rows shorter than k, A = H (dense), A = 1,
fp8 keys with negative scales, and explicit head lists.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from parity import (RTOL, check_heads, check_row, kdtype, oracle_problem, pool_bands, to_gpu,
                    tolerance)

pytestmark = pytest.mark.gpu

S = pytest.importorskip("sparse_attention_indexer_block_amd")


def _np(t):
    return t.cpu().numpy()


def _case(seed, T, L, H, kdt, positions="random", w_scale=0.125, neg_scales=False):
    inp = synth.random_small(seed, T=T, L=L, H=H, k_dtype=kdt, positions=positions, w_scale=w_scale)
    if positions == "random" and T >= 3:
        inp["pos"][0] = 0            # one visible key
        inp["pos"][1] = L - 1        # the whole key array
        inp["pos"][2] = min(L - 1, 127)
    if neg_scales and inp["k_scale"] is not None:
        inp["k_scale"][::3] *= np.float32(-1.0)
    return inp


# ----------------------------------------------------------------- block means

@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
def test_block_means(kdt):
    rng = np.random.default_rng(5)
    L, B = 1000, 128
    if kdt == O.KDT_FP8:
        # every finite E4M3FN code appears, with positive and negative scales
        codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
        K = rng.choice(codes, size=(L, 128)).astype(np.uint8)
        K[:2, :] = np.resize(codes, (2, 128))
        ks = (rng.random(L).astype(np.float32) + np.float32(0.01)) * np.where(rng.random(L) < 0.3, -1, 1).astype(np.float32)
        inp = {"K": K, "k_scale": ks.astype(np.float32)}
        Kt = torch.from_numpy(K).cuda()
        kst = torch.from_numpy(inp["k_scale"]).cuda()
        vals = O.dequant_keys(K, O.KDT_FP8, inp["k_scale"])
    else:
        K = synth.encode_bf16(rng.standard_normal((L, 128), dtype=np.float32))
        Kt = torch.from_numpy(K.view(np.int16)).cuda()
        kst = None
        vals = O.dequant_keys(K, O.KDT_BF16)
    for Bv in [B, 7, 1000, 2048]:
        got = _np(S.block_means(Kt, Bv, kst))
        ref = O.full_block_means(vals, Bv).astype(np.float32)
        np.testing.assert_allclose(got, ref, rtol=2.5e-7, atol=1e-38)


@pytest.mark.parametrize("kdt,B", [(O.KDT_BF16, 128), (O.KDT_FP8, 128), (O.KDT_FP8, 37)])
def test_block_means_update(kdt, B):
    """Cached means kept current while keys are appended: recomputing the rows
    from the first touched block reproduces the full computation bit for bit,
    and rows before it are left untouched."""
    inp = synth.random_small(41, T=1, L=5000, H=8, k_dtype=kdt)
    _, _, K, ks, _ = to_gpu(inp)
    for L0, L1 in [(1000, 1001), (1023, 1024), (1024, 1300), (1, 5000), (4999, 5000)]:
        K0, K1 = K[:L0], K[:L1]
        s0 = ks[:L0] if ks is not None else None
        s1 = ks[:L1] if ks is not None else None
        M1 = -(-L1 // B)
        kbar = torch.full((M1, 128), float("nan"), dtype=torch.float32, device=K.device)
        M0 = -(-L0 // B)
        kbar[:M0] = S.block_means(K0, B, s0)
        keep = kbar[: L0 // B].clone()
        S.block_means_update(K1, B, kbar, L0 // B, s1)
        full = S.block_means(K1, B, s1)
        torch.cuda.synchronize()
        assert torch.equal(kbar, full), (L0, L1)
        assert torch.equal(kbar[: L0 // B], keep)


# ----------------------------------------------------------------- router

ROUTE_CASES = [
    # seed, T, L, H, A, B, kdt
    (1, 5, 300, 64, 8, 128, O.KDT_BF16),
    (2, 17, 1000, 32, 8, 128, O.KDT_FP8),
    (3, 9, 777, 48, 5, 37, O.KDT_BF16),
    (4, 40, 2100, 64, 64, 128, O.KDT_BF16),
    (5, 6, 257, 7, 1, 1, O.KDT_FP8),
    (6, 8, 4096, 64, 8, 4096, O.KDT_BF16),
    # many queries times many blocks: the two-pass router (bf16 pass, float64 settling)
    (7, 1100, 1100, 64, 8, 16, O.KDT_BF16),
    (8, 2200, 2200, 32, 8, 128, O.KDT_FP8),
    (9, 4500, 600, 64, 8, 5, O.KDT_BF16),
    # many queries and more than 128 blocks: bf16 pass over two ranges, separate settling
    (12, 600, 20000, 64, 8, 128, O.KDT_FP8),
    # few query-head rows and several blocks per pooling group
    (10, 6, 50000, 64, 8, 100, O.KDT_FP8),
    (11, 3, 30000, 48, 5, 64, O.KDT_BF16),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}A{c[4]}B{c[5]}k{c[6]}")
def test_route(case):
    seed, T, L, H, A, B, kdt = case
    inp = _case(seed, T, L, H, kdt, neg_scales=True)
    q, w, K, ks, pos = to_gpu(inp)
    heads, r = S.route(q, w, K, pos, B, A, ks, with_r=True)
    P = oracle_problem(inp, B)
    _, ill = check_heads(P, A, _np(heads), _np(r))
    assert ill == 0


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
def test_route_equal_blocks(kdt):
    # every key is the same vector, so all complete blocks of a query have the same mean
    # and no block can be ruled out before the exact products
    T, L, H, A, B = 1500, 1500, 64, 8, 16
    inp = _case(31, T, L, H, kdt, positions="prefill")
    inp["K"][:] = inp["K"][0]
    if inp["k_scale"] is not None:
        inp["k_scale"][:] = inp["k_scale"][0]
    q, w, K, ks, pos = to_gpu(inp)
    heads, r = S.route(q, w, K, pos, B, A, ks, with_r=True)
    P = oracle_problem(inp, B)
    _, ill = check_heads(P, A, _np(heads), _np(r))
    assert ill == 0


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
def test_route_tied_heads_at_the_cut(kdt):
    # heads come in identical pairs (same q row, same weight), so r ties exactly within
    # each pair and, with A odd, the cut splits a pair in every query: no interval can
    # place those heads, the exact values decide and the lower head must win the tie
    T, L, H, A, B = 1500, 1500, 64, 7, 16
    inp = _case(32, T, L, H, kdt, positions="prefill")
    inp["q"][:, 1::2] = inp["q"][:, 0::2]
    inp["w"][:, 1::2] = inp["w"][:, 0::2]
    q, w, K, ks, pos = to_gpu(inp)
    P = oracle_problem(inp, B)
    heads_o, r_o = O.route(P, A)
    for with_r in (False, True):
        out = S.route(q, w, K, pos, B, A, ks, with_r=with_r)
        heads = _np(out[0] if with_r else out)
        for t in range(T):
            assert sorted(heads[t]) == sorted(int(h) for h in heads_o[t]), f"row {t} (with r: {with_r})"


@pytest.mark.parametrize("with_r", [False, True])
@pytest.mark.parametrize("T,L", [(1500, 1500), (400, 3000)], ids=["one_range", "split"])
def test_route_many_queries_float_overflow(T, L, with_r):
    # keys near 2^120 with q near 2^12: the bf16 screen's float products overflow, so
    # no interval or leader certifies anything and every head's complete blocks are
    # settled in float64 (one range per workgroup, and the split form)
    H, A, B = 64, 8, 16
    inp = _case(33, T, L, H, O.KDT_BF16, positions="prefill")
    to_bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    from_bits = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    inp["K"] = to_bits(from_bits(inp["K"]) * np.float32(2.0 ** 118))
    inp["q"] = to_bits(from_bits(inp["q"]) * np.float32(2.0 ** 12))
    q, w, K, ks, pos = to_gpu(inp)
    P = oracle_problem(inp, B)
    out = S.route(q, w, K, pos, B, A, ks, with_r=with_r)
    heads = _np(out[0] if with_r else out)
    _, ill = check_heads(P, A, heads)
    assert ill == 0


@pytest.mark.parametrize("A", [1, 31, 32])
def test_route_many_queries_extreme_A(A):
    # the bf16 router's interval placement at the ends: one head kept, one left out, all kept
    T, L, H, B = 1500, 1500, 32, 16
    inp = _case(34, T, L, H, O.KDT_FP8, positions="prefill", neg_scales=True)
    q, w, K, ks, pos = to_gpu(inp)
    P = oracle_problem(inp, B)
    for with_r in (False, True):
        out = S.route(q, w, K, pos, B, A, ks, with_r=with_r)
        _, ill = check_heads(P, A, _np(out[0] if with_r else out))
        assert ill == 0


# ----------------------------------------------------------------- MISA

MISA_CASES = [
    # seed, T, L, H, A, B, k, kdt, positions
    (11, 7, 500, 64, 8, 128, 64, O.KDT_BF16, "random"),
    (12, 33, 1500, 64, 8, 128, 100, O.KDT_FP8, "random"),
    (13, 16, 4096, 64, 8, 128, 512, O.KDT_BF16, "decode"),
    (14, 70, 70, 32, 4, 16, 9, O.KDT_BF16, "prefill"),
    (15, 12, 900, 64, 64, 128, 50, O.KDT_BF16, "random"),
    (16, 10, 600, 16, 1, 64, 33, O.KDT_FP8, "random"),
    (17, 9, 1200, 40, 13, 100, 1200, O.KDT_BF16, "random"),
    (18, 300, 300, 64, 8, 128, 20, O.KDT_FP8, "prefill"),
    (19, 5, 20000, 32, 8, 128, 700, O.KDT_BF16, "decode"),
    (20, 1100, 1100, 64, 8, 16, 64, O.KDT_FP8, "prefill"),
    # LDS-tiled scoring (more than 256 rows) with 16 and 32 padded head slots, and
    # with rows long enough for the split selection (per-split score ranges)
    (21, 40, 900, 64, 12, 128, 77, O.KDT_FP8, "random"),
    (22, 20, 700, 48, 20, 64, 50, O.KDT_BF16, "random"),
    (23, 40, 17000, 32, 8, 128, 300, O.KDT_FP8, "random"),
    # many rows longer than 8192 keys: the row selection streams through the rows
    (24, 1100, 9000, 16, 4, 128, 300, O.KDT_BF16, "random"),
    # decode batches of several 64-row query groups: key splits a multiple of 8
    # (the groups of a split placed on one XCD) and not (plain order)
    (25, 24, 20000, 64, 8, 128, 500, O.KDT_FP8, "decode"),
    (26, 32, 16384, 64, 8, 128, 700, O.KDT_BF16, "decode"),
    (27, 16, 12000, 32, 8, 128, 400, O.KDT_FP8, "random"),
]


def _check_misa(inp, B, A, k, idx, sc, heads_used=None, label=""):
    P = oracle_problem(inp, B)
    rtol = RTOL[kdtype(inp)]
    if heads_used is None:
        heads_used, _ = O.route(P, A)
    worst = 0.0
    for t in range(P.T):
        n = P.n(t)
        keys = np.arange(n)
        sel, _ = O.first_k(O.routed_scores(P, t, heads_used[t], keys), keys, k)
        hs = heads_used[t]
        worst = max(worst, check_row(
            idx[t], sc[t], k, n, "ascending", sel,
            lambda s, t=t, hs=hs: O.routed_scores(P, t, hs, s),
            lambda s, t=t, hs=hs: tolerance(P, t, hs, s, rtol), label=f"{label} row {t}"))
    return worst


@pytest.mark.parametrize("case", MISA_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}A{c[4]}B{c[5]}k{c[6]}kd{c[7]}{c[8]}")
def test_misa_score_topk(case):
    seed, T, L, H, A, B, k, kdt, positions = case
    inp = _case(seed, T, L, H, kdt, positions=positions, neg_scales=True)
    q, w, K, ks, pos = to_gpu(inp)
    heads = S.route(q, w, K, pos, B, A, ks)
    idx, sc = S.score_topk(q, w, K, pos, B, A, k, ks)
    torch.cuda.synchronize()
    P = oracle_problem(inp, B)
    heads_o, ill = check_heads(P, A, _np(heads))
    assert ill == 0
    worst = _check_misa(inp, B, A, k, _np(idx), _np(sc), heads_o, label="misa")
    print(f"worst error / tolerance = {worst:.3e}")


def test_misa_explicit_heads():
    inp = _case(21, 11, 800, 64, O.KDT_BF16)
    rng = np.random.default_rng(0)
    A = 6
    hs = np.stack([np.sort(rng.choice(64, A, replace=False)) for _ in range(11)]).astype(np.int32)
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.score_topk(q, w, K, pos, 128, A, 40, ks, heads=torch.from_numpy(hs).cuda())
    _check_misa(inp, 128, A, 40, _np(idx), _np(sc), hs, label="explicit heads")


# ----------------------------------------------------------------- MISA-dagger

HIER_CASES = [
    # seed, T, L, H, A, B, kprime, k, kdt
    (31, 6, 900, 64, 8, 128, 200, 50, O.KDT_BF16),
    (32, 9, 3000, 32, 8, 128, 1024, 256, O.KDT_FP8),
    (33, 5, 400, 64, 4, 64, 400, 30, O.KDT_BF16),      # k' >= n: dense
    (34, 8, 20000, 64, 8, 128, 4096, 512, O.KDT_FP8),  # long rows
    (35, 6, 18000, 32, 8, 128, 3000, 400, O.KDT_BF16),  # long rows, bf16 keys, fewer heads than 64
    (36, 5, 17000, 48, 6, 128, 20000, 600, O.KDT_FP8),  # long rows, k' >= n: every key a candidate
    # long rows for batches of three query groups (key splits not / a multiple of 8)
    (37, 20, 24000, 64, 8, 128, 3000, 700, O.KDT_FP8),
    (39, 24, 20480, 64, 8, 128, 2048, 256, O.KDT_BF16),
]


def check_hier(inp, B, A, kprime, k, idx, sc, label="hier"):
    P = oracle_problem(inp, B)
    rtol = RTOL[kdtype(inp)]
    heads, _ = O.route(P, A)
    res, _, cands = O.misa_hier_topk(P, A, kprime, k, heads=heads)
    for t in range(P.T):
        n = P.n(t)
        keys = np.arange(n)
        rs = O.routed_scores(P, t, heads[t], keys)
        sure, maybe = pool_bands(rs, cands[t], tolerance(P, t, heads[t], keys, rtol))
        allh = list(range(P.H))
        check_row(idx[t], sc[t], k, n, "ascending", res[t][0],
                  lambda s, t=t: O.dense_scores(P, t, s),
                  lambda s, t=t: tolerance(P, t, allh, s, rtol),
                  sure_pool=sure, maybe_pool=maybe, label=f"{label} row {t}")


@pytest.mark.parametrize("case", HIER_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}kp{c[6]}k{c[7]}kd{c[8]}")
def test_misa_hier_topk(case):
    seed, T, L, H, A, B, kprime, k, kdt = case
    inp = _case(seed, T, L, H, kdt, positions="random" if L < 10000 else "decode")
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.hier_topk(q, w, K, pos, B, A, kprime, k, ks)
    check_hier(inp, B, A, kprime, k, _np(idx), _np(sc))


def test_misa_hier_topk_long_rows_negative_scales():
    # the candidates' rescoring inside the long-row emission with keys whose
    # scale is negative (the sign flips inside the ReLU)
    inp = _case(38, 5, 19000, 64, O.KDT_FP8, positions="decode", neg_scales=True)
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.hier_topk(q, w, K, pos, 128, 8, 2500, 300, ks)
    check_hier(inp, 128, 8, 2500, 300, _np(idx), _np(sc))


# ----------------------------------------------------------------- HISA

HISA_CASES = [
    # seed, T, L, H, B, m, k, kdt
    (41, 7, 1000, 64, 128, 3, 100, O.KDT_BF16),
    (42, 12, 5000, 32, 128, 16, 512, O.KDT_FP8),
    (43, 5, 600, 64, 64, 20, 40, O.KDT_BF16),     # m*B >= n: dense
    (44, 6, 300, 16, 1, 50, 30, O.KDT_BF16),      # token blocks
    (45, 4, 40000, 32, 128, 64, 2048, O.KDT_FP8),  # long rows
    (46, 20, 30000, 64, 128, 32, 1024, O.KDT_FP8),  # long rows, many queries
]


def check_hisa(inp, B, m, k, idx, sc, label="hisa", pool="mean"):
    P = oracle_problem(inp, B)
    rtol = RTOL[kdtype(inp)]
    res, blocks = O.hisa_topk(P, m, k, pool)
    allh = list(range(P.H))
    for t in range(P.T):
        n = P.n(t)
        beta = O.hisa_block_scores(P, t, pool)
        rho = O.block_logits(P, t) if pool == "mean" else P.q[t] @ O.block_maxima(P, t).T
        # the GPU forms beta in float64 and compares it in float32
        btol = 1e-6 * (np.abs(P.w[t])[:, None] * np.maximum(rho, 0)).sum(axis=0) + 1e-30
        sure_b, maybe_b = pool_bands(beta, blocks[t], btol)
        rng = O.block_ranges(n, B)
        tok = lambda bs: set(s for b in bs for s in range(*rng[b]))
        check_row(idx[t], sc[t], k, n, "ascending", res[t][0],
                  lambda s, t=t: O.dense_scores(P, t, s),
                  lambda s, t=t: tolerance(P, t, allh, s, rtol),
                  sure_pool=tok(sure_b), maybe_pool=tok(maybe_b), label=f"{label} row {t}")


@pytest.mark.parametrize("case", HISA_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}B{c[4]}m{c[5]}k{c[6]}kd{c[7]}")
def test_hisa_topk(case):
    seed, T, L, H, B, m, k, kdt = case
    inp = _case(seed, T, L, H, kdt, positions="random" if L < 10000 else "decode")
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.hisa_topk(q, w, K, pos, B, m, k, ks)
    check_hisa(inp, B, m, k, _np(idx), _np(sc))


@pytest.mark.parametrize("case", HISA_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}B{c[4]}m{c[5]}k{c[6]}kd{c[7]}")
def test_hisa_maxpool_topk(case):
    seed, T, L, H, B, m, k, kdt = case
    inp = _case(seed + 100, T, L, H, kdt, positions="random" if L < 10000 else "decode", neg_scales=True)
    q, w, K, ks, pos = to_gpu(inp)
    idx, sc = S.hisa_maxpool_topk(q, w, K, pos, B, m, k, ks)
    check_hisa(inp, B, m, k, _np(idx), _np(sc), label="hisa max-pool", pool="max")


@pytest.mark.parametrize("kdt", [O.KDT_BF16, O.KDT_FP8])
def test_hisa_maxpool_token_blocks_is_hisa_bitwise(kdt):
    # B = 1: each block's maximum and mean are its one key, so both entry points
    # must return the same bits
    inp = _case(47, 9, 700, 32, kdt, positions="random")
    q, w, K, ks, pos = to_gpu(inp)
    a = S.hisa_topk(q, w, K, pos, 1, 40, 25, ks)
    b = S.hisa_maxpool_topk(q, w, K, pos, 1, 40, 25, ks)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------- MISA inside HISA

MISA_HISA_CASES = [
    # seed, T, L, H, A, B, m, k, kdt
    (61, 7, 1000, 64, 8, 128, 3, 100, O.KDT_BF16),
    (62, 12, 5000, 32, 8, 128, 16, 512, O.KDT_FP8),
    (63, 5, 600, 64, 4, 64, 20, 40, O.KDT_BF16),       # m*B >= n: MISA
    (64, 6, 300, 16, 3, 1, 50, 30, O.KDT_BF16),        # token blocks
    (65, 4, 40000, 32, 8, 128, 64, 2048, O.KDT_FP8),   # long rows
    (66, 9, 2000, 48, 48, 100, 5, 64, O.KDT_BF16),     # A = H: HISA
    (67, 1100, 1100, 64, 8, 16, 8, 64, O.KDT_FP8),     # many queries: the two-pass router
]


def check_misa_hisa(inp, B, A, m, k, idx, sc, heads_used, label="misa-hisa"):
    P = oracle_problem(inp, B)
    rtol = RTOL[kdtype(inp)]
    res, blocks, _ = O.misa_hisa_topk(P, A, m, k, heads=heads_used)
    for t in range(P.T):
        n = P.n(t)
        hs = list(heads_used[t])
        beta = O.routed_block_scores(P, t, hs)
        rho = O.block_logits(P, t)[hs]
        # the GPU forms beta_R in float64 and compares it in float32
        btol = 1e-6 * (np.abs(P.w[t, hs])[:, None] * np.maximum(rho, 0)).sum(axis=0) + 1e-30
        sure_b, maybe_b = pool_bands(beta, blocks[t], btol)
        rng = O.block_ranges(n, B)
        tok = lambda bs: set(s for b in bs for s in range(*rng[b]))
        check_row(idx[t], sc[t], k, n, "ascending", res[t][0],
                  lambda s, t=t, hs=hs: O.routed_scores(P, t, hs, s),
                  lambda s, t=t, hs=hs: tolerance(P, t, hs, s, rtol),
                  sure_pool=tok(sure_b), maybe_pool=tok(maybe_b), label=f"{label} row {t}")


@pytest.mark.parametrize("case", MISA_HISA_CASES,
                         ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}A{c[4]}B{c[5]}m{c[6]}k{c[7]}kd{c[8]}")
def test_misa_hisa_topk(case):
    seed, T, L, H, A, B, m, k, kdt = case
    inp = _case(seed, T, L, H, kdt, positions="random" if L < 10000 else "decode")
    q, w, K, ks, pos = to_gpu(inp)
    heads = S.route(q, w, K, pos, B, A, ks)
    idx, sc = S.misa_hisa_topk(q, w, K, pos, B, A, m, k, ks)
    torch.cuda.synchronize()
    P = oracle_problem(inp, B)
    heads_o, ill = check_heads(P, A, _np(heads))
    assert ill == 0
    check_misa_hisa(inp, B, A, m, k, _np(idx), _np(sc), heads_o)


def test_misa_hisa_explicit_heads_and_cached_means():
    T, L, H, A, B, m, k = 10, 3000, 64, 6, 64, 7, 200
    inp = _case(68, T, L, H, O.KDT_FP8)
    rng = np.random.default_rng(1)
    hs = np.stack([rng.choice(H, A, replace=False) for _ in range(T)]).astype(np.int32)  # any order
    q, w, K, ks, pos = to_gpu(inp)
    kbar = S.block_means(K, B, ks)
    for kb in (None, kbar):
        idx, sc = S.misa_hisa_topk(q, w, K, pos, B, A, m, k, ks, heads=torch.from_numpy(hs).cuda(), kbar=kb)
        inp_k = inp if kb is None else dict(inp, kbar=_np(kb))
        check_misa_hisa(inp_k, B, A, m, k, _np(idx), _np(sc), hs, label="explicit heads")


def test_misa_hisa_all_heads_is_hisa_bitwise():
    T, L, H, B, m, k = 8, 2500, 32, 128, 6, 300
    inp = _case(69, T, L, H, O.KDT_BF16)
    q, w, K, ks, pos = to_gpu(inp)
    a = S.misa_hisa_topk(q, w, K, pos, B, H, m, k, ks)
    b = S.hisa_topk(q, w, K, pos, B, m, k, ks)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------- properties

def test_dense_equals_misa_with_all_heads():
    inp = _case(51, 9, 1100, 32, O.KDT_FP8)
    q, w, K, ks, pos = to_gpu(inp)
    a = S.score_topk(q, w, K, pos, 128, 32, 77, ks)
    hs = torch.arange(32, dtype=torch.int32, device="cuda").repeat(9, 1).contiguous()
    b = S.score_topk(q, w, K, pos, 128, 32, 77, ks, heads=hs)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_determinism_and_poisoned_outputs():
    inp = _case(52, 20, 3000, 64, O.KDT_BF16)
    q, w, K, ks, pos = to_gpu(inp)
    outs = []
    for fill in (0x7F, 0x00):
        idx = torch.full((20, 300), 0, dtype=torch.int32, device="cuda")
        sc = torch.zeros((20, 300), dtype=torch.float32, device="cuda")
        idx.view(torch.uint8).fill_(fill)
        sc.view(torch.uint8).fill_(fill)
        S.score_topk(q, w, K, pos, 128, 8, 300, ks, out=(idx, sc))
        outs.append((idx.clone(), sc.clone()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))
    _check_misa(inp, 128, 8, 300, _np(outs[0][0]), _np(outs[0][1]), label="poisoned")


def test_causality_on_gpu():
    inp = _case(53, 6, 2000, 64, O.KDT_BF16)
    q, w, K, ks, pos = to_gpu(inp)
    a = [x.clone() for x in S.score_topk(q, w, K, pos, 128, 8, 100, ks)]
    h = [x.clone() for x in S.hisa_topk(q, w, K, pos, 128, 4, 100, ks)]
    K2 = K.clone()
    t = 3
    K2[int(inp["pos"][t]) + 1:] = 0x40E0  # 7.0 in bf16
    b = S.score_topk(q, w, K2, pos, 128, 8, 100, ks)
    h2 = S.hisa_topk(q, w, K2, pos, 128, 4, 100, ks)
    assert torch.equal(a[0][t], b[0][t]) and torch.equal(a[1][t], b[1][t])
    assert torch.equal(h[0][t], h2[0][t]) and torch.equal(h[1][t], h2[1][t])


def test_weight_doubling_is_exact():
    inp = _case(54, 8, 1500, 64, O.KDT_FP8)
    q, w, K, ks, pos = to_gpu(inp)
    a = S.score_topk(q, w, K, pos, 128, 8, 90, ks)
    b = S.score_topk(q, w * 2, K, pos, 128, 8, 90, ks)
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1] * 2, b[1])


def test_rows_without_keys():
    inp = _case(55, 4, 500, 64, O.KDT_BF16)
    inp["pos"][:] = np.array([-1, -5, 0, 499], dtype=np.int32)
    q, w, K, ks, pos = to_gpu(inp)
    for idx, sc in (S.score_topk(q, w, K, pos, 128, 8, 16, ks),
                    S.hier_topk(q, w, K, pos, 128, 8, 32, 16, ks),
                    S.hisa_topk(q, w, K, pos, 128, 2, 16, ks)):
        idx, sc = _np(idx), _np(sc)
        assert (idx[:2] == -1).all() and np.isneginf(sc[:2]).all()
        assert idx[2, 0] == 0 and (idx[2, 1:] == -1).all()
        assert (idx[3] >= 0).all()


# ----------------------------------------------------------------- cached block means

KBAR_CASES = [
    # seed, T, L, H, A, B, kdt
    (61, 7, 3000, 64, 8, 128, O.KDT_BF16),
    (62, 9, 20000, 32, 8, 128, O.KDT_FP8),
    (63, 5, 700, 64, 4, 64, O.KDT_FP8),
]


@pytest.mark.parametrize("source", ["pooled", "arbitrary"])
@pytest.mark.parametrize("case", KBAR_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}B{c[5]}kd{c[6]}")
def test_cached_block_means(case, source):
    """Every entry point with cached means (the library's own, or arbitrary
    rows, which must be used as given) against the oracle fed the same rows."""
    seed, T, L, H, A, B, kdt = case
    inp = _case(seed, T, L, H, kdt, positions="random")
    q, w, K, ks, pos = to_gpu(inp)
    M = -(-L // B)
    if source == "pooled":
        kbar = S.block_means(K, B, ks)
    else:
        rows = np.random.default_rng(seed).standard_normal((M, 128)).astype(np.float32) * 0.2
        kbar = torch.from_numpy(rows).cuda()
    inp = dict(inp, kbar=_np(kbar))
    heads, r = S.route(q, w, K, pos, B, A, ks, with_r=True, kbar=kbar)
    P = oracle_problem(inp, B)
    heads_o, ill = check_heads(P, A, _np(heads), _np(r))
    assert ill == 0
    idx, sc = S.score_topk(q, w, K, pos, B, A, 64, ks, kbar=kbar)
    _check_misa(inp, B, A, 64, _np(idx), _np(sc), heads_o, label="cached misa")
    idx, sc = S.hier_topk(q, w, K, pos, B, A, 256, 64, ks, kbar=kbar)
    check_hier(inp, B, A, 256, 64, _np(idx), _np(sc), label="cached hier")
    idx, sc = S.hisa_topk(q, w, K, pos, B, 4, 64, ks, kbar=kbar)
    check_hisa(inp, B, 4, 64, _np(idx), _np(sc), label="cached hisa")
    idx, sc = S.misa_hisa_topk(q, w, K, pos, B, A, 4, 64, ks, kbar=kbar)
    check_misa_hisa(inp, B, A, 4, 64, _np(idx), _np(sc), heads_o, label="cached misa-hisa")


KBAR_MANY_CASES = [
    # seed, T, L, H, A, B, kdt: enough queries for the bf16 router, with every block in
    # one range (settled in the same launch) and over several ranges (split form)
    (64, 700, 2000, 64, 8, 16, O.KDT_BF16),
    (65, 400, 5000, 32, 7, 16, O.KDT_FP8),
]


@pytest.mark.parametrize("source", ["pooled", "arbitrary"])
@pytest.mark.parametrize("case", KBAR_MANY_CASES, ids=lambda c: f"T{c[1]}L{c[2]}H{c[3]}B{c[5]}kd{c[6]}")
def test_cached_block_means_many_queries(case, source):
    seed, T, L, H, A, B, kdt = case
    inp = _case(seed, T, L, H, kdt, positions="prefill")
    q, w, K, ks, pos = to_gpu(inp)
    M = -(-L // B)
    if source == "pooled":
        kbar = S.block_means(K, B, ks)
    else:
        rows = np.random.default_rng(seed).standard_normal((M, 128)).astype(np.float32) * 0.2
        kbar = torch.from_numpy(rows).cuda()
    inp = dict(inp, kbar=_np(kbar))
    P = oracle_problem(inp, B)
    heads, r = S.route(q, w, K, pos, B, A, ks, with_r=True, kbar=kbar)
    heads_o, ill = check_heads(P, A, _np(heads), _np(r))
    assert ill == 0
    heads2 = S.route(q, w, K, pos, B, A, ks, kbar=kbar)  # placed by intervals
    _, ill = check_heads(P, A, _np(heads2))
    assert ill == 0
    idx, sc = S.score_topk(q, w, K, pos, B, A, 64, ks, kbar=kbar)
    _check_misa(inp, B, A, 64, _np(idx), _np(sc), heads_o, label="cached misa, many queries")
