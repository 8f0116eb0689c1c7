"""C-ABI checks that need no GPU: the library loads, exports every function
include/misa.h declares, and rejects bad arguments before enqueueing anything."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_block_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "misa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"misa_route", "misa_score_topk", "misa_hier_topk", "hisa_topk", "hisa_maxpool_topk",
            "misa_hisa_topk"} <= set(names)
    lib = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in misa.h but not exported"


def test_status_strings():
    L = S.lib()
    assert L.misa_status_str(0) == b"MISA_OK"
    assert L.misa_status_str(-1) == b"MISA_ERR_INVALID_ARG"
    assert L.misa_status_str(-2) == b"MISA_ERR_UNSUPPORTED"
    assert L.misa_status_str(-3) == b"MISA_ERR_WORKSPACE"
    assert L.misa_status_str(-4) == b"MISA_ERR_HIP"
    assert L.misa_status_str(7) == b"unknown misa_status"


FAKE = 1 << 20  # an aligned, never-dereferenced address: validation must fail first


def _problem(**kw):
    base = dict(T=4, H=64, d=128, L=1024, B=128, k_dtype=0, q=FAKE, w=FAKE, K=FAKE, k_scale=None, pos=FAKE,
                kbar=None)
    base.update(kw)
    return S.Problem(base["T"], base["H"], base["d"], base["L"], base["B"], base["k_dtype"],
                     base["q"], base["w"], base["K"], base["k_scale"], base["pos"], base["kbar"])


def _route(p, A=8, heads=FAKE, ws=FAKE, nbytes=1 << 40):
    return S.lib().misa_route(ctypes.byref(p), A, heads, None, ws, nbytes, None)


def _score(p, A=8, k=16, idx=FAKE, sc=FAKE, ws=FAKE, nbytes=1 << 40):
    return S.lib().misa_score_topk(ctypes.byref(p), A, None, k, idx, sc, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), -1), (dict(H=0), -1), (dict(d=0), -1), (dict(L=0), -1), (dict(B=0), -1),
    (dict(k_dtype=3), -1), (dict(d=64), -2), (dict(H=65), -2), (dict(K=None), -1),
    (dict(q=None), -1), (dict(w=None), -1), (dict(pos=None), -1), (dict(q=FAKE + 2), -1),
    (dict(K=FAKE + 8), -1), (dict(k_dtype=1), -1), (dict(k_scale=FAKE), -1),
    (dict(kbar=FAKE + 4), -1), (dict(L=(1 << 23) + 1), -2),
])
def test_problem_validation(kw, status):
    assert _route(_problem(**kw)) == status
    assert _score(_problem(**kw)) == status
    assert S.lib().misa_last_error() != b""


def test_parameter_validation():
    p = _problem()
    L = S.lib()
    assert _route(p, A=0) == -1
    assert _route(p, A=65) == -1
    assert _route(p, heads=None) == -1
    assert _score(p, k=0) == -1
    assert _score(p, idx=None) == -1
    assert _score(p, sc=FAKE + 1) == -1
    assert L.misa_hier_topk(ctypes.byref(p), 8, None, 15, 16, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    assert L.hisa_topk(ctypes.byref(p), 0, 16, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    assert L.hisa_topk(ctypes.byref(p), 4, 0, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    assert L.hisa_maxpool_topk(ctypes.byref(p), 0, 16, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    assert L.hisa_maxpool_topk(ctypes.byref(p), 4, 0, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    pk = _problem(kbar=FAKE)  # cached means do not apply to max pooling
    assert L.hisa_maxpool_topk(ctypes.byref(pk), 4, 16, FAKE, FAKE, FAKE, 1 << 40, None) == -1
    mh = lambda A, m, k, heads=None: L.misa_hisa_topk(ctypes.byref(p), A, heads, m, k, FAKE, FAKE, FAKE,
                                                       1 << 40, None)
    assert mh(0, 4, 16) == -1
    assert mh(65, 4, 16) == -1
    assert mh(8, 0, 16) == -1
    assert mh(8, 4, 0) == -1
    assert mh(8, 4, 16, heads=FAKE + 2) == -1
    # workspace too small, missing or misaligned
    need = L.misa_workspace_bytes(ctypes.byref(p), S.OP_SCORE_TOPK, 8, 1, 16, 1)
    assert need >= 256
    assert _score(p, nbytes=need - 1) == -3
    assert _score(p, ws=None) == -3
    assert _score(p, ws=FAKE + 16) == -3


def test_empty_batch_is_a_noop():
    p = _problem(T=0, q=None, w=None, pos=None)
    # nothing is enqueued, so no GPU is needed and outputs may be NULL
    assert _route(p, heads=None, ws=None, nbytes=0) == 0
    assert _score(p, idx=None, sc=None, ws=None, nbytes=0) == 0


def test_block_means_update_validation():
    L = S.lib()
    p = _problem(L=1000, B=128)  # 8 blocks
    f = lambda fb, kbar=FAKE: L.misa_block_means_update(ctypes.byref(p), fb, kbar, FAKE, 1 << 40, None)
    assert f(-1) == -1
    assert f(9) == -1
    assert f(3, kbar=None) == -1
    assert f(8) == 0  # nothing to recompute: returns before any launch


def test_workspace_sizes():
    L = S.lib()
    p = _problem(T=8, L=131072, k_dtype=1, k_scale=FAKE)
    ws = lambda op, A=8, kp=8192, k=2048, m=64: L.misa_workspace_bytes(ctypes.byref(p), op, A, kp, k, m)
    # the score rows alone take T*L*4 bytes
    assert ws(S.OP_SCORE_TOPK) >= 8 * 131072 * 4
    assert ws(S.OP_HIER_TOPK) > ws(S.OP_SCORE_TOPK)
    assert ws(S.OP_ROUTE) > 0 and ws(S.OP_HISA_TOPK) > 0 and ws(S.OP_BLOCK_MEANS) > 0
    assert ws(S.OP_HIER_TOPK, kp=100) == 0          # k' < k
    assert ws(S.OP_SCORE_TOPK, A=65) == 0
    assert ws(S.OP_HISA_TOPK, m=0) == 0
    assert ws(S.OP_MISA_HISA_TOPK) > ws(S.OP_HISA_TOPK)  # + the routed heads' packed rows
    assert ws(S.OP_MISA_HISA_TOPK, A=0) == 0 and ws(S.OP_MISA_HISA_TOPK, m=0) == 0
    assert ws(99) == 0
    for op in range(6):
        assert ws(op) % 256 == 0


@pytest.mark.parametrize("T,L,B,H", [(8, 4096, 4096, 64), (3, 1, 1, 7), (5, 1, 128, 64), (6, 257, 1, 7),
                                     (16, 131072, 128, 32), (8, 131200, 128, 64), (1, 1 << 23, 128, 64),
                                     (16384, 16384, 128, 64), (2, 300, 7, 48)])
def test_workspace_sizes_for_edge_shapes(T, L, B, H):
    # host-side planning only (no device call): single-block arrays, one-key blocks,
    # the largest supported L and router shapes on both sides of every path switch
    Lb = S.lib()
    p = _problem(T=T, L=L, B=B, H=H)
    for op in range(6):
        n = Lb.misa_workspace_bytes(ctypes.byref(p), op, min(8, H), min(8192, L), min(2048, L), 64)
        assert n > 0 and n % 256 == 0, (op, n)


def test_profile_api_without_gpu():
    assert S.lib().misa_profile_reset() == 0
    ms, n = S.profile_read("")
    assert (ms, n) == (0.0, 0)


def test_block_scores_validation():
    L = S.lib()
    p = _problem()
    M = (1024 + 127) // 128
    assert L.hisa_block_scores(ctypes.byref(p), FAKE, M - 1, FAKE, 1 << 40, None) == -1   # beta_ld < ceil(L/B)
    assert L.hisa_block_scores(ctypes.byref(p), None, M, FAKE, 1 << 40, None) == -1       # beta NULL
    assert L.hisa_block_scores(ctypes.byref(p), FAKE, M, FAKE, 16, None) == -3            # workspace too small
    assert L.misa_workspace_bytes(ctypes.byref(p), S.OP_BLOCK_SCORES, 1, 1, 1, 1) == \
        L.misa_workspace_bytes(ctypes.byref(p), S.OP_ROUTE, 1, 1, 1, 1)


def test_noalloc_rejects_oversized_problems_before_any_gpu_call():
    L = S.lib()
    p = _problem(T=64, L=1 << 21, k_dtype=1, k_scale=FAKE)
    assert L.misa_workspace_bytes(ctypes.byref(p), S.OP_HIER_TOPK, 8, 8192, 2048, 1) > S.STATIC_SCRATCH_BYTES
    st = L.misa_hier_topk_noalloc(ctypes.byref(p), 8, None, 8192, 2048, FAKE, FAKE, None)
    assert st == -3 and b"static scratch" in L.misa_last_error()
    assert L.misa_hier_topk_noalloc(ctypes.byref(_problem()), 8, None, 100, 200, FAKE, FAKE, None) == -1  # k' < k
