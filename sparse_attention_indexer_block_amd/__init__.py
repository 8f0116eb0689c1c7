"""Python binding of libmisa.so, the MI355X (gfx950) lightning-indexer library.

Argument marshalling only: every step of every call runs in the library's HIP
kernels on the current torch stream. PyTorch provides device memory and the
stream; there is no CPU or PyTorch fallback, and importing this package fails
loudly when the HIP library has not been built.

Entry points (same names as the C ABI in include/misa.h):
    block_means(K, B, k_scale=None)                     -> kbar [ceil(L/B), 128] f32
    block_means_update(K, B, kbar, first_block, k_scale=None) -> kbar (rows first_block.. recomputed)
    route(q, w, K, pos, B, A, k_scale=None, with_r=False) -> heads [T, A] i32 (, r [T, H] f32)
    score_topk(q, w, K, pos, B, A, k, k_scale=None, heads=None) -> (idx [T, k] i32, scores [T, k] f32)
    hier_topk(q, w, K, pos, B, A, kprime, k, k_scale=None, heads=None) -> (idx, scores)
    hier_topk_noalloc(q, w, K, pos, B, A, kprime, k, k_scale=None, heads=None) -> (idx, scores)
    hisa_topk(q, w, K, pos, B, m, k, k_scale=None)      -> (idx, scores)
    hisa_block_scores(q, w, K, pos, B, k_scale=None)    -> beta [T, ceil(L/B)] f32
    misa_hisa_topk(q, w, K, pos, B, A, m, k, k_scale=None, heads=None) -> (idx, scores)

Inputs are CUDA (HIP) tensors: q [T,H,128] bfloat16 (or int16 bf16 bits),
w [T,H] float32, K [L,128] bfloat16 / int16 bits, or uint8 / float8_e4m3fn
codes with k_scale [L] float32, pos [T] int32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmisa.so")

QDT_BF16, QDT_FP8 = 0, 1
OP_ROUTE, OP_SCORE_TOPK, OP_HIER_TOPK, OP_HISA_TOPK, OP_BLOCK_MEANS, OP_MISA_HISA_TOPK, OP_BLOCK_SCORES = \
    0, 1, 2, 3, 4, 5, 6
KDT_BF16, KDT_FP8 = 0, 1
STATUS = {0: "MISA_OK", -1: "MISA_ERR_INVALID_ARG", -2: "MISA_ERR_UNSUPPORTED",
          -3: "MISA_ERR_WORKSPACE", -4: "MISA_ERR_HIP"}


class MisaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("L", ctypes.c_int32), ("B", ctypes.c_int32), ("k_dtype", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("w", ctypes.c_void_p), ("K", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("kbar", ctypes.c_void_p),
                ("q_dtype", ctypes.c_int32), ("q_scale", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmisa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_indexer_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Problem)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "misa_workspace_bytes": (sz, [P, i32, i32, i32, i32, i32]),
            "misa_block_means": (i32, [P, vp, vp, sz, vp]),
            "misa_block_means_update": (i32, [P, i32, vp, vp, sz, vp]),
            "misa_route": (i32, [P, i32, vp, vp, vp, sz, vp]),
            "misa_score_topk": (i32, [P, i32, vp, i32, vp, vp, vp, sz, vp]),
            "misa_hier_topk": (i32, [P, i32, vp, i32, i32, vp, vp, vp, sz, vp]),
            "misa_hier_topk_noalloc": (i32, [P, i32, vp, i32, i32, vp, vp, vp]),
            "hisa_topk": (i32, [P, i32, i32, vp, vp, vp, sz, vp]),
            "hisa_maxpool_topk": (i32, [P, i32, i32, vp, vp, vp, sz, vp]),
            "hisa_block_scores": (i32, [P, vp, ctypes.c_int64, vp, sz, vp]),
            "misa_hisa_topk": (i32, [P, i32, vp, i32, i32, vp, vp, vp, sz, vp]),
            "misa_status_str": (ctypes.c_char_p, [i32]),
            "misa_last_error": (ctypes.c_char_p, []),
            "misa_profile_enable": (i32, [i32]),
            "misa_profile_read": (i32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]),
            "misa_profile_reset": (i32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MisaError(status, lib().misa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_problem(q: Optional[torch.Tensor], w: Optional[torch.Tensor], K: torch.Tensor,
                 pos: Optional[torch.Tensor], B: int, k_scale: Optional[torch.Tensor] = None,
                 kbar: Optional[torch.Tensor] = None, q_scale: Optional[torch.Tensor] = None):
    """Fill the C problem struct from tensors (no copies). `kbar` is an optional
    float32 [ceil(L/B), d] tensor of cached block means (see block_means).
    q as uint8 / float8_e4m3fn codes means fp8 queries, with q_scale [T,H]
    float32 (value = code * q_scale[t,h])."""
    _dev(K, "K")
    if K.dtype in (torch.uint8, torch.float8_e4m3fn):
        kdt = KDT_FP8
        if k_scale is None:
            raise ValueError("fp8 keys need k_scale")
        _dev(k_scale, "k_scale")
        if k_scale.dtype != torch.float32 or k_scale.numel() != K.shape[0]:
            raise ValueError("k_scale must be float32 [L]")
    elif K.dtype in (torch.bfloat16, torch.int16):
        kdt = KDT_BF16
        if k_scale is not None:
            raise ValueError("k_scale is only for fp8 keys")
    else:
        raise ValueError(f"unsupported key dtype {K.dtype}")
    L, d = K.shape
    T, H = 0, 1
    qdt = QDT_BF16
    if q is not None:
        _dev(q, "q"), _dev(w, "w"), _dev(pos, "pos")
        if q.dtype in (torch.uint8, torch.float8_e4m3fn):
            qdt = QDT_FP8
            if q_scale is None:
                raise ValueError("fp8 queries need q_scale")
            _dev(q_scale, "q_scale")
            if q_scale.dtype != torch.float32 or tuple(q_scale.shape) != tuple(q.shape[:2]):
                raise ValueError("q_scale must be float32 [T, H]")
        elif q.dtype in (torch.bfloat16, torch.int16):
            if q_scale is not None:
                raise ValueError("q_scale is only for fp8 queries")
        else:
            raise ValueError("q must be bfloat16 (or int16 bf16 bits), or uint8 / float8_e4m3fn codes")
        if w.dtype != torch.float32 or pos.dtype != torch.int32:
            raise ValueError("w must be float32 and pos int32")
        T, H, dq = q.shape
        if dq != d or tuple(w.shape) != (T, H) or tuple(pos.shape) != (T,):
            raise ValueError("shape mismatch between q [T,H,d], w [T,H], pos [T] and K [L,d]")
    if kbar is not None:
        _dev(kbar, "kbar")
        if kbar.dtype != torch.float32 or tuple(kbar.shape) != (-(-L // int(B)), d):
            raise ValueError("kbar must be float32 [ceil(L/B), d]")
    p = Problem(T, H, d, L, int(B), kdt, _ptr(q), _ptr(w), _ptr(K), _ptr(k_scale), _ptr(pos),
                _ptr(kbar), qdt, _ptr(q_scale if qdt == QDT_FP8 else None))
    return p


def workspace_bytes(p: Problem, op: int, A: int = 1, kprime: int = 1, k: int = 1, m: int = 1) -> int:
    n = lib().misa_workspace_bytes(ctypes.byref(p), op, A, kprime, k, m)
    if n == 0:
        raise MisaError(-1, f"invalid request for op {op} (A={A}, k'={kprime}, k={k}, m={m})")
    return n


def _workspace(p: Problem, op: int, device, ws: Optional[torch.Tensor], **kw):
    n = workspace_bytes(p, op, **kw)
    if ws is not None and ws.numel() >= n:
        return ws, n
    return torch.empty(n, dtype=torch.uint8, device=device), n


def block_means(K, B, k_scale=None, ws=None):
    p = make_problem(None, None, K, None, B, k_scale)
    M = -(-p.L // B)
    kbar = torch.empty((M, p.d), dtype=torch.float32, device=K.device)
    ws, n = _workspace(p, OP_BLOCK_MEANS, K.device, ws)
    _check(lib().misa_block_means(ctypes.byref(p), _ptr(kbar), _ptr(ws), n, _stream()))
    return kbar


def block_means_update(K, B, kbar, first_block, k_scale=None, ws=None):
    """Recompute rows first_block.. of cached block means kbar in place for the
    (grown) key array K; rows before first_block are kept."""
    p = make_problem(None, None, K, None, B, k_scale)
    M = -(-p.L // B)
    if tuple(kbar.shape) != (M, p.d) or kbar.dtype != torch.float32 or not kbar.is_contiguous():
        raise ValueError(f"kbar must be a contiguous float32 [{M}, {p.d}] tensor")
    ws, n = _workspace(p, OP_BLOCK_MEANS, K.device, ws)
    _check(lib().misa_block_means_update(ctypes.byref(p), int(first_block), _ptr(kbar), _ptr(ws), n, _stream()))
    return kbar


def route(q, w, K, pos, B, A, k_scale=None, with_r=False, ws=None, kbar=None, q_scale=None):
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    heads = torch.empty((p.T, A), dtype=torch.int32, device=q.device)
    r = torch.empty((p.T, p.H), dtype=torch.float32, device=q.device) if with_r else None
    ws, n = _workspace(p, OP_ROUTE, q.device, ws, A=A)
    _check(lib().misa_route(ctypes.byref(p), A, _ptr(heads), _ptr(r), _ptr(ws), n, _stream()))
    return (heads, r) if with_r else heads


def _outputs(p, k, device):
    return (torch.empty((p.T, k), dtype=torch.int32, device=device),
            torch.empty((p.T, k), dtype=torch.float32, device=device))


def score_topk(q, w, K, pos, B, A, k, k_scale=None, heads=None, ws=None, out=None, kbar=None, q_scale=None):
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    if heads is not None:
        _dev(heads, "heads")
        if heads.dtype != torch.int32 or tuple(heads.shape) != (p.T, A):
            raise ValueError("heads must be int32 [T, A]")
    idx, sc = out if out is not None else _outputs(p, k, q.device)
    ws, n = _workspace(p, OP_SCORE_TOPK, q.device, ws, A=A, k=k)
    _check(lib().misa_score_topk(ctypes.byref(p), A, _ptr(heads), k, _ptr(idx), _ptr(sc),
                                 _ptr(ws), n, _stream()))
    return idx, sc


def hier_topk(q, w, K, pos, B, A, kprime, k, k_scale=None, heads=None, ws=None, out=None,
              kbar=None, q_scale=None):
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    if heads is not None:
        _dev(heads, "heads")
        if heads.dtype != torch.int32 or tuple(heads.shape) != (p.T, A):
            raise ValueError("heads must be int32 [T, A]")
    idx, sc = out if out is not None else _outputs(p, k, q.device)
    ws, n = _workspace(p, OP_HIER_TOPK, q.device, ws, A=A, kprime=kprime, k=k)
    _check(lib().misa_hier_topk(ctypes.byref(p), A, _ptr(heads), kprime, k, _ptr(idx), _ptr(sc),
                                _ptr(ws), n, _stream()))
    return idx, sc


def hier_topk_noalloc(q, w, K, pos, B, A, kprime, k, k_scale=None, heads=None, out=None, kbar=None, q_scale=None):
    """misa_hier_topk_noalloc: hier_topk with the library's static device
    scratch instead of a workspace (nothing is allocated by the call; pass
    `out` to allocate nothing here either)."""
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    if heads is not None:
        _dev(heads, "heads")
        if heads.dtype != torch.int32 or tuple(heads.shape) != (p.T, A):
            raise ValueError("heads must be int32 [T, A]")
    idx, sc = out if out is not None else _outputs(p, k, q.device)
    _check(lib().misa_hier_topk_noalloc(ctypes.byref(p), A, _ptr(heads), kprime, k, _ptr(idx), _ptr(sc),
                                        _stream()))
    return idx, sc


STATIC_SCRATCH_BYTES = 32 << 20  # MISA_STATIC_SCRATCH_BYTES


def hisa_topk(q, w, K, pos, B, m, k, k_scale=None, ws=None, out=None, kbar=None, q_scale=None):
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    idx, sc = out if out is not None else _outputs(p, k, q.device)
    ws, n = _workspace(p, OP_HISA_TOPK, q.device, ws, m=m, k=k)
    _check(lib().hisa_topk(ctypes.byref(p), m, k, _ptr(idx), _ptr(sc), _ptr(ws), n, _stream()))
    return idx, sc


def hisa_block_scores(q, w, K, pos, B, k_scale=None, ws=None, kbar=None, q_scale=None):
    """HISA Stage 1 block scores beta [T, ceil(L/B)] float32; entries past a
    query's visible blocks are -inf (filled here before the call; the library
    writes only the visible blocks)."""
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    M = -(-p.L // int(B))
    beta = torch.full((p.T, M), float("-inf"), dtype=torch.float32, device=q.device)
    ws, n = _workspace(p, OP_BLOCK_SCORES, q.device, ws)
    _check(lib().hisa_block_scores(ctypes.byref(p), _ptr(beta), M, _ptr(ws), n, _stream()))
    return beta


def hisa_maxpool_topk(q, w, K, pos, B, m, k, k_scale=None, ws=None, out=None, q_scale=None):
    p = make_problem(q, w, K, pos, B, k_scale, None, q_scale)
    idx, sc = out if out is not None else _outputs(p, k, q.device)
    ws, n = _workspace(p, OP_HISA_TOPK, q.device, ws, m=m, k=k)
    _check(lib().hisa_maxpool_topk(ctypes.byref(p), m, k, _ptr(idx), _ptr(sc), _ptr(ws), n, _stream()))
    return idx, sc


def misa_hisa_topk(q, w, K, pos, B, A, m, k, k_scale=None, heads=None, ws=None, out=None, kbar=None, q_scale=None):
    p = make_problem(q, w, K, pos, B, k_scale, kbar, q_scale)
    if heads is not None:
        _dev(heads, "heads")
        if heads.dtype != torch.int32 or tuple(heads.shape) != (p.T, A):
            raise ValueError("heads must be int32 [T, A]")
    idx, sc = out if out is not None else _outputs(p, k, q.device)
    ws, n = _workspace(p, OP_MISA_HISA_TOPK, q.device, ws, A=A, m=m, k=k)
    _check(lib().misa_hisa_topk(ctypes.byref(p), A, _ptr(heads), m, k, _ptr(idx), _ptr(sc), _ptr(ws), n,
                                _stream()))
    return idx, sc


def profile_enable(on: bool = True):
    _check(lib().misa_profile_enable(1 if on else 0))


def profile_read(name_substr: str = ""):
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(lib().misa_profile_read(name_substr.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def profile_reset():
    _check(lib().misa_profile_reset())
