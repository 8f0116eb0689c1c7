"""Seeded synthetic inputs for the lightning-indexer hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
builds inputs only: it holds none of the indexer's arithmetic (no scores, no
block means, no routing, no selection).  Both the HIP library and the CPU
oracle receive the arrays made here and decode them on their own.

Workload shapes follow the five decode / prefill configurations of the
MISA and HISA indexer studies:

* DeepSeek-V3.2 uses H_I = 64 indexer heads, GLM-5 uses H_I = 32; routing keeps
  h = 8 of them (MISA page, "Resultados Experimentales" / Technical summary).
* MISA-dagger enlarges the candidate set to k' = 8192 before the full-head rerank
  (MISA page, "Variante Jerarquica").
* HISA uses blocks of B = 128 tokens, keeps m = 64 blocks and refines to
  k = 2048 tokens (HISA page, section 5 "Kernel-level acceleration" and section 6).
* Needle-in-a-haystack style planted keys stand in for the retrieval test both
  pages run (HISA page, section 5 "Needle-in-a-Haystack"); no benchmark item is
  reproduced.

Encodings:
* bf16 values are produced by round-to-nearest-even from fp32 (torch's CPU cast)
  and handed over as raw uint16 bit patterns.
* fp8 keys are OCP E4M3FN bytes with one fp32 scale per token, scale = amax/448;
  values are clipped to +-448 before the cast so nothing saturates to NaN.
* fp8 queries (q_fp8=True) are E4M3FN bytes with one fp32 scale per
  (query, head) row, quantised the same way.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

KDT_BF16 = 0
KDT_FP8 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic indexer problem description (shapes and knobs, no data)."""

    name: str
    T: int                 # number of queries
    L: int                 # number of keys
    H: int                 # indexer heads
    d: int = 128           # head dim
    B: int = 128           # router / HISA block size
    A: int = 8             # routed (active) heads
    k: int = 2048          # final top-k
    kprime: int = 8192     # MISA-dagger candidate count
    m: int = 64            # HISA blocks kept
    k_dtype: int = KDT_BF16
    positions: str = "decode"   # "decode": last T positions; "prefill": pos[t] = t
    needles: int = 0            # planted needle keys per query
    needle_mode: str = "uniform"  # uniform | stratified | mid_lowblock
    block_offsets: float = 0.0  # variance of per-block mean offsets added to K


# The five workloads, in the order the benchmark table lists them.
CONFIGS = {
    "c1_tiny_decode": Workload("c1_tiny_decode", T=16, L=4096, H=64, k=512,
                               needles=4, needle_mode="uniform"),
    "c2_decode_batch": Workload("c2_decode_batch", T=32, L=32768, H=64, k=2048,
                                needles=16, needle_mode="stratified"),
    "c3_causal_prefill": Workload("c3_causal_prefill", T=16384, L=16384, H=64, k=2048,
                                  positions="prefill", block_offsets=0.5),
    "c4_hier_decode_128k": Workload("c4_hier_decode_128k", T=8, L=131072, H=64, k=2048,
                                    kprime=8192, k_dtype=KDT_FP8, needles=32,
                                    needle_mode="uniform"),
    "c5_glm5_hisa_128k": Workload("c5_glm5_hisa_128k", T=16, L=131072, H=32, k=2048,
                                  m=64, k_dtype=KDT_FP8, needles=4,
                                  needle_mode="mid_lowblock"),
}

CONFIG_ORDER = list(CONFIGS)


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) with round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact); used only to build needles."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3FN bytes (RNE); callers pre-scale into [-448, 448]."""
    xc = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(xc)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_keys_fp8(kf: np.ndarray):
    """Per-token fp8 quantisation: scale = amax/448 (1.0 for an all-zero row)."""
    amax = np.abs(kf).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = encode_e4m3fn(kf / scale[:, None])
    return codes, scale


def quantize_queries_fp8(q32: np.ndarray):
    """Per-(query, head) fp8 quantisation of q [T,H,d]: codes [T,H,d] uint8 and
    scales [T,H] float32 (amax/448; 1.0 for an all-zero row)."""
    T, H, d = q32.shape
    codes, scale = quantize_keys_fp8(q32.reshape(T * H, d))
    return codes.reshape(T, H, d), scale.reshape(T, H)


def fp8_codes_to_f32(codes: np.ndarray) -> np.ndarray:
    """E4M3FN bytes -> float32 (exact); used only to build needles."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def positions_for(wl: Workload) -> np.ndarray:
    if wl.positions == "prefill":
        assert wl.T <= wl.L
        return np.arange(wl.T, dtype=np.int32)
    return np.arange(wl.L - wl.T, wl.L, dtype=np.int32)


def _needle_slots(rng, wl: Workload, pos: np.ndarray):
    """Distinct needle positions per query, never shared between queries."""
    used = set()
    out = []
    for t in range(wl.T):
        hi = int(pos[t])  # needles live strictly before the query's own key
        slots = []
        tries = 0
        while len(slots) < wl.needles and tries < 100000:
            tries += 1
            j = len(slots)
            if wl.needle_mode == "stratified":
                seg = hi // wl.needles
                s = int(rng.integers(j * seg, max(j * seg + 1, (j + 1) * seg)))
            elif wl.needle_mode == "mid_lowblock":
                lo_b = (hi // 4) // wl.B
                hi_b = max(lo_b + 1, (3 * hi // 4) // wl.B)
                b = int(rng.integers(lo_b, hi_b))
                s = b * wl.B + int(rng.integers(0, wl.B))
                # one needle per block, blocks not shared between queries
                if any((u // wl.B) == b for u in used) or s >= hi:
                    continue
            else:
                s = int(rng.integers(0, max(1, hi)))
            if s in used or s >= hi:
                continue
            used.add(s)
            slots.append(s)
        out.append(slots)
    return out


def make_inputs(wl: Workload, seed: int = 0, T: Optional[int] = None, q_fp8: bool = False):
    """Build one seeded problem.

    Returns a dict of numpy arrays:
      q      [T,H,d] uint16 (bf16 bits), or uint8 E4M3FN codes with q_fp8
      q_scale[T,H]   float32 per-(query, head) scale (q_fp8 only, else None)
      w      [T,H]   float32
      K      [L,d]   uint16 (bf16 bits) or uint8 (e4m3fn bytes)
      k_scale[L]     float32 (fp8 only, else None)
      pos    [T]     int32
      needles list of per-query planted key positions
    Streams: q, w, K and needles each draw from their own child of
    SeedSequence(seed), so changing one recipe leaves the others intact.
    """
    if T is not None:
        wl = dataclasses.replace(wl, T=T)
    ss = np.random.SeedSequence(seed)
    rq, rw, rk, rn = [np.random.default_rng(s) for s in ss.spawn(4)]
    pos = positions_for(wl)

    q32 = rq.standard_normal((wl.T, wl.H, wl.d), dtype=np.float32)
    if q_fp8:
        q_bits, q_scale = quantize_queries_fp8(q32)
        qv = fp8_codes_to_f32(q_bits) * q_scale[:, :, None]
    else:
        q_bits, q_scale = encode_bf16(q32), None
        qv = bf16_bits_to_f32(q_bits)
    w = (rw.standard_normal((wl.T, wl.H), dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    kf = rk.standard_normal((wl.L, wl.d), dtype=np.float32)
    if wl.block_offsets > 0:
        nb = (wl.L + wl.B - 1) // wl.B
        mu = rk.standard_normal((nb, wl.d), dtype=np.float32) * np.float32(np.sqrt(wl.block_offsets))
        kf += np.repeat(mu, wl.B, axis=0)[: wl.L]

    needles = [[] for _ in range(wl.T)]
    if wl.needles > 0:
        needles = _needle_slots(rn, wl, pos)
        for t, slots in enumerate(needles):
            hstar = int(np.argmax(w[t]))
            for s in slots:
                kf[s] = qv[t, hstar] + np.float32(0.1) * rn.standard_normal(wl.d, dtype=np.float32)
                if wl.needle_mode == "mid_lowblock":
                    b0 = (s // wl.B) * wl.B
                    b1 = min(b0 + wl.B, wl.L)
                    others = [u for u in range(b0, b1) if u != s]
                    kf[others] -= np.float32(2.0) * qv[t, hstar] / np.float32(max(1, len(others)))

    if wl.k_dtype == KDT_FP8:
        K, k_scale = quantize_keys_fp8(kf)
    else:
        K, k_scale = encode_bf16(kf), None
    return {"q": q_bits, "q_scale": q_scale, "w": w, "K": K, "k_scale": k_scale, "pos": pos,
            "needles": needles, "wl": wl}


def random_small(seed: int, T: int, L: int, H: int, d: int = 128, k_dtype: int = KDT_BF16,
                 positions: str = "random", w_scale: float = 0.125, int_grid: bool = False,
                 q_fp8: bool = False):
    """Small randomised problems for sweeps and edge cases.

    positions: "random" (uniform in [0, L)), "decode" (last T), "prefill" (pos[t]=t, T<=L)
    int_grid: draw q, K and w from a small dyadic grid so exact ties are common.
    q_fp8: q as E4M3FN codes with a per-(query, head) scale (inp["q_scale"]).
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, T, L, H, d, k_dtype]))
    if int_grid:
        q32 = rng.integers(-2, 3, size=(T, H, d)).astype(np.float32) * np.float32(0.5)
        kf = rng.integers(-2, 3, size=(L, d)).astype(np.float32) * np.float32(0.5)
        w = rng.choice(np.array([-1.0, -0.5, 0.0, 0.5, 1.0], dtype=np.float32), size=(T, H))
    else:
        q32 = rng.standard_normal((T, H, d), dtype=np.float32)
        kf = rng.standard_normal((L, d), dtype=np.float32)
        w = (rng.standard_normal((T, H), dtype=np.float32) * np.float32(w_scale)).astype(np.float32)
    if positions == "decode":
        pos = np.arange(L - T, L, dtype=np.int32)
    elif positions == "prefill":
        pos = (np.arange(T) % L).astype(np.int32)
    else:
        pos = rng.integers(0, L, size=T).astype(np.int32)
    if k_dtype == KDT_FP8:
        K, k_scale = quantize_keys_fp8(kf)
    else:
        K, k_scale = encode_bf16(kf), None
    if q_fp8:
        q, q_scale = quantize_queries_fp8(q32)
    else:
        q, q_scale = encode_bf16(q32), None
    return {"q": q, "q_scale": q_scale, "w": w.astype(np.float32), "K": K, "k_scale": k_scale,
            "pos": pos, "needles": [[] for _ in range(T)]}
