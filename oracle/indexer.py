"""CPU oracle for the MISA / MISA-dagger / HISA lightning-indexer hot path.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg use this module.  The HIP library never imports, links or calls it,
and it shares no code with the HIP library (only the seeded input generator
feeds both).

Everything here is plain, slow and meant to be read against the pages:
numpy in float64, one query at a time, a matrix product and a sort as the only
library steps.  Every input is an exact value (bf16 and E4M3FN are decoded from
their bit layouts, fp32 weights and scales widen exactly) and every product of
two inputs is exact in float64.

Citations name the page and its section:
  [DSA]   MISA write-up (zingnex forum), "DSA" and "the indexer's cost dilemma";
          HISA write-up (zhichai), section 2 "How DSA works".
  [MISA]  MISA technical summary (gist.science), "Metodologia: MISA" - block
          router over M = ceil(L/B) mean-pooled key blocks, top-h heads, then
          sparse token scoring with only the routed heads and top-k.
  [MISA+] same summary, "Variante Jerarquica (MISA-dagger)" - routed pass picks
          k' candidates, the full H_I-head indexer reranks them to top-k.
  [HISA]  HISA write-up, section 3 "Stage 1" (blocks of B, mean-pooled
          representatives, top-m blocks) and "Stage 2" (token-level indexer
          inside the chosen blocks).

Where the pages leave a formula open, the fixed reading is:
  * index score I_S(t,s) = sum_{h in S} w[t,h] * ReLU(q[t,h] . k[s]); dense DSA
    is S = all heads.
  * key s is visible to query t iff s <= pos[t]; n_t = pos[t] + 1 (clamped to
    [0, L]).
  * blocks of query t: M_t = ceil(n_t / B); block b covers
    [b*B, min((b+1)*B, n_t)) and its representative is the mean of those keys,
    so the last block of a query may be a partial ("tail") block.
  * router score r(t,h) = w[t,h] * max_b ReLU(q[t,h] . Kbar_{t,b}); the routed
    set is the first A heads under the key (-r, h).
  * HISA block score beta(t,b) = sum_h w[t,h] * ReLU(q[t,h] . Kbar_{t,b}).
  * HISA with max pooling (the HISA write-up's limitations section names max
    pooling in place of mean pooling as a possible improvement): the
    representative of a block is, per dimension, the largest of its visible
    keys' values (the tail block over its visible keys only); beta and the
    refine are otherwise unchanged.  Cached means do not apply to it.
  * MISA inside HISA (the head axis and the token axis combined, as the MISA
    summary's "Contribuciones Clave" and "Significado y Afirmaciones" call them
    complementary): the routed heads R_t replace all H heads in both HISA
    stages, beta_R(t,b) = sum_{h in R_t} w[t,h] * ReLU(q[t,h] . Kbar_{t,b}) and
    I_R on the chosen blocks' tokens.
  * every selection keeps the first min(k, n) items under (-score, index);
    -0.0 compares equal to +0.0.
"""
from __future__ import annotations

import numpy as np

KDT_BF16 = 0
KDT_FP8 = 1
QDT_BF16 = 0
QDT_FP8 = 1


# ---------------------------------------------------------------- decoding

def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64, from the format: 1 sign, 8 exponent
    (bias 127), 7 mantissa bits; exponent 0 is subnormal, 255 is inf/NaN."""
    b = np.asarray(bits).astype(np.uint32) & 0xFFFF
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = ((b >> 7) & 0xFF).astype(np.int64)
    m = (b & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 128.0, e - 127)
    sub = sign * np.ldexp(m / 128.0, -126)
    special = np.where(m == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 255, special, normal))


def decode_e4m3fn(bits) -> np.ndarray:
    """OCP E4M3FN bytes -> float64: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity."""
    b = np.asarray(bits).astype(np.uint32) & 0xFF
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = ((b >> 3) & 0xF).astype(np.int64)
    m = (b & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, e - 7)
    sub = sign * np.ldexp(m / 8.0, -6)
    val = np.where(e == 0, sub, normal)
    return np.where((b & 0x7F) == 0x7F, np.nan, val)


def dequant_keys(K, k_dtype: int, k_scale=None) -> np.ndarray:
    """Key values in float64: bf16 keys as decoded; fp8 keys are code * scale
    with one fp32 scale per token (the product is exact in float64)."""
    if k_dtype == KDT_BF16:
        return decode_bf16(K)
    codes = decode_e4m3fn(K)
    return codes * np.asarray(k_scale, dtype=np.float32).astype(np.float64)[:, None]


def dequant_queries(q, q_dtype: int, q_scale=None) -> np.ndarray:
    """Query values in float64: bf16 queries as decoded; fp8 queries are E4M3FN
    codes times one fp32 scale per (query, head) (the product is exact)."""
    if q_dtype == QDT_BF16:
        return decode_bf16(q)
    codes = decode_e4m3fn(q)
    return codes * np.asarray(q_scale, dtype=np.float32).astype(np.float64)[:, :, None]


class Problem:
    """Decoded inputs of one indexer call (float64 copies, exact).

    kbar, when given, is a float32 [ceil(L/B), d] array of cached block means:
    row b stands for the mean of block b wherever that block is complete and
    lies before the query's own last block (the router's block statistics are
    query independent there [MISA]); a query's last block is always pooled from
    its visible keys.

    q is bf16 bits, or (q_dtype QDT_FP8) E4M3FN codes with q_scale [T,H]: the
    value of q[t,h,i] is code * q_scale[t,h]; the definitions are unchanged."""

    def __init__(self, q_bits, w, K, pos, B, k_dtype=KDT_BF16, k_scale=None, kbar=None,
                 q_dtype=QDT_BF16, q_scale=None):
        self.q = dequant_queries(q_bits, q_dtype, q_scale)             # [T,H,d]
        self.w = np.asarray(w, dtype=np.float32).astype(np.float64)   # [T,H]
        self.K = dequant_keys(K, k_dtype, k_scale)                     # [L,d]
        self.pos = np.asarray(pos, dtype=np.int64)
        self.B = int(B)
        self.T, self.H, self.d = self.q.shape
        self.L = self.K.shape[0]
        self.kbar = None if kbar is None else np.asarray(kbar, dtype=np.float32).astype(np.float64)

    def n(self, t: int) -> int:
        """Visible prefix length of query t: keys s <= pos[t]."""
        return int(min(max(self.pos[t] + 1, 0), self.L))


# ---------------------------------------------------------------- scores

def _canon(x):
    """Make -0.0 compare and sort as +0.0."""
    return np.asarray(x, dtype=np.float64) + 0.0


def head_logits(P: Problem, t: int, heads, keys) -> np.ndarray:
    """z(t,h,s) = q[t,h] . k[s] for the given heads and key indices [DSA]."""
    return P.q[t, list(heads)] @ P.K[np.asarray(keys, dtype=np.int64)].T


def routed_scores(P: Problem, t: int, heads, keys) -> np.ndarray:
    """I_S(t,s) = sum_{h in S} w[t,h] * ReLU(z(t,h,s)) over the routed subset S
    only, with no renormalisation of w [MISA, sparse token scoring]."""
    heads = list(heads)
    z = head_logits(P, t, heads, keys)
    return _canon((P.w[t, heads][:, None] * np.maximum(z, 0.0)).sum(axis=0))


def dense_scores(P: Problem, t: int, keys) -> np.ndarray:
    """The full DSA indexer: every one of the H heads scores every key [DSA].
    Written separately from routed_scores so that 'A = H gives DSA' is a real
    cross-check rather than the same code twice."""
    kk = P.K[np.asarray(keys, dtype=np.int64)]
    out = np.zeros(len(kk))
    for h in range(P.H):
        out += P.w[t, h] * np.maximum(kk @ P.q[t, h], 0.0)
    return _canon(out)


def magnitude_terms(P: Problem, t: int, heads, keys):
    """Companion magnitudes for floating-point tolerances (not part of the
    method): Ibar = sum_h |w| ReLU(z) and Jhat = sum_h |w| sum_i |q_i k_i|."""
    heads = list(heads)
    kk = P.K[np.asarray(keys, dtype=np.int64)]
    qa = np.abs(P.q[t, heads])
    wa = np.abs(P.w[t, heads])[:, None]
    z = P.q[t, heads] @ kk.T
    ibar = (wa * np.maximum(z, 0.0)).sum(axis=0)
    jhat = (wa * (qa @ np.abs(kk).T)).sum(axis=0)
    return ibar, jhat


# ---------------------------------------------------------------- blocks

def block_ranges(n: int, B: int):
    """The prefix [0, n) cut into M = ceil(n/B) contiguous blocks; the last one
    may be partial [MISA, M = ceil(L/B) blocks; HISA Stage 1]."""
    M = -(-n // B)
    return [(b * B, min((b + 1) * B, n)) for b in range(M)]


def block_means(P: Problem, t: int) -> np.ndarray:
    """Kbar_{t,b}: the mean of the visible keys of each block [MISA, the router's
    block statistics are averaged indexer keys; HISA Stage 1, each block is
    represented by the mean of its keys]."""
    rng = block_ranges(P.n(t), P.B)
    out = np.zeros((len(rng), P.d))
    for b, (s0, s1) in enumerate(rng):
        if P.kbar is not None and b < len(rng) - 1:
            out[b] = P.kbar[b]          # cached mean of a complete earlier block
        else:
            out[b] = P.K[s0:s1].sum(axis=0) / (s1 - s0)
    return out


def full_block_means(K_values: np.ndarray, B: int) -> np.ndarray:
    """Means of the blocks of the whole key array (the last may be partial);
    the query-independent part of the router's statistics."""
    L = K_values.shape[0]
    return np.stack([K_values[s0:s1].sum(axis=0) / (s1 - s0) for s0, s1 in block_ranges(L, B)]) \
        if L > 0 else np.zeros((0, K_values.shape[1]))


def block_maxima(P: Problem, t: int) -> np.ndarray:
    """Max-pooled representatives: per dimension, the largest visible key value
    of each block [HISA write-up, limitations: max pooling in place of mean
    pooling]."""
    rng = block_ranges(P.n(t), P.B)
    out = np.zeros((len(rng), P.d))
    for b, (s0, s1) in enumerate(rng):
        out[b] = P.K[s0:s1].max(axis=0)
    return out


def block_logits(P: Problem, t: int) -> np.ndarray:
    """rho(t,h,b) = q[t,h] . Kbar_{t,b}, shape [H, M_t]."""
    return P.q[t] @ block_means(P, t).T


# ---------------------------------------------------------------- selection

def first_k(scores, idx, k: int):
    """The first min(k, n) items under the key (-score, index).  Returns
    (chosen indices, their scores) in that order."""
    scores = _canon(scores)
    idx = np.asarray(idx, dtype=np.int64)
    order = np.lexsort((idx, -scores))[: min(int(k), len(idx))]
    return idx[order], scores[order]


# ---------------------------------------------------------------- the method

def route(P: Problem, A: int):
    """MISA router [MISA, lightweight block-pooled router]: per head, the
    affinity to every block representative, aggregated as
    r = w * max_b ReLU(rho); keep the top-A heads, lower index first on ties.
    Returns (heads [T,A] ascending, r [T,H])."""
    heads = np.zeros((P.T, A), dtype=np.int64)
    r = np.zeros((P.T, P.H))
    for t in range(P.T):
        rho = block_logits(P, t)
        peak = np.maximum(rho, 0.0).max(axis=1) if rho.shape[1] else np.zeros(P.H)
        r[t] = _canon(P.w[t] * peak)
        chosen, _ = first_k(r[t], np.arange(P.H), A)
        heads[t] = np.sort(chosen)
    return heads, r


def misa_topk(P: Problem, A: int, k: int, heads=None):
    """MISA [MISA, sparse token scoring]: only the routed heads score the whole
    visible prefix; top-k on the reduced score.  Returns a list of
    (indices, scores) per query, plus the heads used."""
    if heads is None:
        heads, _ = route(P, A)
    out = []
    for t in range(P.T):
        keys = np.arange(P.n(t))
        out.append(first_k(routed_scores(P, t, heads[t], keys), keys, k))
    return out, heads


def dense_topk(P: Problem, k: int):
    """The dense DSA indexer: all H heads, top-k over the visible prefix [DSA]."""
    out = []
    for t in range(P.T):
        keys = np.arange(P.n(t))
        out.append(first_k(dense_scores(P, t, keys), keys, k))
    return out


def misa_hier_topk(P: Problem, A: int, kprime: int, k: int, heads=None):
    """MISA-dagger [MISA+]: the routed pass keeps an enlarged set of k'
    candidates; the full H-head indexer rescores only those and keeps top-k."""
    if heads is None:
        heads, _ = route(P, A)
    out, cands = [], []
    for t in range(P.T):
        keys = np.arange(P.n(t))
        cand, _ = first_k(routed_scores(P, t, heads[t], keys), keys, kprime)
        cands.append(cand)
        out.append(first_k(dense_scores(P, t, cand), cand, k))
    return out, heads, cands


def hisa_block_scores(P: Problem, t: int, pool: str = "mean") -> np.ndarray:
    """beta(t,b): the indexer formula with all H heads applied to the block
    representatives [HISA Stage 1: the query scores only the representatives];
    pool="max" takes the max-pooled representatives instead of the means."""
    rho = block_logits(P, t) if pool == "mean" else P.q[t] @ block_maxima(P, t).T
    return _canon((P.w[t][:, None] * np.maximum(rho, 0.0)).sum(axis=0))


def hisa_topk(P: Problem, m: int, k: int, pool: str = "mean"):
    """HISA [HISA Stage 1 + Stage 2]: keep the top-m blocks by beta (lower block
    index first on ties), run the token-level indexer on the visible tokens of
    those blocks only, keep top-k.  pool selects mean (the pages' method) or
    max-pooled block representatives.  Returns (per-query results, chosen
    blocks)."""
    assert pool in ("mean", "max")
    out, chosen = [], []
    for t in range(P.T):
        beta = hisa_block_scores(P, t, pool)
        blocks, _ = first_k(beta, np.arange(len(beta)), m)
        chosen.append(np.sort(blocks))
        rng = block_ranges(P.n(t), P.B)
        cand = np.concatenate([np.arange(*rng[b]) for b in np.sort(blocks)]) if len(blocks) \
            else np.zeros(0, dtype=np.int64)
        out.append(first_k(dense_scores(P, t, cand), cand, k))
    return out, chosen


def routed_block_scores(P: Problem, t: int, heads) -> np.ndarray:
    """beta_R(t,b): the block score of HISA Stage 1 with only the routed heads
    R_t [HISA Stage 1; MISA, the router's head subset]."""
    heads = list(heads)
    rho = block_logits(P, t)[heads]
    return _canon((P.w[t, heads][:, None] * np.maximum(rho, 0.0)).sum(axis=0))


def misa_hisa_topk(P: Problem, A: int, m: int, k: int, heads=None):
    """MISA inside HISA: route A heads per query [MISA], keep the top-m blocks
    by beta_R (lower block index first on ties) [HISA Stage 1], score the
    visible tokens of those blocks with I_R and keep top-k [HISA Stage 2 with
    the routed heads].  Returns (per-query results, chosen blocks, heads)."""
    if heads is None:
        heads, _ = route(P, A)
    out, chosen = [], []
    for t in range(P.T):
        beta = routed_block_scores(P, t, heads[t])
        blocks, _ = first_k(beta, np.arange(len(beta)), m)
        blocks = np.sort(blocks)
        chosen.append(blocks)
        rng = block_ranges(P.n(t), P.B)
        cand = np.concatenate([np.arange(*rng[b]) for b in blocks]) if len(blocks) \
            else np.zeros(0, dtype=np.int64)
        out.append(first_k(routed_scores(P, t, heads[t], cand), cand, k))
    return out, chosen, heads
