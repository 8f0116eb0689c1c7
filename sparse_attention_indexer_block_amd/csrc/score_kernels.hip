// Token scoring on the matrix cores (gfx950 MFMA, bf16 in / fp32 accumulate).
//
// I_S(t,s) = sum_{h in S} w[t,h] * ReLU(q[t,h] . k[s])   (MISA technical summary,
// "Metodologia: MISA": only the routed heads score the prefix; with S = all
// heads this is the DSA indexer of the MISA forum post's "DSA" section).
//
// Layout of the contraction: the M side of each 16x16x32 MFMA holds (query,
// routed-head slot) rows gathered from q in registers, the N side holds 16
// keys staged through LDS, and K = head dim 128 takes four MFMAs. Because all
// AP slots of a query sit in one MFMA row group, the epilogue (ReLU, times w,
// head sum) is a lane-local sum plus at most two cross-lane adds; per-head
// logits never leave registers. fp8 keys are widened to bf16 exactly when the
// tile is written to LDS; the per-token scale is positive-homogeneous through
// ReLU, so |scale| multiplies the head sum and the scale's sign is folded into
// the key.
#include "device_common.h"
#include "launch.h"

namespace misa {

constexpr int kLdsStride = kHeadDim + 8;  // bf16 per key row in LDS (16 B pad)

template <int AP, int WR, int RPW, int CPW, bool FP8, bool GATHER>
__global__ __launch_bounds__(256) void k_score(ScoreArgs p) {
  constexpr int WC = 4 / WR;
  constexpr int ROWS = WR * RPW * 16;
  constexpr int QW = ROWS / AP;                     // queries per workgroup
  constexpr int KT = WC * CPW * 16;                 // keys per LDS tile
  constexpr int TPQ = AP >= 16 ? AP / 16 : 1;       // row tiles per query
  constexpr int CH_PER_ROW = FP8 ? 8 : 16;          // 16-byte global chunks per key row
  constexpr int CHUNKS = KT * CH_PER_ROW / 256;     // chunks per thread per tile
  static_assert(AP >= 4 && (AP & (AP - 1)) == 0, "AP must be a power of two >= 4");
  static_assert(ROWS % AP == 0 && QW >= 1, "row tiles must hold whole queries");
  static_assert(AP < 16 || RPW % TPQ == 0, "a wave must hold whole queries");
  static_assert(!GATHER || QW == 1, "gather mode scores one query per workgroup");
  static_assert(CHUNKS >= 1 && KT * CH_PER_ROW % 256 == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint16_t ktile[2][KT * kLdsStride];
  __shared__ float ksc[2][KT];
  __shared__ int kkey[2][KT];
  __shared__ int qn[QW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WC, wc = wave % WC;
  const int g = GATHER ? (int)blockIdx.y : (p.reverse ? p.ngroups - 1 - (int)blockIdx.x : (int)blockIdx.x);
  const int split = GATHER ? (int)blockIdx.x : (int)blockIdx.y;

  if (tid < QW) {
    const int t = g * QW + tid;
    int nn = 0;
    if (t < p.T) nn = GATHER ? p.ncand[t] : visible_len(p.pos[t], p.L);
    qn[tid] = nn;
  }
  __syncthreads();
  int nmax = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) nmax = qn[i] > nmax ? qn[i] : nmax;
  const int ntiles = (nmax + KT - 1) / KT;
  const int tile0 = split * p.tiles_per_split;
  const int tile1 = min(ntiles, tile0 + p.tiles_per_split);
  if (tile0 >= tile1) return;  // uniform over the workgroup

  // ---- A operand (gathered q rows) and epilogue weights, kept in registers.
  bf16x8 afrag[RPW][4];
  float wv[RPW][4];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rt = wr * RPW + r;
    {
      const int row = rt * 16 + (lane & 15);
      const int qi = row / AP, j = row % AP, t = g * QW + qi;
      int h = -1;
      if (t < p.T && j < p.A) h = p.heads ? p.heads[(size_t)t * p.A + j] : j;
      if (h >= p.H) h = -1;  // out-of-range head ids score nothing
      if (h >= 0) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(
            p.q + ((size_t)t * p.H + h) * kHeadDim + 32 * (lane >> 4));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) afrag[r][ks] = src[ks];
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) afrag[r][ks] = bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + 4 * (lane >> 4) + i;
      const int qi = row / AP, j = row % AP, t = g * QW + qi;
      float wvv = 0.f;
      if (t < p.T && j < p.A) {
        const int h = p.heads ? p.heads[(size_t)t * p.A + j] : j;
        if (h >= 0 && h < p.H) wvv = p.w[(size_t)t * p.H + h];
      }
      wv[r][i] = wvv;
    }
  }

  // ---- staging of one key tile: global -> registers -> LDS
  u32x4 stage[CHUNKS];
  uint32_t stage_flip[CHUNKS];  // fp8: 0x80008000 when the key's scale is negative
  float stage_sc = 0.f;
  int stage_key = -1;
  const int qt0 = g * QW;  // gather: the single query

  auto key_of = [&](int tile, int kr) -> int {
    const int col = tile * KT + kr;
    if constexpr (GATHER) {
      return col < qn[0] ? p.cand[(size_t)qt0 * p.cand_ld + col] : -1;
    } else {
      return col < p.L ? col : -1;
    }
  };

  auto load_tile = [&](int tile) {
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int c = tid + 256 * u;
      const int kr = c / CH_PER_ROW, part = c % CH_PER_ROW;
      const int s = key_of(tile, kr);
      stage_flip[u] = 0u;
      if (s >= 0) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(p.K) +
                              (size_t)s * (FP8 ? kHeadDim : 2 * kHeadDim) + 16 * part;
        stage[u] = *reinterpret_cast<const u32x4*>(base);
        if constexpr (FP8) stage_flip[u] = p.kscale[s] < 0.f ? 0x80008000u : 0u;
      } else {
        stage[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < KT) {
      stage_key = key_of(tile, tid);
      stage_sc = (FP8 && stage_key >= 0) ? fabsf(p.kscale[stage_key]) : 1.f;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int c = tid + 256 * u;
      const int kr = c / CH_PER_ROW, part = c % CH_PER_ROW;
      if constexpr (FP8) {
        // 16 e4m3 codes -> 16 bf16 (exact); fold a negative scale's sign in.
        const uint32_t f = stage_flip[u];
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          lo[2 * e] = fp8x2_to_bf16x2<false>(stage[u][e]) ^ f;
          lo[2 * e + 1] = fp8x2_to_bf16x2<true>(stage[u][e]) ^ f;
          hi[2 * e] = fp8x2_to_bf16x2<false>(stage[u][2 + e]) ^ f;
          hi[2 * e + 1] = fp8x2_to_bf16x2<true>(stage[u][2 + e]) ^ f;
        }
        uint16_t* dst = &ktile[buf][kr * kLdsStride + 16 * part];
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 8) = hi;
      } else {
        *reinterpret_cast<u32x4*>(&ktile[buf][kr * kLdsStride + 8 * part]) = stage[u];
      }
    }
    if (tid < KT) {
      ksc[buf][tid] = stage_sc;
      kkey[buf][tid] = stage_key;
    }
  };

  load_tile(tile0);
  store_tile(0);
  __syncthreads();

  for (int tile = tile0; tile < tile1; ++tile) {
    const int cur = (tile - tile0) & 1;
    const bool more = tile + 1 < tile1;
    if (more) load_tile(tile + 1);

    // ---- MFMA: acc[r][c] = q rows (r) x 16 keys (c), K = 128 in 4 steps
    f32x4 acc[RPW][CPW];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int col = (wc * CPW + c) * 16 + (lane & 15);
      const bf16x8* bsrc =
          reinterpret_cast<const bf16x8*>(&ktile[cur][col * kLdsStride + 32 * (lane >> 4)]);
      bf16x8 bfrag[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bfrag[ks] = bsrc[ks];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[r][ks], bfrag[ks], a4, 0, 0, 0);
        acc[r][c] = a4;
      }
    }

    // ---- epilogue: ReLU, times w, sum over the query's head slots
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      const int colt = (wc * CPW + c) * 16 + (lane & 15);
      const float kscale = FP8 ? ksc[cur][colt] : 1.f;
      const int key = kkey[cur][colt];
#pragma unroll
      for (int r0 = 0; r0 < RPW; r0 += TPQ) {
        float part = 0.f;
#pragma unroll
        for (int rr = 0; rr < TPQ; ++rr) {
#pragma unroll
          for (int i = 0; i < 4; ++i) part += wv[r0 + rr][i] * fmaxf(acc[r0 + rr][c][i], 0.f);
        }
        if constexpr (AP >= 8) part += __shfl_xor(part, 16, kWave);
        if constexpr (AP >= 16) part += __shfl_xor(part, 32, kWave);
        const int rt0 = wr * RPW + r0;
        const int qi = AP >= 16 ? (rt0 * 16) / AP : (rt0 * 16 + 4 * (lane >> 4)) / AP;
        const bool writer = AP >= 16 ? (lane < 16) : (AP == 8 ? ((lane & 16) == 0) : true);
        const int t = g * QW + qi;
        const int col = tile * KT + colt;
        if (writer && col < qn[qi] && key >= 0) {
          p.S[(size_t)t * p.S_ld + col] = part * kscale;
        }
      }
    }

    if (more) store_tile(cur ^ 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host side: pick an instantiation for the padded head count and batch.

static int pad_heads(int A) {
  int ap = 4;
  while (ap < A) ap <<= 1;
  return ap;
}

template <int AP, int WR, int RPW, int CPW, bool GATHER>
static hipError_t run_score(const LaunchCtx& cx, ScoreArgs a, bool fp8, const char* name) {
  constexpr int WC = 4 / WR;
  constexpr int QW = WR * RPW * 16 / AP;
  constexpr int KT = WC * CPW * 16;
  const long long max_cols = GATHER ? a.cand_ld : (long long)a.L;
  const int tiles = (int)((max_cols + KT - 1) / KT);
  int groups, splits;
  if (GATHER) {
    groups = a.T;
    // aim for ~2048 workgroups in total, at least 2 tiles each
    splits = (2048 + groups - 1) / groups;
    splits = splits > (tiles + 1) / 2 ? (tiles + 1) / 2 : splits;
  } else {
    groups = (a.T + QW - 1) / QW;
    splits = (2048 + groups - 1) / groups;
    splits = splits > (tiles + 3) / 4 ? (tiles + 3) / 4 : splits;
  }
  if (splits < 1) splits = 1;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  splits = (tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (splits < 1) splits = 1;
  a.ngroups = groups;
  dim3 grid = GATHER ? dim3(splits, groups) : dim3(groups, splits);
  if (fp8) return cx.launch(name, k_score<AP, WR, RPW, CPW, true, GATHER>, grid, dim3(256), 0, a);
  return cx.launch(name, k_score<AP, WR, RPW, CPW, false, GATHER>, grid, dim3(256), 0, a);
}

hipError_t launch_score_keys(const LaunchCtx& cx, ScoreArgs a, bool fp8) {
  if (a.T == 0) return hipSuccess;
  const int ap = pad_heads(a.A);
  const long long rows = (long long)a.T * ap;
  // Prefill-like batches (many queries whose prefixes grow) go heavy-first.
  a.reverse = 1;
  switch (ap) {
    case 4:
      if (rows <= 64) return run_score<4, 4, 1, 4, false>(cx, a, fp8, "score_keys");
      if (rows <= 128) return run_score<4, 4, 2, 4, false>(cx, a, fp8, "score_keys");
      return run_score<4, 4, 4, 4, false>(cx, a, fp8, "score_keys");
    case 8:
      if (rows <= 64) return run_score<8, 4, 1, 4, false>(cx, a, fp8, "score_keys");
      if (rows <= 128) return run_score<8, 4, 2, 4, false>(cx, a, fp8, "score_keys");
      return run_score<8, 4, 4, 4, false>(cx, a, fp8, "score_keys");
    case 16:
      if (rows <= 64) return run_score<16, 4, 1, 4, false>(cx, a, fp8, "score_keys");
      if (rows <= 128) return run_score<16, 4, 2, 4, false>(cx, a, fp8, "score_keys");
      return run_score<16, 4, 4, 4, false>(cx, a, fp8, "score_keys");
    case 32:
      if (rows <= 128) return run_score<32, 4, 2, 4, false>(cx, a, fp8, "score_keys");
      return run_score<32, 4, 4, 4, false>(cx, a, fp8, "score_keys");
    default:
      return run_score<64, 4, 4, 4, false>(cx, a, fp8, "score_keys");
  }
}

hipError_t launch_score_gather(const LaunchCtx& cx, ScoreArgs a, bool fp8) {
  if (a.T == 0) return hipSuccess;
  a.reverse = 0;
  a.heads = nullptr;
  a.A = a.H;
  const int ap = pad_heads(a.H);
  switch (ap) {
    case 4:
    case 8:
    case 16:
      return run_score<16, 1, 1, 1, true>(cx, a, fp8, "score_gather");
    case 32:
      return run_score<32, 1, 2, 1, true>(cx, a, fp8, "score_gather");
    default:
      return run_score<64, 1, 4, 1, true>(cx, a, fp8, "score_gather");
  }
}

}  // namespace misa
