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

// Key rows in LDS: 288 bytes apart (a 32-byte pad), and lane group j = l / 16
// of an MFMA operand reads 16-byte chunk 4 ks + j of its row in K step ks (the
// head dims are taken in that order by both operands, which leaves the dot
// product unchanged). A 16-byte LDS read serves each half-wave (32 lanes)
// together, and it is free of bank conflicts when the 32 lanes' addresses
// fall in distinct 16-byte slots modulo 512 bytes: a 288-byte row stride puts
// the 16 rows of a half-wave on the 16 even slots, and lane group j + 1 sits
// one slot after lane group j. (With 272-byte rows and each lane group
// reading 64 contiguous bytes, the SQ_LDS_BANK_CONFLICT counter read 16.9 M
// cycles per 16384-query causal prefill call, against none for a linear
// read; the counter is the reference for this rule.)
constexpr int kLdsStride = kHeadDim + 16;  // bf16 per key row in LDS

// ReLU of an MFMA result as one integer max on its bits: negative values (and
// -0.0) have the sign bit set and become +0.0. fmaxf would add a quieting step
// for signalling NaNs, which MFMA results on finite inputs never are.

// Row layout of the A operand. With AP <= 16 head slots and RPW a multiple of
// G = AP / 4, G row tiles form a "quad" of four queries: row r of tile k in the
// quad is query r / 4, head slot 4 k + r % 4, so the four MFMA result rows a
// lane holds are four heads of one query in every tile of the quad; the head
// sum needs no cross-lane step and every lane stores its own query's score.
// Otherwise rows are linear (row = tile * 16 + r, query row / AP): a query
// fills AP / 16 whole tiles, or a tile holds 16 / AP queries, and the sum adds
// the lane groups with one or two exchanges.
template <int AP, int RPW>
struct RowMap {
  static constexpr bool QUAD = AP <= 16 && RPW % (AP / 4) == 0;
  static constexpr int G = QUAD ? AP / 4 : (AP >= 16 ? AP / 16 : 1);  // row tiles per slot
  static constexpr int NQ = RPW / G;  // slots (quads or queries) per wave
  // (query index inside the workgroup, head slot) of row r of row tile rt
  static __device__ __forceinline__ void at(int rt, int r, int& qi, int& j) {
    if constexpr (QUAD) {
      qi = (rt / G) * 4 + (r >> 2);
      j = 4 * (rt % G) + (r & 3);
    } else {
      const int row = rt * 16 + r;
      qi = row / AP;
      j = row % AP;
    }
  }
  // query whose sums this lane holds for the slot that starts at row tile rt0
  static __device__ __forceinline__ int slot_query(int rt0, int lane) {
    int qi, j;
    at(rt0, 4 * (lane >> 4), qi, j);
    return qi;
  }
  // lanes that store a slot's sums (after the exchange the others hold copies)
  static __device__ __forceinline__ bool writer(int lane) {
    return QUAD || (AP >= 16 ? lane < 16 : (lane & 16) == 0);
  }
  static __device__ __forceinline__ float finish(float part) {
    if constexpr (!QUAD) {
      if constexpr (AP >= 8) part += __shfl_xor(part, 16, kWave);
      if constexpr (AP >= 16) part += __shfl_xor(part, 32, kWave);
    }
    return part;
  }
};

// Prefill-shaped batches: 256 rows per workgroup (WR row-wave groups of RPW
// tiles), key tiles of KT keys staged through LDS and shared by the waves.
// Scores go to S[t, col] for every col below the tile end (a key past the
// query's visible length gets an unused value inside the padded row; rows of
// lanes without a query go to the dump row S[T]), so the epilogue has no
// branch. RMM: also the per-split {min, max} score key of each query.
template <int AP, int WR, int RPW, int CPW, bool FP8, bool RMM>
__global__ __launch_bounds__(256) void k_score(ScoreArgs p) {
  using RM = RowMap<AP, RPW>;
  // key tiles in flight per workgroup (fewer when the row tiles use many registers)
  constexpr int R = (RPW >= 4 && !FP8) ? 2 : 4;
  constexpr int WC = 4 / WR;
  constexpr int ROWS = WR * RPW * 16;
  constexpr int QW = ROWS / AP;                     // queries per workgroup
  constexpr int KT = WC * CPW * 16;                 // keys per LDS tile
  constexpr int NQ = RM::NQ;                        // quads / queries per wave
  constexpr int CH_PER_ROW = FP8 ? 8 : 16;          // 16-byte global chunks per key row
  constexpr int CHUNKS = KT * CH_PER_ROW / 256;     // chunks per thread per tile
  static_assert(AP >= 4 && (AP & (AP - 1)) == 0, "AP must be a power of two >= 4");
  static_assert(ROWS % AP == 0 && QW >= 1, "row tiles must hold whole queries");
  static_assert(RPW % RM::G == 0, "a wave must hold whole quads or queries");
  static_assert(CHUNKS >= 1 && KT * CH_PER_ROW % 256 == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint16_t ktile[2][KT * kLdsStride];
  __shared__ float ksc[2][KT];
  __shared__ int qn[QW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC;
  const int g = p.reverse ? p.ngroups - 1 - (int)blockIdx.x : (int)blockIdx.x;
  const int split = (int)blockIdx.y;

  if (p.zero) {  // every workgroup clears its share
    const long long nthreads = 256ll * gridDim.x * gridDim.y;
    for (long long i = ((long long)blockIdx.y * gridDim.x + blockIdx.x) * 256 + tid; i < p.zero_n; i += nthreads)
      p.zero[i] = 0u;
  }
  if (tid < QW) {
    const int t = g * QW + tid;
    qn[tid] = t < p.T ? visible_len(p.pos[t], p.L) : 0;
  }
  __syncthreads();
  int nmax = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) nmax = qn[i] > nmax ? qn[i] : nmax;
  const int ntiles = (nmax + KT - 1) / KT;
  const int tile0 = split * p.tiles_per_split;
  const int tile1 = min(ntiles, tile0 + p.tiles_per_split);
  if (tile0 >= tile1) {  // uniform over the workgroup
    if (RMM && tid < QW && g * QW + tid < p.T) {
      p.rmm[((size_t)split * p.T + g * QW + tid) * 2] = 0xffffffffu;  // empty range
      p.rmm[((size_t)split * p.T + g * QW + tid) * 2 + 1] = 0u;
    }
    return;
  }

  // ---- staging of key tiles: global -> registers (R tiles in flight) -> LDS
  u32x4 stage[R][CHUNKS];
  float stage_sc[R];

  // Key tiles through a buffer resource over the key rows (raw buffer, the
  // third descriptor word of the gfx9 family): a tile's rows are contiguous, so
  // chunk c of tile t lies at byte t KT (row bytes) + 16 c. The whole offset
  // is the per-lane one, which the hardware checks against the buffer's size
  // (a scalar offset would not be checked): the rows of a last, partial tile
  // past the keys read as zeros (never stored) and touch no memory. L <= 2^23
  // keys keeps every offset below 2^32.
  constexpr int kRowBytes = CH_PER_ROW * 16;
  const long long kbytes = (long long)p.L * kRowBytes;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.K), (short)0, (int)(uint32_t)(kbytes < 0xffffffffll ? kbytes : 0xffffffffll), 0x00020000);
  auto load_tile = [&](int tile, int rr) {
    const uint32_t toff = (uint32_t)tile * (uint32_t)(KT * kRowBytes);
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u)
      stage[rr][u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(toff + 16u * (tid + 256 * u)), 0, 0));
    if (FP8 && tid < KT) stage_sc[rr] = p.kscale[min(tile * KT + tid, p.L - 1)];
  };

  auto store_tile = [&](int buf, int rr) {
#pragma unroll
    for (int u = 0; u < CHUNKS; ++u) {
      const int c = tid + 256 * u;
      const int kr = c / CH_PER_ROW, part = c % CH_PER_ROW;
      if constexpr (FP8) {
        // 16 e4m3 codes -> 16 bf16 (exact)
        u32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          lo[2 * e] = fp8x2_to_bf16x2<false>(stage[rr][u][e]);
          lo[2 * e + 1] = fp8x2_to_bf16x2<true>(stage[rr][u][e]);
          hi[2 * e] = fp8x2_to_bf16x2<false>(stage[rr][u][2 + e]);
          hi[2 * e + 1] = fp8x2_to_bf16x2<true>(stage[rr][u][2 + e]);
        }
        uint16_t* dst = &ktile[buf][kr * kLdsStride + 16 * part];
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 8) = hi;
      } else {
        *reinterpret_cast<u32x4*>(&ktile[buf][kr * kLdsStride + 8 * part]) = stage[rr][u];
      }
    }
    if (FP8 && tid < KT) ksc[buf][tid] = stage_sc[rr];
  };

  // ---- A operand (q rows of the scored heads) and epilogue weights, kept in
  // registers; issued before the key stream.
  bf16x8 afrag[RPW][4];
  float wv[RPW][4];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rt = wr * RPW + r;
    {
      int qi, j;
      RM::at(rt, lane & 15, qi, j);
      const int t = g * QW + qi;
      if (t < p.T && j < p.A) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(
            reinterpret_cast<const uint16_t*>(p.q) + ((size_t)t * p.H + j) * kHeadDim + 8 * (lane >> 4));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) afrag[r][ks] = src[4 * ks];  // dims 32 ks + 8 (lane / 16)
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) afrag[r][ks] = bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int qi, j;
      RM::at(rt, 4 * (lane >> 4) + i, qi, j);
      const int t = g * QW + qi;
      wv[r][i] = (t < p.T && j < p.A) ? p.w[(size_t)t * p.H + j] : 0.f;
    }
  }

#pragma unroll
  for (int rr = 0; rr < R; ++rr)
    if (tile0 + rr < tile1) load_tile(tile0 + rr, rr);

  // per quad (or query) of this lane: visible length, output row, score range
  int q_n[NQ];
  float* q_row[NQ];
  float smin[NQ], smax[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const int qi = RM::slot_query(wr * RPW + s * RM::G, lane);
    const int t = g * QW + qi;
    q_n[s] = qn[qi];
    q_row[s] = p.S + (size_t)(RM::writer(lane) && t < p.T ? t : p.T) * p.S_ld;
    smin[s] = __builtin_huge_valf();
    smax[s] = -__builtin_huge_valf();
  }

  for (int tbase = tile0; tbase < tile1; tbase += R) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const int tile = tbase + rr;
      if (tile >= tile1) break;  // uniform
      const int cur = (tile - tile0) & 1;
      store_tile(cur, rr);
      __syncthreads();
      if (tile + R < tile1) load_tile(tile + R, rr);

#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        // ---- MFMA: acc[r] = q rows (r) x 16 keys, K = 128 in 4 steps
        const int colt = (wc * CPW + c) * 16 + (lane & 15);
        const bf16x8* bsrc =
            reinterpret_cast<const bf16x8*>(&ktile[cur][colt * kLdsStride + 8 * (lane >> 4)]);
        bf16x8 bfrag[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bfrag[ks] = bsrc[4 * ks];  // the A operand's dims
        f32x4 acc[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[r][ks], bfrag[ks], a4, 0, 0, 0);
          acc[r] = a4;
        }
        // ---- epilogue: ReLU, times w, sum over the query's head slots, times |scale|
        float kscale = 1.f;
        if constexpr (FP8) {
          kscale = ksc[cur][colt];
          // a negative scale flips the key's sign inside the ReLU (rare: uniform branch)
          if (wave_ballot(kscale < 0.f)) {
            const float sgn = kscale < 0.f ? -1.f : 1.f;
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[r][i] *= sgn;
            kscale = fabsf(kscale);
          }
        }
        const int col = tile * KT + colt;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
          float part = 0.f;
#pragma unroll
          for (int k = 0; k < RM::G; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) part += wv[s * RM::G + k][i] * relu(acc[s * RM::G + k][i]);
          const float v = RM::finish(part) * kscale;
          q_row[s][col] = v;
          if constexpr (RMM) {
            const bool vis = col < q_n[s];
            smin[s] = fminf(smin[s], vis ? v : __builtin_huge_valf());
            smax[s] = fmaxf(smax[s], vis ? v : -__builtin_huge_valf());
          }
        }
      }
    }
  }

  if constexpr (RMM) {
    // lanes that share a query sit in one 16-lane group: reduce there
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      float lo = smin[s], hi = smax[s];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
      }
      const int t = g * QW + RM::slot_query(wr * RPW + s * RM::G, lane);
      if (RM::writer(lane) && (lane & 15) == 0 && t < p.T) {
        // an empty range (no visible key here) stays {max key, 0}
        const bool any = lo <= hi;
        p.rmm[((size_t)split * p.T + t) * 2] = any ? score_key(lo) : 0xffffffffu;
        p.rmm[((size_t)split * p.T + t) * 2 + 1] = any ? score_key(hi) : 0u;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-shaped batches: every (query, head-slot) row of the workgroup fits in
// one wave (RPW row tiles), so the waves split the keys instead of the rows and
// each wave loads its own B fragments straight from global memory: no LDS, no
// barriers, D groups of 16 keys in flight per wave. Lane l covers key
// (l mod 16) of a group and head dims [32*(l/16), 32*(l/16) + 32).
//
// QF8 (fp8 queries and fp8 keys): one v_mfma_scale_f32_16x16x128_f8f6f4 per
// row tile and key group takes all 128 dims (both block scales 2^0), with the
// E4M3 codes of q and of the key as its operands, each lane holding the same
// 32 dims of its row and of its key; a row's per-(query, head) scale is
// positive-homogeneous through ReLU like the key's, so its sign is folded into
// the row's codes and |scale| into the row's weight.
template <int AP, int RPW, int WR, bool FP8, bool GATHER, bool QF8 = false>
__global__ __launch_bounds__(256) void k_score_direct(ScoreArgs p) {
  static_assert(!QF8 || FP8, "fp8 queries are scored against fp8 keys");
  constexpr int WC = 4 / WR;                        // key groups per tile (waves sharing rows)
  constexpr int ROWS = WR * RPW * 16;               // rows per workgroup
  constexpr int QW = ROWS / AP;                     // queries per workgroup
  using RM = RowMap<AP, RPW>;
  constexpr int NQ = RM::NQ;                        // quads / queries per wave
  constexpr int D = (RPW >= 8 && !FP8) ? 2 : 4;     // key groups in flight per wave
  constexpr int NV = FP8 ? 2 : 4;                   // 16-byte loads per lane per group
  constexpr int KT = 16 * WC;                       // keys per tile
  static_assert(WR == 1 || WR == 2 || WR == 4, "WR must divide the four waves");
  static_assert(AP >= 4 && (AP & (AP - 1)) == 0, "AP must be a power of two >= 4");
  static_assert(ROWS % AP == 0 && QW >= 1, "row tiles must hold whole queries");
  static_assert(RPW % RM::G == 0, "a wave must hold whole quads or queries");
  static_assert(WR == 1 || RPW * 16 % AP == 0, "row waves must hold whole queries");
  static_assert(!GATHER || QW == 1, "gather mode scores one query per workgroup");

  __shared__ int qn[QW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave / WC, wc = wave % WC;  // row group and key group of this wave
  // Key ranges: a 1-D grid of ngroups x nsplit workgroups. Workgroup i runs on
  // XCD i mod 8, each XCD with its own L2: when nsplit is a multiple of 8, the
  // query groups of one key split get consecutive slots of one XCD, so that
  // the split's keys come from HBM once and the other groups read them from
  // that L2 (with the groups of a split on different XCDs, the 256-row
  // batch of 32 queries over 32K keys fetched 4x its keys).
  int g, split;
  if constexpr (GATHER) {
    g = (int)blockIdx.y;
    split = (int)blockIdx.x;
  } else {
    const int lin = (int)blockIdx.x, G = p.ngroups;
    if (G > 1 && p.nsplit % 8 == 0) {
      const int slot = lin >> 3;
      split = (lin & 7) + 8 * (slot / G);
      g = slot % G;
    } else {
      split = lin / G;
      g = lin % G;
    }
    if (p.reverse) g = G - 1 - g;
  }
  // The query lengths' inputs are the first reads (from always-valid
  // addresses): the later wait for them then waits for nothing else.
  const int tqc = min(g * QW + (tid < QW ? tid : 0), p.T - 1);
  const int pos_raw = p.pos[tqc];
  const int* ncnt = GATHER ? (p.blocks ? p.nblocks : p.ncand) : p.pos;
  const int n_raw = ncnt[tqc];  // listed blocks or candidates (gather modes)
  int last_raw = 0;             // block lists: the last listed block (requested below)

  // With several key waves per row group (WC > 1) the workgroup's q rows and
  // weights are loaded once into LDS (one pad word per row keeps the 16-byte
  // row reads conflict-free) instead of once per wave.
  constexpr bool STAGE = WC > 1;
  constexpr int RW = QF8 ? kHeadDim / 16 : kHeadDim / 8;  // 16-byte words per q row
  constexpr int QSTR = RW + 1;
  constexpr int SQ = STAGE ? (ROWS * RW + 255) / 256 : 0;  // 16-byte q words per thread (rounded up)
  __shared__ u32x4 qsh[STAGE ? ROWS * QSTR : 1];
  __shared__ float wsh[STAGE ? ROWS : 1];
  u32x4 qstage[SQ > 0 ? SQ : 1];
  float wstage = 0.f;
  const uint8_t* qbytes = reinterpret_cast<const uint8_t*>(p.q);
  // fp8 rows with their own scales: the sign goes into the codes, |scale| into the weight
  auto row_flip = [&](int t, int j) -> uint32_t {
    if constexpr (QF8) return (p.qscale && p.qscale[(size_t)t * p.H + j] < 0.f) ? 0x80808080u : 0u;
    else return 0u;
  };
  auto row_weight = [&](int t, int j) -> float {
    const float wt = p.w[(size_t)t * p.H + j];
    if constexpr (QF8) return p.qscale ? wt * fabsf(p.qscale[(size_t)t * p.H + j]) : wt;
    else return wt;
  };
  if constexpr (STAGE && !QF8) {
#pragma unroll
    for (int u = 0; u < SQ; ++u) {
      const int i = tid + 256 * u, row = i >> 4, v = i & 15;
      const int qi = row / AP, j = row % AP, t = g * QW + qi;
      qstage[u] = (t < p.T && j < p.A)
                      ? reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                                       ((size_t)t * p.H + j) * kHeadDim)[v]
                      : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < ROWS) {
      const int qi = tid / AP, j = tid % AP, t = g * QW + qi;
      wstage = (t < p.T && j < p.A) ? p.w[(size_t)t * p.H + j] : 0.f;
    }
  }
  if constexpr (STAGE && QF8) {
#pragma unroll
    for (int u = 0; u < SQ; ++u) {
      const int i = tid + 256 * u, row = i / RW, v = i % RW;
      const int qi = row / AP, j = row % AP, t = g * QW + qi;
      if (i < ROWS * RW && t < p.T && j < p.A) {
        u32x4 x = reinterpret_cast<const u32x4*>(qbytes + ((size_t)t * p.H + j) * RW * 16)[v];
        const uint32_t f = row_flip(t, j);
        x[0] ^= f;
        x[1] ^= f;
        x[2] ^= f;
        x[3] ^= f;
        qstage[u] = x;
      } else {
        qstage[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < ROWS) {
      const int qi = tid / AP, j = tid % AP, t = g * QW + qi;
      wstage = (t < p.T && j < p.A) ? row_weight(t, j) : 0.f;
    }
  }

  const int tile0 = split * p.tiles_per_split;
  const int qt0 = g * QW;
  const int kcol = lane & 15;
  const int slice = lane >> 4;

  // Every request reads from a valid address (a column past the end reads key
  // 0 and carries key -1, so it is never written): a load issued under a lane
  // mask beside a register fill for the other lanes would make the compiler
  // wait for it before it could request the next group.
  auto key_of = [&](int gi) -> int {
    const int col = (tile0 + gi) * KT + 16 * wc + kcol;
    if constexpr (GATHER) {
      // one load per group either way (no branch between the request and its use)
      const int cc = min(col, qn[0] - 1);  // qn[0] >= 1 whenever groups are loaded
      const int bsz = p.blocks ? p.B : 1;
      const int* src = p.blocks ? p.blocks + (size_t)qt0 * p.blocks_ld : p.cand + (size_t)qt0 * p.cand_ld;
      const int blk = cc / bsz;
      const int key = src[blk] * bsz + (cc - blk * bsz);
      return col < qn[0] ? key : -1;
    } else {
      return col < p.L ? col : -1;
    }
  };

  u32x4 kv[D][NV];
  float ksv[D];
  int keyv[D];
  auto load_key = [&](int s, int slot) {
    keyv[slot] = s;
    const int r = s >= 0 ? s : 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint8_t*>(p.K) + (size_t)r * (FP8 ? kHeadDim : 2 * kHeadDim) + slice * NV * 16);
#pragma unroll
    for (int v = 0; v < NV; ++v) kv[slot][v] = src[v];
    ksv[slot] = FP8 ? p.kscale[r] : 1.f;
  };
  auto load_group = [&](int gi, int slot) { load_key(key_of(gi), slot); };

  // Plain key ranges: the keys a split may touch are known from L alone, so the
  // first D groups are requested before the query lengths arrive (keys past a
  // query's visible length are masked below). All D are requested whether or
  // not the split has that many: a request under a uniform branch makes the
  // compiler's wait counting conservative for every later group.
  if constexpr (!GATHER) {
#pragma unroll
    for (int d = 0; d < D; ++d) load_group(d, d);
  }
  // Gather modes: the first D groups' candidate indices, and then their key
  // rows, are requested before the query's candidate count arrives, from
  // positions clamped to the row's capacity and keys clamped to [0, L) (always
  // valid rows); columns past the count are masked once it is known.
  if constexpr (GATHER) {
    const int bsz = p.blocks ? p.B : 1;
    const long long cap = p.blocks ? p.blocks_ld * (long long)p.B : p.cand_ld;
    const int* src = p.blocks ? p.blocks + (size_t)qt0 * p.blocks_ld : p.cand + (size_t)qt0 * p.cand_ld;
    int iraw[D], off[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int col = (tile0 + d) * KT + 16 * wc + kcol;
      const int cc = (int)min((long long)col, cap - 1);
      const int blk = cc / bsz;
      iraw[d] = src[blk];
      off[d] = cc - blk * bsz;
    }
    // block lists: the query's last listed block (for its candidate count),
    // requested here so that the count does not wait for the key rows
    const int* lsrc = p.blocks ? p.blocks + (size_t)qt0 * p.blocks_ld : p.pos;
    last_raw = lsrc[p.blocks ? min(max(n_raw - 1, 0), (int)p.blocks_ld - 1) : 0];
    int kraw[D];
#pragma unroll
    for (int d = 0; d < D; ++d) kraw[d] = min(max(iraw[d] * bsz + off[d], 0), p.L - 1);
#pragma unroll
    for (int d = 0; d < D; ++d) load_key(kraw[d], d);
  }

  if (p.zero) {  // every workgroup clears its share
    const long long nthreads = 256ll * gridDim.x * gridDim.y;
    for (long long i = ((long long)blockIdx.y * gridDim.x + blockIdx.x) * 256 + tid; i < p.zero_n; i += nthreads)
      p.zero[i] = 0u;
  }
  if (tid < QW) {
    const int t = g * QW + tid;
    int nn = 0;
    if (t < p.T) {
      if (GATHER && p.blocks) {
        // candidates = the visible keys of the listed blocks (ascending); only
        // the last listed block can be the query's partial last block
        const int nb = n_raw;
        if (nb > 0) {
          const int last = last_raw;
          const long long tail = (long long)visible_len(pos_raw, p.L) - (long long)last * p.B;
          nn = (nb - 1) * p.B + (int)(tail < p.B ? tail : p.B);
        }
        if (split == 0) p.ncand_out[t] = nn;
      } else {
        nn = GATHER ? n_raw : visible_len(pos_raw, p.L);
      }
    }
    qn[tid] = nn;
  }
  if constexpr (STAGE) {
#pragma unroll
    for (int u = 0; u < SQ; ++u) {
      const int i = tid + 256 * u;
      if (QF8 ? i < ROWS * RW : true) qsh[(i / RW) * QSTR + (i % RW)] = qstage[u];
    }
    if (tid < ROWS) wsh[tid] = wstage;
  }
  __syncthreads();
  int nmax = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) nmax = qn[i] > nmax ? qn[i] : nmax;
  const int ntiles = (nmax + KT - 1) / KT;
  const int tile1 = min(ntiles, tile0 + p.tiles_per_split);
  if (tile0 >= tile1) {  // uniform over the workgroup
    if (!GATHER && p.rmm && tid < QW && g * QW + tid < p.T) {
      p.rmm[((size_t)split * p.T + g * QW + tid) * 2] = 0xffffffffu;  // empty range
      p.rmm[((size_t)split * p.T + g * QW + tid) * 2 + 1] = 0u;
    }
    if constexpr (!GATHER) __builtin_amdgcn_s_waitcnt(0);  // early key requests land first
    return;
  }
  const int ngroups = tile1 - tile0;  // this wave's groups: one per tile, key offset 16*wc
  // ---- A operand (q rows of the scored heads) and epilogue weights, kept in
  // registers; issued before the key stream so the first MFMA waits on one
  // round trip only.
  // A operand per row tile: 4 x 8 bf16 (bf16 rows), or 32 fp8 codes (QF8)
  bf16x8 afrag[QF8 ? 1 : RPW][4];
  i32x8 afrag8[QF8 ? RPW : 1];
  float wv[RPW][4];
#pragma unroll
  for (int r = 0; r < RPW && STAGE; ++r) {
    // staged rows are in (query, slot) order: row qi * AP + j
    int qi, j;
    RM::at(wr * RPW + r, lane & 15, qi, j);
    if constexpr (QF8) {
      const u32x4 lo = qsh[(qi * AP + j) * QSTR + 2 * slice], hi = qsh[(qi * AP + j) * QSTR + 2 * slice + 1];
      afrag8[r] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        afrag[r][ks] = __builtin_bit_cast(bf16x8, qsh[(qi * AP + j) * QSTR + 4 * slice + ks]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      RM::at(wr * RPW + r, 4 * slice + i, qi, j);
      wv[r][i] = wsh[qi * AP + j];
    }
  }
#pragma unroll
  for (int r = 0; r < RPW && !STAGE; ++r) {
    {
      int qi, j;
      RM::at(wr * RPW + r, lane & 15, qi, j);
      const int t = g * QW + qi;
      if constexpr (QF8) {
        if (t < p.T && j < p.A) {
          const u32x4* src = reinterpret_cast<const u32x4*>(qbytes + ((size_t)t * p.H + j) * kHeadDim + 32 * slice);
          const u32x4 lo = src[0], hi = src[1];
          const int f = (int)row_flip(t, j);
          afrag8[r] = i32x8{(int)lo[0] ^ f, (int)lo[1] ^ f, (int)lo[2] ^ f, (int)lo[3] ^ f,
                            (int)hi[0] ^ f, (int)hi[1] ^ f, (int)hi[2] ^ f, (int)hi[3] ^ f};
        } else {
          afrag8[r] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
      } else {
        if (t < p.T && j < p.A) {
          const bf16x8* src = reinterpret_cast<const bf16x8*>(
              reinterpret_cast<const uint16_t*>(p.q) + ((size_t)t * p.H + j) * kHeadDim + 32 * slice);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) afrag[r][ks] = src[ks];
        } else {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) afrag[r][ks] = bf16x8{};
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int qi, j;
      RM::at(wr * RPW + r, 4 * slice + i, qi, j);
      const int t = g * QW + qi;
      if constexpr (QF8) wv[r][i] = (t < p.T && j < p.A) ? row_weight(t, j) : 0.f;
      else wv[r][i] = (t < p.T && j < p.A) ? p.w[(size_t)t * p.H + j] : 0.f;
    }
  }

  if constexpr (GATHER) {
    // the first D groups were requested before the count: mask their columns
#pragma unroll
    for (int d = 0; d < D; ++d)
      if ((tile0 + d) * KT + 16 * wc + kcol >= qn[0]) keyv[d] = -1;
  }

  // stores need no mask: a key past the query's candidates or visible length
  // lands inside the padded row, and lanes without a query (or holding copies)
  // write to the dump row S[T]
  int q_n[NQ];
  float* q_row[NQ];
  float smin[NQ], smax[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const int qi = RM::slot_query(wr * RPW + s * RM::G, lane);
    const int t = g * QW + qi;
    q_n[s] = qn[qi];
    q_row[s] = p.S + (size_t)(RM::writer(lane) && t < p.T ? t : p.T) * p.S_ld;
    smin[s] = __builtin_huge_valf();
    smax[s] = -__builtin_huge_valf();
  }

  for (int gb = 0; gb < ngroups; gb += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int gi = gb + d;
      if (gi >= ngroups) break;  // uniform
      // B fragments for the four K steps (fp8 codes widen exactly to bf16), or
      // the key's 32 fp8 codes as they are (QF8)
      bf16x8 bfrag[QF8 ? 1 : 4];
      i32x8 bfrag8;
      if constexpr (QF8) {
        bfrag8 = i32x8{(int)kv[d][0][0], (int)kv[d][0][1], (int)kv[d][0][2], (int)kv[d][0][3],
                       (int)kv[d][1][0], (int)kv[d][1][1], (int)kv[d][1][2], (int)kv[d][1][3]};
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if constexpr (FP8) {
            const uint32_t w0 = kv[d][ks >> 1][(ks & 1) * 2], w1 = kv[d][ks >> 1][(ks & 1) * 2 + 1];
            u32x4 b;
            b[0] = fp8x2_to_bf16x2<false>(w0);
            b[1] = fp8x2_to_bf16x2<true>(w0);
            b[2] = fp8x2_to_bf16x2<false>(w1);
            b[3] = fp8x2_to_bf16x2<true>(w1);
            bfrag[ks] = __builtin_bit_cast(bf16x8, b);
          } else {
            bfrag[ks] = __builtin_bit_cast(bf16x8, kv[d][ks]);
          }
        }
      }
      float kscale = ksv[d];
      const int key = keyv[d];
      const int col = (tile0 + gi) * KT + 16 * wc + kcol;
      if constexpr (GATHER)  // block-list candidates are recorded for the selection
        if (p.blocks && slice == 0 && key >= 0) p.cand_out[(size_t)qt0 * p.cand_ld + col] = key;
      if (gi + D < ngroups) load_group(gi + D, d);

      f32x4 acc[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (QF8) {
          // all 128 dims at once; E8M0 block scales 127 = 2^0 for both operands
          a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afrag8[r], bfrag8, a4, 0, 0, 0, 127, 0, 127);
        } else {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[r][ks], bfrag[ks], a4, 0, 0, 0);
        }
        acc[r] = a4;
      }
      if constexpr (FP8) {
        // a negative scale flips the key's sign inside the ReLU (rare: uniform branch)
        if (wave_ballot(kscale < 0.f)) {
          const float sgn = kscale < 0.f ? -1.f : 1.f;
#pragma unroll
          for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][i] *= sgn;
          kscale = fabsf(kscale);
        }
      }
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < RM::G; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) part += wv[s * RM::G + k][i] * relu(acc[s * RM::G + k][i]);
        const float v = RM::finish(part) * kscale;
        q_row[s][col] = v;
        const bool vis = col < q_n[s];  // (a gathered column past the candidates has key -1)
        smin[s] = fminf(smin[s], vis ? v : __builtin_huge_valf());
        smax[s] = fmaxf(smax[s], vis ? v : -__builtin_huge_valf());
      }
    }
  }

  if (ngroups < D) __builtin_amdgcn_s_waitcnt(0);  // unused requests land before the wave ends
  if (!GATHER && p.rmm) {
    // per query: lanes of one wave reduce, then the key groups meet in LDS
    __shared__ float rlo[WC][QW], rhi[WC][QW];
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      float lo = smin[s], hi = smax[s];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
      }
      const int qi = RM::slot_query(wr * RPW + s * RM::G, lane);
      if (RM::writer(lane) && (lane & 15) == 0) {
        rlo[wc][qi] = lo;
        rhi[wc][qi] = hi;
      }
    }
    __syncthreads();
    if (tid < QW && g * QW + tid < p.T) {
      float lo = rlo[0][tid], hi = rhi[0][tid];
#pragma unroll
      for (int w2 = 1; w2 < WC; ++w2) {
        lo = fminf(lo, rlo[w2][tid]);
        hi = fmaxf(hi, rhi[w2][tid]);
      }
      const bool any = lo <= hi;
      p.rmm[((size_t)split * p.T + g * QW + tid) * 2] = any ? score_key(lo) : 0xffffffffu;
      p.rmm[((size_t)split * p.T + g * QW + tid) * 2 + 1] = any ? score_key(hi) : 0u;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: pick an instantiation for the padded head count and batch.

int score_max_splits() { return 2048; }

static int pad_heads(int A) {
  int ap = 4;
  while (ap < A) ap <<= 1;
  return ap;
}

template <int AP, int WR, int RPW, int CPW>
static hipError_t run_score(const LaunchCtx& cx, ScoreArgs a, bool fp8, const char* name,
                            int* nsplit_out) {
  constexpr int WC = 4 / WR;
  constexpr int QW = WR * RPW * 16 / AP;
  constexpr int KT = WC * CPW * 16;
  const int tiles = (int)(((long long)a.L + KT - 1) / KT);
  // about 4096 workgroups: causal batches give query groups very different tile
  // counts, and splits of ~16 tiles even out what each compute unit is handed
  // (16384 x 16384 causal: 258 us against 273 us with ~2048 workgroups)
  const int target = a.target_wgs > 0 ? a.target_wgs : 4096;
  const int groups = (a.T + QW - 1) / QW;
  const int min_tiles = a.target_wgs > 0 ? 1 : 4;
  int splits = (target + groups - 1) / groups;
  splits = splits > (tiles + min_tiles - 1) / min_tiles ? (tiles + min_tiles - 1) / min_tiles : splits;
  if (splits < 1) splits = 1;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  splits = (tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (splits < 1) splits = 1;
  a.ngroups = groups;
  a.nsplit = splits;
  if (nsplit_out) *nsplit_out = splits;
  const dim3 grid(groups, splits);
#define MISA_SCORE_LAUNCH(F8, RM) cx.launch(name, k_score<AP, WR, RPW, CPW, F8, RM>, grid, dim3(256), 0, a)
  if (a.rmm) return fp8 ? MISA_SCORE_LAUNCH(true, true) : MISA_SCORE_LAUNCH(false, true);
  return fp8 ? MISA_SCORE_LAUNCH(true, false) : MISA_SCORE_LAUNCH(false, false);
#undef MISA_SCORE_LAUNCH
}

template <int AP, int RPW, int WR, bool GATHER>
static hipError_t run_direct(const LaunchCtx& cx, ScoreArgs a, bool fp8, const char* name,
                             int* nsplit_out) {
  constexpr int QW = WR * RPW * 16 / AP;
  constexpr int KT = 16 * (4 / WR);
  const long long max_cols = GATHER ? (long long)a.cand_max : (long long)a.L;
  const int tiles = (int)((max_cols + KT - 1) / KT);
  const int groups = GATHER ? a.T : (a.T + QW - 1) / QW;
  const int target = a.target_wgs > 0 ? a.target_wgs : 512;
  int splits = (target + groups - 1) / groups;
  const int min_tiles = a.target_wgs > 0 ? 1 : 4;  // four key groups per wave by default
  if (splits > (tiles + min_tiles - 1) / min_tiles) splits = (tiles + min_tiles - 1) / min_tiles;
  if (splits < 1) splits = 1;
  a.tiles_per_split = (tiles + splits - 1) / splits;
  splits = (tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  if (splits < 1) splits = 1;
  a.ngroups = groups;
  a.nsplit = splits;
  if (nsplit_out) *nsplit_out = splits;
  const dim3 grid = GATHER ? dim3(splits, groups) : dim3(groups * splits);
  if (a.q_fp8) {
    if (!fp8) return hipErrorInvalidValue;  // fp8 queries are scored against fp8 keys
    return cx.launch(name, k_score_direct<AP, RPW, WR, true, GATHER, true>, grid, dim3(256), 0, a);
  }
  if (fp8) return cx.launch(name, k_score_direct<AP, RPW, WR, true, GATHER>, grid, dim3(256), 0, a);
  return cx.launch(name, k_score_direct<AP, RPW, WR, false, GATHER>, grid, dim3(256), 0, a);
}

// Decode batches: up to four row tiles (64 rows) per wave, the four waves
// splitting the keys; batches of more than 64 routed rows are cut into query
// groups of 64 rows (C2-like batches, 256 rows: 9.3 us per launch against
// 10.5 us with all rows in one workgroup, which loaded 64 KiB of q rows to score
// 128 keys). Returns false when the batch is too large.
template <int AP>
static bool direct_keys(const LaunchCtx& cx, ScoreArgs a, bool fp8, long long rows, int* nsplit_out,
                        hipError_t* err) {
  const char* nm = "score_keys";
  if (AP <= 16 && rows <= 16) {
    *err = run_direct<AP <= 16 ? AP : 16, 1, 1, false>(cx, a, fp8, nm, nsplit_out);
  } else if (AP <= 32 && rows <= 32) {
    *err = run_direct<AP <= 32 ? AP : 32, 2, 1, false>(cx, a, fp8, nm, nsplit_out);
  } else if (rows <= 256) {
    *err = run_direct<AP, 4, 1, false>(cx, a, fp8, nm, nsplit_out);
  } else {
    return false;
  }
  return true;
}

bool score_fp8q_supported(int T, int A) { return A >= 1 && A <= kMaxHeads && (long long)T * pad_heads(A) <= 256; }

hipError_t launch_score_keys(const LaunchCtx& cx, ScoreArgs a, bool fp8, int* nsplit_out) {
  if (a.T == 0) return hipSuccess;
  if (a.S_ld % 128 != 0 || a.S_ld < a.L) return hipErrorInvalidValue;  // whole tiles per row
  const int ap = pad_heads(a.A);
  const long long rows = (long long)a.T * ap;
  // Prefill-like batches (many queries whose prefixes grow) go heavy-first.
  a.reverse = 1;
  const char* nm = "score_keys";
  hipError_t err = hipSuccess;
  bool done = false;
  switch (ap) {
    case 4: done = direct_keys<4>(cx, a, fp8, rows, nsplit_out, &err); break;
    case 8: done = direct_keys<8>(cx, a, fp8, rows, nsplit_out, &err); break;
    case 16: done = direct_keys<16>(cx, a, fp8, rows, nsplit_out, &err); break;
    case 32: done = direct_keys<32>(cx, a, fp8, rows, nsplit_out, &err); break;
    default: done = direct_keys<64>(cx, a, fp8, rows, nsplit_out, &err); break;
  }
  if (done) return err;
  if (a.q_fp8) return hipErrorInvalidValue;  // fp8 queries: decode-shaped batches only
  // larger batches (prefill): LDS-staged key tiles shared by 256 rows
  switch (ap) {
    case 4: return run_score<4, 4, 4, 8>(cx, a, fp8, nm, nsplit_out);
    case 8: return run_score<8, 4, 4, 8>(cx, a, fp8, nm, nsplit_out);
    case 16: return run_score<16, 4, 4, 8>(cx, a, fp8, nm, nsplit_out);
    case 32: return run_score<32, 4, 4, 8>(cx, a, fp8, nm, nsplit_out);
    default: return run_score<64, 4, 4, 8>(cx, a, fp8, nm, nsplit_out);
  }
}

hipError_t launch_score_gather(const LaunchCtx& cx, ScoreArgs a, bool fp8) {
  if (a.T == 0) return hipSuccess;
  if (a.S_ld % 128 != 0 || a.S_ld < a.cand_max) return hipErrorInvalidValue;  // whole tiles per row
  a.reverse = 0;
  a.rmm = nullptr;
  a.A = a.H;
  const int ap = pad_heads(a.H);
  const char* nm = "score_gather";
  switch (ap) {
    case 4:
    case 8:
    case 16:
      return run_direct<16, 1, 1, true>(cx, a, fp8, nm, nullptr);
    case 32:
      return run_direct<32, 2, 1, true>(cx, a, fp8, nm, nullptr);
    default:
      return run_direct<64, 4, 1, true>(cx, a, fp8, nm, nullptr);
  }
}

}  // namespace misa
