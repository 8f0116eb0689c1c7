// Router side of the indexer: block statistics of the keys and the per-head
// routing score (MISA technical summary, "Metodologia: MISA": the router pools
// the prefix into M = ceil(L/B) blocks of averaged keys, scores every head
// against them and keeps the best h heads; HISA write-up, section 3 Stage 1
// uses the same block representatives for its block filter).
//
// Precision: block sums are accumulated in float64 (bf16 keys, and fp8 codes
// times fp32 scales, add up exactly at these sizes) and the head scores are
// float64 dot products, so the routed head set agrees with an exact
// evaluation except where two heads tie to float64 rounding.
#include "device_common.h"
#include "launch.h"

namespace misa {

// -------------------------------------------------------------------------
// One 16-byte slice of key s, dims [DPT*dg, DPT*dg + DPT) (DPT = 8 bf16 or 16
// fp8 codes), widened to float64; fp8 codes are multiplied by the key's scale,
// which is exact in float64.
template <bool FP8>
struct KeySlice {
  static constexpr int DPT = FP8 ? 16 : 8;
  static __device__ __forceinline__ u32x4 load(const void* K, int s, int dg) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(K) + (size_t)s * kHeadDim * (FP8 ? 1 : 2);
    return *reinterpret_cast<const u32x4*>(base + 16 * dg);
  }
  static __device__ __forceinline__ void widen(u32x4 v, double sc, double* out) {
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[2 * j] = (double)bf16_bits_to_f32(v[j] & 0xffffu);
        out[2 * j + 1] = (double)bf16_bits_to_f32(v[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a, b, c, d;
        fp8x2_to_f32<false>(v[j], a, b);
        fp8x2_to_f32<true>(v[j], c, d);
        out[4 * j + 0] = (double)a * sc;
        out[4 * j + 1] = (double)b * sc;
        out[4 * j + 2] = (double)c * sc;
        out[4 * j + 3] = (double)d * sc;
      }
    }
  }
};

// Sum of key rows [s0, s1) in float64, one workgroup of NTH threads;
// thread (rl, dg) takes rows rl, rl + RL, ... and one 16-byte slice of dims. A
// whole 128-key block's rows of a thread (U slices) are loaded
// before any is added, so the loads overlap. Column sums of RR row groups
// (FOLD: the upper half of the RL row groups first added into the lower half)
// are left in red for the caller to add up: value e of slice dg of row group rl
// sits at red[rl * kRedStride + e * NG + dg] (so one store instruction of a wave
// covers contiguous doubles, and the padded row stride puts alternate row
// groups on the other half of the LDS banks); column c of that layout holds
// dim (c % NG) * DPT + c / NG.
// MAX: per-dimension maximum instead of the sum (max-pooled representatives;
// exact, the widened values being exact in float64).
constexpr int kRedStride = kHeadDim + 8;  // doubles per row group of the reduction buffer
// Four waves per block, so that a workgroup whose rows arrive last adds them
// up on all four SIMDs of its CU; the reduction buffer is folded once (FOLD)
// to stay at 17 KiB, so that every workgroup of a 128K-key problem (1024
// blocks plus the query tails) is resident at once.
constexpr int kSumThreads = 256;

template <bool FP8, bool MAX = false, int NTH = kSumThreads, bool FOLD = false>
struct RowSum {
  static constexpr int DPT = KeySlice<FP8>::DPT;
  static constexpr int NG = kHeadDim / DPT;  // slices per key
  static constexpr int RL = NTH / NG;        // row groups
  static constexpr int RR = FOLD ? RL / 2 : RL;  // row groups left in the reduction buffer
  static constexpr int U = 128 / RL;         // rows per thread per pass (128 keys per pass)
  static __device__ __forceinline__ int dim_of(int c) { return (c % NG) * DPT + c / NG; }
  static __device__ __forceinline__ void run(const void* K, const float* kscale, int s0, int s1, double* red) {
    const int tid = threadIdx.x, dg = tid % NG, rl = tid / NG;
    double acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = MAX ? -__builtin_huge_val() : 0.0;
    for (int sb = s0 + rl; sb < s1; sb += RL * U) {
      // every row's loads are issued before any is used, from clamped rows (a
      // load inside a condition would be waited for inside it); rows past s1
      // are masked afterwards
      u32x4 v[U];
      float scr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = min(sb + RL * u, s1 - 1);
        v[u] = KeySlice<FP8>::load(K, s, dg);
        scr[u] = FP8 ? kscale[s] : 1.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = sb + RL * u < s1;
        if (!ok) v[u] = u32x4{0u, 0u, 0u, 0u};
        const double sc = ok ? (double)scr[u] : 0.0;
        double x[DPT];
        KeySlice<FP8>::widen(v[u], sc, x);
        if constexpr (MAX) {
          if (ok) {
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[e] = x[e] > acc[e] ? x[e] : acc[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[e] += x[e];
        }
      }
    }
    if constexpr (FOLD) {
      // the upper half of the row groups hands its partials to the lower half
      if (rl >= RR) {
#pragma unroll
        for (int e = 0; e < DPT; ++e) red[(rl - RR) * kRedStride + e * NG + dg] = acc[e];
      }
      __syncthreads();
      if (rl < RR) {
#pragma unroll
        for (int e = 0; e < DPT; ++e) {
          const double y = red[rl * kRedStride + e * NG + dg];
          if constexpr (MAX) acc[e] = y > acc[e] ? y : acc[e];
          else acc[e] += y;
        }
      }
      __syncthreads();
      if (rl < RR) {
#pragma unroll
        for (int e = 0; e < DPT; ++e) red[rl * kRedStride + e * NG + dg] = acc[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPT; ++e) red[rl * kRedStride + e * NG + dg] = acc[e];
    }
    __syncthreads();
  }
};

// Workgroups [0, ntail): tsum[t,:] = sum of the keys of query t's last block
// [(M_t-1)*B, n_t), possibly partial; zero when the query sees no key (they
// come first so that the tails, which often all read the same last block,
// start before the long tail of the grid). Workgroup ntail + i: block
// b = b_base + i in [0, M): ksum[b,:] = sum of the keys of block
// b = [b*B, min((b+1)*B, L)) in float64, and (optional) kbar = ksum / count
// rounded once to float32. MAX: the
// per-dimension maxima of the same keys instead of their sums (max-pooled
// block representatives; no kbar or kb16), zero for a query with no key.
template <bool FP8, bool MAX>
__global__ __launch_bounds__(kSumThreads) void k_block_sums(const void* K, const float* kscale, int L,
                                                    int B, int M, double* ksum, float* kbar,
                                                    uint16_t* kb16, const int32_t* pos, double* tsum,
                                                    int ntail, int b_base) {
  using RS = RowSum<FP8, MAX, kSumThreads, true>;
  constexpr int RL = RS::RR;
  __shared__ double red[RL * kRedStride];
  const int wg = (int)blockIdx.x;
  const bool is_tail = wg < ntail;
  const int b = is_tail ? -1 : wg - ntail + b_base;
  int s0, s1;
  if (!is_tail) {
    s0 = (int)((long long)b * B);
    s1 = (int)((long long)s0 + B < L ? (long long)s0 + B : L);
  } else {
    const int n = visible_len(pos[wg], L);
    const int Mt = (int)(((long long)n + B - 1) / B);
    s0 = Mt > 0 ? (int)((long long)(Mt - 1) * B) : 0;
    s1 = n;
  }
  RS::run(K, kscale, s0, s1, red);
  const int tid = threadIdx.x;
  if (tid < kHeadDim) {
    // thread c adds column c of the row groups (contiguous LDS reads); it holds dim d
    double s = MAX ? -__builtin_huge_val() : 0.0;
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      const double x = red[r * kRedStride + tid];
      if constexpr (MAX) s = x > s ? x : s;
      else s += x;
    }
    const int d = RS::dim_of(tid);
    if (MAX && s1 <= s0) s = 0.0;  // no key
    if (!is_tail) {
      ksum[(size_t)b * kHeadDim + d] = s;
      if constexpr (MAX) return;
      const double mean = s / (double)(s1 - s0);
      if (kbar) kbar[(size_t)b * kHeadDim + d] = (float)mean;
      if (kb16) {
        // bf16 hi / lo split of the mean for the router's fast pass
        uint32_t hi, lo;
        split_bf16(mean, hi, lo);
        kb16[(size_t)b * 2 * kHeadDim + d] = (uint16_t)hi;
        kb16[(size_t)b * 2 * kHeadDim + kHeadDim + d] = (uint16_t)lo;
      }
    } else {
      tsum[(size_t)wg * kHeadDim + d] = s;
    }
  }
}

// -------------------------------------------------------------------------
// Router scores rho(t,h,b) = q[t,h] . Kbar_b as float64 matrix products.
// grid (ntiles, ceil(T / QG)), 256 threads: tile c holds blocks
// [16c, 16c + 16), staged once in LDS and kept in registers for QG queries; wave w takes heads [16w, 16w + 16). One v_mfma_f64_16x16x4 step
// takes four head dims; lane l feeds head (A) and block (B) l % 16 with dims
// [32(l/16), 32(l/16) + 32), one per step, so its operands are contiguous.
// The result D[row][col] sits at lane col + 16 * (row % 4), element row / 4.
// Without WITH_BETA (head ranking) it writes part[t, tile, h], the maximum
// of ReLU(q . Ksum_b) over the tile's complete blocks before the query's last
// block, with plain stores (every tile that holds such a block writes; the
// ranking kernel reads exactly those tiles). The value is the raw product with
// the block's sum (or its cached mean), which the ranking kernel divides by the
// block size once: dividing the maximum gives the same value as dividing every
// block's product, division by a positive constant being monotone. When tsum
// is given, the tile holding the query's last (possibly partial) block also
// writes that block's ReLU(rho) to part[T * ntiles + t, h]; otherwise the
// last block is left to the ranking kernel. With
// WITH_BETA it writes the HISA block score beta(t,b) = sum_h w[t,h] ReLU(rho)
// of every visible block, the last one from the query's tail sum tsum.
constexpr int kRouteTile = 16;  // blocks per workgroup

// max over the 16 lanes of each row of the wave (every lane gets its row's max)
template <int CTRL>
__device__ __forceinline__ double dpp_max(double v) {
  const int2 b = __builtin_bit_cast(int2, v);
  int2 o;
  o.x = __builtin_amdgcn_update_dpp(0, b.x, CTRL, 0xf, 0xf, false);
  o.y = __builtin_amdgcn_update_dpp(0, b.y, CTRL, 0xf, 0xf, false);
  const double ov = __builtin_bit_cast(double, o);
  return ov > v ? ov : v;
}
__device__ __forceinline__ double row_max16(double v) {
  v = dpp_max<0x121>(v);  // row_ror:1
  v = dpp_max<0x122>(v);  // row_ror:2
  v = dpp_max<0x124>(v);  // row_ror:4
  return dpp_max<0x128>(v);  // row_ror:8
}

// The last, possibly partial block [(M_t - 1) B, n_t) of query t, pooled from
// the keys in float64 by one workgroup of 256 threads, and ReLU(q . sum /
// count) of every head into slot[0, 64) (heads past H get unused values).
// Thread (h, j) forms head h over dims [32 j, 32 j + 32); the four partial
// products are added in the order j = 0, 1, 2, 3.
template <bool KF8, bool QF8>
__device__ __forceinline__ void route_tail(const void* q, const float* qscale, int H, int t, int n, int B,
                                           const void* K, const float* kscale, double* slot) {
  using RS = RowSum<KF8, false, 256, true>;
  constexpr int RB = QF8 ? kHeadDim : 2 * kHeadDim;  // bytes per q row
  constexpr int QW = RB / 64;                          // 16-byte words of a thread's 32 dims
  __shared__ double red[RS::RR * kRedStride];
  __shared__ double tl[kHeadDim];  // the last block's key sum
  __shared__ double pd[4][kWave];  // products over 32 dims
  const int tid = threadIdx.x, h = tid & 63, j = tid >> 6;
  const int hc = h < H ? h : 0;
  const int Mt = (int)(((long long)n + B - 1) / B);
  const int s0 = Mt > 0 ? (int)((long long)(Mt - 1) * B) : 0;
  // the q row and its scale are requested before the keys (used after them)
  u32x4 qd[QW];
  {
    const u32x4* row = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(q) +
                                                      ((size_t)t * H + hc) * RB) + QW * j;
#pragma unroll
    for (int v = 0; v < QW; ++v) qd[v] = row[v];
  }
  const float sc = QF8 ? qscale[(size_t)t * H + hc] : 1.f;
  RS::run(K, kscale, s0, n, red);  // synchronises
  if (tid < kHeadDim) {
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < RS::RR; ++r) sum += red[r * kRedStride + tid];
    tl[RS::dim_of(tid)] = sum;
  }
  __syncthreads();
  double dp = 0.0;
  if constexpr (QF8) {
    const double qsc = (double)sc;  // code * scale is exact in float64
#pragma unroll
    for (int v = 0; v < QW; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float a0, a1, a2, a3;
        fp8x2_to_f32<false>(qd[v][c], a0, a1);
        fp8x2_to_f32<true>(qd[v][c], a2, a3);
        const int d = 32 * j + 16 * v + 4 * c;
        dp += ((double)a0 * qsc) * tl[d];
        dp += ((double)a1 * qsc) * tl[d + 1];
        dp += ((double)a2 * qsc) * tl[d + 2];
        dp += ((double)a3 * qsc) * tl[d + 3];
      }
  } else {
#pragma unroll
    for (int v = 0; v < QW; ++v)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d = 32 * j + 8 * v + 2 * c;
        dp += (double)bf16_bits_to_f32(qd[v][c] & 0xffffu) * tl[d];
        dp += (double)bf16_bits_to_f32(qd[v][c] >> 16) * tl[d + 1];
      }
  }
  pd[j][h] = dp;
  __syncthreads();
  if (j == 0) {
    const double dt = ((pd[0][h] + pd[1][h]) + pd[2][h]) + pd[3][h];
    const double v = Mt > 0 ? dt / (double)(n - s0) : 0.0;  // the block's own count of keys
    slot[h] = v > 0.0 ? v : 0.0;
  }
  __syncthreads();  // the buffers are reused by the group's next query
}

// QF8: q holds E4M3FN codes with one scale per (query, head) in qscale (null:
// scale 1, rows that already carry their scales); the value code * scale is
// formed exactly in float64.
// MEANS: the complete blocks come as cached float means (kbar), else as float64
// sums (ksum).
// TK (head ranking with cached means, no pooled tails): workgroup column 0
// pools every query's last block from K (TK = 1: bf16 keys, 2: fp8 keys with
// kscale) into the slot after the tile maxima; the tiles are columns 1 .. ntiles.
template <bool WITH_BETA, int kRouteQG, bool QF8, bool MEANS, int TK>
__global__ __launch_bounds__(256) void k_route_mfma(const void* q, const float* qscale, const float* w,
                                                    const int32_t* pos, int T, int H, int L, int B,
                                                    int ntiles, const double* ksum,
                                                    const float* kbar, const double* tsum,
                                                    const void* K, const float* kscale,
                                                    double* part, float* beta, int beta_ld,
                                                    int max_pool) {
  __shared__ f64x2 kt[kRouteTile][kHeadDim / 2 + 1];  // padded rows
  __shared__ double bsum[4][kRouteTile];
  __shared__ f64x2 tls[kRouteQG][kHeadDim / 2];  // the group's query tail sums
  if constexpr (TK != 0) {
    if (blockIdx.x == 0) {  // uniform: the query group's last blocks
      const int tq = blockIdx.y * kRouteQG;
      for (int i = 0; i < kRouteQG && tq + i < T; ++i)
        route_tail<TK == 2, QF8>(q, qscale, H, tq + i, visible_len(pos[tq + i], L), B, K, kscale,
                                 part + ((size_t)T * ntiles + tq + i) * kWave);
      return;
    }
  }
  const int tile = (int)blockIdx.x - (TK != 0 ? 1 : 0), tq0 = blockIdx.y * kRouteQG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int M = (int)(((long long)L + B - 1) / B);
  const int b0 = tile * kRouteTile;
  const int blk = b0 + col;
  const int h_a = kRouteTile * wv + col;  // head fed by this lane's A operand
  // Every global read below is issued from an address that is always valid and
  // masked once it has arrived (a load inside a condition is waited for inside
  // it): the tile's block statistics first, then the q rows, then the lengths.
  int pos_q[kRouteQG];  // lengths first (raw positions; masked below)
#pragma unroll
  for (int i = 0; i < kRouteQG; ++i) pos_q[i] = pos[min(tq0 + i, T - 1)];
  f32x4 xm[2];  // cached means (8 KB per tile): two 16-byte loads per thread
  f64x2 xs[4];  // or block sums (16 KB per tile): four
  if constexpr (MEANS) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 256 * u, r = i >> 5, c4 = i & 31;
      xm[u] = reinterpret_cast<const f32x4*>(kbar + (size_t)min(b0 + r, M - 1) * kHeadDim)[c4];
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, r = i >> 6, c2 = i & 63;
      xs[u] = reinterpret_cast<const f64x2*>(ksum + (size_t)min(b0 + r, M - 1) * kHeadDim)[c2];
    }
  }
  // per query of the group: the A operand (32 bf16 dims, or 32 fp8 codes and
  // the row's scale) in a two-slot ring so the next query's rows load during
  // this one's products, and the visible blocks
  constexpr int QW16 = QF8 ? 2 : 4;
  u32x4 qv[2][4];
  float qsc[2] = {1.f, 1.f};  // widened to float64 where used (exact)
#define MISA_LOAD_Q(i, slot)                                                                     \
  do {                                                                                           \
    const int t_ = tq0 + (i);                                                                    \
    const bool ok_ = t_ < T && h_a < H;                                                          \
    const size_t row_ = (size_t)(ok_ ? t_ : 0) * H + (ok_ ? h_a : 0);                            \
    const u32x4* src_ = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(q) +     \
                                                       row_ * kHeadDim * (QF8 ? 1 : 2) + 32 * g * (QF8 ? 1 : 2)); \
    _Pragma("unroll") for (int v_ = 0; v_ < QW16; ++v_) qv[slot][v_] = src_[v_];                 \
    /* (w stands in as a valid address when the rows carry their scales) */                      \
    const float sc_ = QF8 ? (qscale ? qscale : w)[row_] : 1.f;                                   \
    if (!ok_) {                                                                                  \
      _Pragma("unroll") for (int v_ = 0; v_ < QW16; ++v_) qv[slot][v_] = u32x4{0u, 0u, 0u, 0u}; \
    }                                                                                            \
    if (QF8) qsc[slot] = ok_ ? (qscale ? sc_ : 1.f) : 0.f;                                       \
  } while (0)
  MISA_LOAD_Q(0, 0);
  // the group's tail sums into LDS (read by the lanes of each query's last block)
  if (tsum && tid < kRouteQG * (kHeadDim / 2)) {
    const int i = tid / (kHeadDim / 2), c2 = tid % (kHeadDim / 2);
    tls[i][c2] = reinterpret_cast<const f64x2*>(tsum + (size_t)min(tq0 + i, T - 1) * kHeadDim)[c2];
  }
  int n_q[kRouteQG];
#pragma unroll
  for (int i = 0; i < kRouteQG; ++i) n_q[i] = tq0 + i < T ? visible_len(pos_q[i], L) : 0;
  if constexpr (MEANS) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 256 * u, r = i >> 5, c4 = i & 31;
      const f32x4 x = b0 + r < M ? xm[u] : f32x4{0.f, 0.f, 0.f, 0.f};
      kt[r][2 * c4] = f64x2{(double)x[0], (double)x[1]};
      kt[r][2 * c4 + 1] = f64x2{(double)x[2], (double)x[3]};
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, r = i >> 6;
      kt[i >> 6][i & 63] = b0 + r < M ? xs[u] : f64x2{0.0, 0.0};
    }
  }
  // full blocks hold sums (divide by B), cached means or maxima (divide by 1)
  const double div_full = MEANS || max_pool ? 1.0 : (double)B;
  __syncthreads();
  f64x2 kv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) kv[v] = kt[col][16 * g + v];

#pragma unroll
  for (int i = 0; i < kRouteQG; ++i) {
    const int t = tq0 + i;
    if (t >= T) break;  // uniform
    if (i + 1 < kRouteQG) MISA_LOAD_Q(i + 1, (i + 1) & 1);
    const int n = n_q[i];
    const int Mt = (int)(((long long)n + B - 1) / B);
    // every visible block, the last one from the query's tail sum when the
    // block-sum pass pooled it (tsum); otherwise (cached means, head ranking)
    // the complete blocks only: column 0 pools the last block
    const bool with_tail = WITH_BETA || tsum != nullptr;  // uniform
    const int Mc = with_tail ? Mt : Mt - 1;
    if (b0 >= Mc) continue;  // uniform: no block of this tile is taken
    const bool valid = blk < Mc;
    const bool tail = with_tail && blk == Mt - 1;
    // B operand: the block sums, or this query's own sum for its last block
    f64x2 kb[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) kb[v] = valid ? kv[v] : f64x2{0.0, 0.0};
    if (tail) {
#pragma unroll
      for (int v = 0; v < 16; ++v) kb[v] = tls[i][16 * g + v];
    }
    // two accumulation chains (even and odd dims) keep the matrix unit busy
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; s += 2) {
      double a0, a1;
      if constexpr (QF8) {
        // codes s and s + 1 of the lane's 32, times the row's scale (exact)
        const uint32_t word = qv[i & 1][s >> 4][(s >> 2) & 3];
        float f0, f1;
        fp8x2_to_f32<false>((s & 2) ? (word >> 16) : word, f0, f1);
        a0 = (double)f0 * (double)qsc[i & 1];
        a1 = (double)f1 * (double)qsc[i & 1];
      } else {
        const uint32_t word = qv[i & 1][s >> 3][(s >> 1) & 3];
        a0 = (double)bf16_bits_to_f32(word & 0xffffu);
        a1 = (double)bf16_bits_to_f32(word >> 16);
      }
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, kb[s >> 1][0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, kb[s >> 1][1], acc1, 0, 0, 0);
    }
    const f64x4 acc = acc0 + acc1;
    // this lane holds heads 16 wv + 4 e + g (e = 0..3) against block blk
    if constexpr (!WITH_BETA) {
      // this tile's maximum of ReLU(q . Ksum_b) per head over its complete
      // blocks, raw (see above); the last block's ReLU(rho) to rtail
      double* pp = part + ((size_t)t * ntiles + tile) * kWave + kRouteTile * wv + g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double m = row_max16((valid && !tail && acc[e] > 0.0) ? acc[e] : 0.0);
        // device-scope stores: written through to memory, where the ranking
        // kernel's workgroups (on other XCDs) read them without a probe of
        // this XCD's L2
        if (col == 0) __hip_atomic_store(pp + 4 * e, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (tail) {
        double* rt = part + ((size_t)T * ntiles + t) * kWave + kRouteTile * wv + g;
        const double cnt = (double)(n - (Mt - 1) * B);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double v = acc[e] / cnt;
          __hip_atomic_store(rt + 4 * e, v > 0.0 ? v : 0.0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if constexpr (WITH_BETA) {
      const double cnt = tail ? (max_pool ? 1.0 : (double)(n - (Mt - 1) * B)) : div_full;
      double bs = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hh = kRouteTile * wv + 4 * e + g;
        const double rho = acc[e] / cnt;
        bs += (hh < H && rho > 0.0) ? (double)w[(size_t)t * H + hh] * rho : 0.0;
      }
      bs += __shfl_xor(bs, 16, kWave);
      bs += __shfl_xor(bs, 32, kWave);
      if (lane < kRouteTile) bsum[wv][lane] = bs;
      __syncthreads();
      if (tid < kRouteTile && b0 + tid < Mt) {
        const double s = bsum[0][tid] + bsum[1][tid] + bsum[2][tid] + bsum[3][tid];
        beta[(size_t)t * beta_ld + b0 + tid] = (float)s;
      }
      __syncthreads();
    }
  }
}

#undef MISA_LOAD_Q

// Final router step, one workgroup of 256 threads per query:
// r(t,h) = w[t,h] * max(the complete blocks' maximum, ReLU(rho of the last
// block)), then the first A heads under (-r, h). The complete blocks' maxima
// come from the router tiles (part: raw products, divided here once by
// div_full, the block size, or 1 for cached means), and the last block's
// ReLU(rho) from the slot after them (written by the tile holding that block
// from the block-sum pass's tail sum, or by the router's tail workgroups with
// cached means). heads[t,:] is written in
// ascending head order; with qr the routed q rows and weights are packed in the
// same order for the scoring kernel. QF8: the rows are fp8 codes; a packed row
// is the head's codes with the sign of its scale folded in (bit 7 flipped when
// the scale is negative) and its weight is w * |scale|, so that
// w * ReLU(q . k) of the packed row equals the head's term.
template <bool QF8>
__global__ __launch_bounds__(256) void k_route_select(const void* q, const float* qscale, const float* w, int H,
                                                     int A, const int32_t* pos, int L, int B, int ntiles,
                                                     double div_full, const double* part, int32_t* heads,
                                                     float* r_out, void* qr, float* wr) {
  constexpr int RB = QF8 ? kHeadDim : 2 * kHeadDim;  // bytes per q row
  constexpr int RW = RB / 16;                          // 16-byte words per q row
  __shared__ double pm[4][kWave];  // complete blocks' maxima, per thread group
  __shared__ double rs[kWave];
  __shared__ int rank_part[4][kWave];
  __shared__ u32x4 qs[kWave * RW];  // q[t] as 16-byte words
  const int t = blockIdx.x, tid = threadIdx.x, h = tid & 63, j = tid >> 6;
  const bool active = h < H;
  const int n = visible_len(pos[t], L);
  const int Mt = (int)(((long long)n + B - 1) / B);
  const int nc = Mt > 1 ? (Mt - 1 + kRouteTile - 1) / kRouteTile : 0;  // tiles with complete blocks
  // every global read is issued up front from an address that is always valid
  // (a load inside a condition is waited for inside it); values are masked after
  const int hc = active ? h : 0;
  const float wt_raw = w[(size_t)t * H + hc];
  const float sc_raw = QF8 ? qscale[(size_t)t * H + hc] : 1.f;
  const int nw = H * RW;  // 16-byte words of q[t]
  u32x4 qst[4];  // q[t] for the packed rows (read even when not packed: no branch to wait in)
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(q) + (size_t)t * H * RB);
#pragma unroll
    for (int u = 0; u < 4; ++u) qst[u] = src[min(tid + 256 * u, nw - 1)];
  }
  // every tile's slot is requested before the query's length arrives (slots
  // past its complete blocks hold stale values and are masked afterwards)
  const double mt_raw = part[((size_t)gridDim.x * ntiles + t) * kWave + h];  // gridDim.x = T
  double m = 0.0;  // values >= +0.0
  for (int c0 = 0; c0 < ntiles; c0 += 64) {  // 16 loads in flight per thread
    double x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = part[((size_t)t * ntiles + min(c0 + j + 4 * u, ntiles - 1)) * kWave + h];
#pragma unroll
    for (int u = 0; u < 16; ++u) m = (c0 + j + 4 * u < nc && x[u] > m) ? x[u] : m;
  }
  pm[j][h] = m;
  const float wt = active ? wt_raw : 0.f;
  const float sc = active ? sc_raw : 1.f;
  if (qr) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (tid + 256 * u < nw) qs[tid + 256 * u] = qst[u];
  }
  const double mtail = Mt > 0 ? mt_raw : 0.0;  // the last block's ReLU(rho)
  __syncthreads();  // pm complete
  if (j == 0) {
    double mfull = pm[0][h];
#pragma unroll
    for (int i = 1; i < 4; ++i) mfull = pm[i][h] > mfull ? pm[i][h] : mfull;
    mfull /= div_full;
    const double mm = mtail > mfull ? mtail : mfull;  // ReLU: mfull >= +0.0
    const double r = active ? (double)wt * mm + 0.0 : -__builtin_huge_val();
    if (r_out && active) r_out[(size_t)t * H + h] = (float)r;
    rs[h] = r;
  }
  __syncthreads();
  if (!heads) return;
  {
    // rank of head h: wave j compares it with heads [16j, 16j + 16)
    const double rh = rs[h];
    double r2[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) r2[u] = rs[16 * j + u];
    int c = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) c += (r2[u] > rh) || (r2[u] == rh && 16 * j + u < h);
    rank_part[j][h] = c;
  }
  __syncthreads();
  if (j != 0) return;
  const int rank = rank_part[0][h] + rank_part[1][h] + rank_part[2][h] + rank_part[3][h];
  const bool sel = active && rank < A;
  const uint64_t mask = wave_ballot(sel);
  if (sel) {
    const int slot = lanes_below(mask);
    heads[(size_t)t * A + slot] = h;
    if (qr) {
      wr[(size_t)t * A + slot] = QF8 ? wt * fabsf(sc) : wt;
      const uint32_t flip = (QF8 && sc < 0.f) ? 0x80808080u : 0u;
      u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(qr) + ((size_t)t * A + slot) * RB);
#pragma unroll
      for (int v = 0; v < RW; ++v) {
        u32x4 x = qs[h * RW + v];
        x[0] ^= flip;
        x[1] ^= flip;
        x[2] ^= flip;
        x[3] ^= flip;
        dst[v] = x;
      }
    }
  }
}

// Pack the q rows and weights of caller-given heads in slot order; one wave
// per (query, slot), each lane copying 4 bytes (ids outside [0,H) give zero
// rows and weights). QF8: as in k_route_select, the sign of the scale is
// folded into the codes and |scale| into the weight.
template <bool QF8>
__global__ __launch_bounds__(64) void k_gather_heads(const void* q, const float* qscale, const float* w,
                                                     const int32_t* heads, int H, int A, void* qr, float* wr) {
  constexpr int RB = QF8 ? kHeadDim : 2 * kHeadDim;
  const int t = blockIdx.y, j = blockIdx.x, lane = threadIdx.x;
  const int h = heads[(size_t)t * A + j];
  const bool ok = h >= 0 && h < H;
  const float sc = (QF8 && ok) ? qscale[(size_t)t * H + h] : 1.f;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(q) +
                                                          ((size_t)t * H + (ok ? h : 0)) * RB);
  uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(qr) + ((size_t)t * A + j) * RB);
  if (lane * 4 < RB) dst[lane] = ok ? (src[lane] ^ ((QF8 && sc < 0.f) ? 0x80808080u : 0u)) : 0u;
  if (lane == 0) wr[(size_t)t * A + j] = ok ? (QF8 ? w[(size_t)t * H + h] * fabsf(sc) : w[(size_t)t * H + h]) : 0.f;
}

// -------------------------------------------------------------------------
// Host launchers.

hipError_t launch_block_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                             int L, int B, double* ksum, float* kbar, int T, const int32_t* pos,
                             double* tsum, bool tails_only, uint16_t* kb16, int first_block, bool max_pool) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int base = tails_only ? M : (first_block < M ? first_block : M);
  const int ntail = tsum ? T : 0;
  const int grid = M - base + ntail;
  if (grid == 0) return hipSuccess;
  const char* nm = tails_only ? "tail_sums" : "block_sums";
#define MISA_SUMS_LAUNCH(F8, MX)                                                                    \
  cx.launch(nm, k_block_sums<F8, MX>, dim3(grid), dim3(kSumThreads), 0, K, kscale, L, B, M, ksum,            \
            MX ? nullptr : kbar, MX ? nullptr : kb16, pos, tsum, ntail, base)
  if (max_pool) return fp8 ? MISA_SUMS_LAUNCH(true, true) : MISA_SUMS_LAUNCH(false, true);
  return fp8 ? MISA_SUMS_LAUNCH(true, false) : MISA_SUMS_LAUNCH(false, false);
#undef MISA_SUMS_LAUNCH
}

int route_chunks(int L, int B) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int c = (M + kRouteTile - 1) / kRouteTile;
  return c < 1 ? 1 : c;
}

hipError_t launch_route(const LaunchCtx& cx, const void* q, bool q_fp8, const float* qscale, const float* w,
                        const int32_t* pos, int T, int H, int L, int B, int A, const double* ksum,
                        const float* kbar, const double* tsum, const void* K, const float* kscale, bool k_fp8,
                        double* part, int32_t* heads, float* r_out, float* beta, int beta_ld, void* qr, float* wr,
                        bool max_pool) {
  if (T == 0) return hipSuccess;
  const int nt = route_chunks(L, B);
  const bool f8 = q_fp8;
  if (f8 && (heads || r_out) && !qscale) return hipErrorInvalidValue;  // selection needs the scales
  if (!beta && (!part || max_pool)) return hipErrorInvalidValue;  // ranking: maxima of mean-pooled blocks
  hipError_t e;
  // one query per workgroup while that leaves few workgroups per CU; past
  // that, groups of queries share each staged tile
  const long long work = (long long)nt * T;
  const int qg = work > 16384 ? 8 : (work > 2048 ? 2 : 1);
  // head ranking without pooled tails (cached means): the launch's column 0
  // pools the queries' last blocks from the keys
  const bool pool_tails = !beta && tsum == nullptr;
  if (pool_tails && (kbar == nullptr || K == nullptr)) return hipErrorInvalidValue;
  const dim3 grid(nt + (pool_tails ? 1 : 0), (T + qg - 1) / qg);
#define MISA_ROUTE_LAUNCH1(BETA, QG, QF, MN, TKV)                                                         \
  cx.launch("route_mfma", k_route_mfma<BETA, QG, QF, MN, TKV>, grid, dim3(256), 0, q, qscale, w, pos, T, H, L, B, \
            nt, ksum, kbar, tsum, K, kscale, part, beta, beta_ld, max_pool ? 1 : 0)
#define MISA_ROUTE_POOL(QG, QF) \
  (k_fp8 ? MISA_ROUTE_LAUNCH1(false, QG, QF, true, 2) : MISA_ROUTE_LAUNCH1(false, QG, QF, true, 1))
#define MISA_ROUTE_LAUNCH(BETA, QG)                                                                        \
  (pool_tails ? (f8 ? MISA_ROUTE_POOL(QG, true) : MISA_ROUTE_POOL(QG, false))                              \
   : f8 ? (kbar ? MISA_ROUTE_LAUNCH1(BETA, QG, true, true, 0) : MISA_ROUTE_LAUNCH1(BETA, QG, true, false, 0)) \
        : (kbar ? MISA_ROUTE_LAUNCH1(BETA, QG, false, true, 0) : MISA_ROUTE_LAUNCH1(BETA, QG, false, false, 0)))
  if (beta)
    e = qg == 8 ? MISA_ROUTE_LAUNCH(true, 8) : (qg == 2 ? MISA_ROUTE_LAUNCH(true, 2) : MISA_ROUTE_LAUNCH(true, 1));
  else
    e = qg == 8 ? MISA_ROUTE_LAUNCH(false, 8) : (qg == 2 ? MISA_ROUTE_LAUNCH(false, 2) : MISA_ROUTE_LAUNCH(false, 1));
#undef MISA_ROUTE_LAUNCH
#undef MISA_ROUTE_POOL
#undef MISA_ROUTE_LAUNCH1
  if (e != hipSuccess) return e;
  if (!heads && !r_out) return hipSuccess;  // block scores only
  if (beta) return hipErrorInvalidValue;     // the ranking reads the maxima pass
  const double div_full = kbar ? 1.0 : (double)B;
#define MISA_SELECT_LAUNCH(QF)                                                                          \
  cx.launch("route_select", k_route_select<QF>, dim3(T), dim3(256), 0, q, qscale, w, H, A, pos, L, B, nt, \
            div_full, (const double*)part, heads, r_out, qr, wr)
  return f8 ? MISA_SELECT_LAUNCH(true) : MISA_SELECT_LAUNCH(false);
#undef MISA_SELECT_LAUNCH
}

hipError_t launch_gather_heads(const LaunchCtx& cx, const void* q, bool q_fp8, const float* qscale, const float* w,
                               const int32_t* heads, int T, int H, int A, void* qr, float* wr) {
  if (T == 0) return hipSuccess;
  if (q_fp8 && !qscale) return hipErrorInvalidValue;
  if (q_fp8)
    return cx.launch("gather_heads", k_gather_heads<true>, dim3(A, T), dim3(64), 0, q, qscale, w, heads, H, A, qr, wr);
  return cx.launch("gather_heads", k_gather_heads<false>, dim3(A, T), dim3(64), 0, q, qscale, w, heads, H, A, qr, wr);
}

}  // namespace misa
