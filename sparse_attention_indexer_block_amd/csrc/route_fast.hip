// MISA head routing (MISA technical summary, "Metodologia: MISA": the router
// scores every indexer head against the mean-pooled key blocks and keeps the
// best h heads) in two steps that give the same head set as an exact
// evaluation:
//
//  1. k_route_fast: rho~(t,h,b) = q[t,h] . (hi_b + lo_b) with bf16 matrix
//     products, where hi_b + lo_b is the block mean split into two bf16
//     terms, plus a proven bound err(t,h,b) >= |rho~ - rho| from a third
//     product |q| . |hi_b|. Per (query, head) it keeps, over the complete
//     blocks before the query's last one, the largest and second-largest
//     rho~, the block of the largest and the largest bound, per range of
//     TPW block tiles.
//  2. k_route_exact: per (query, head) the maximum of rho over those blocks is
//     settled in float64: only blocks whose rho~ lies within twice the bound
//     of the largest rho~ can hold the maximum, and only those are evaluated
//     exactly (usually the leader alone); every rho~ is provably negative
//     when the largest is below -bound (maximum 0 after the ReLU). The
//     query's last block is always evaluated exactly.
//     Then r(t,h) = w[t,h] * max(0, max_b rho) and the first A heads under
//     (-r, h), as the float64 router would pick them.
//
// Bound: hi = bf16(float(m)) and lo = bf16(float(m - hi)) leave
// |m - hi - lo| <= 2^-17.9 |m| per dim, and the float accumulation of the 256
// exact bf16 products of a 16x16x32 chain errs by at most 256 * 2^-24 of
// their absolute sum; both are below 2^-15 * sum_d |q_d| |m_d|, and the bound
// used is 2^-14 * |q|.|hi| (|hi| within 2^-8 of |m|), leaving a factor of two.
#include "device_common.h"
#include "launch.h"

namespace misa {

constexpr int kFastTile = 16;  // blocks per MFMA column tile

struct RoutePart {
  float best;    // largest rho~ over the complete blocks seen
  float second;  // second largest
  float err;     // largest bound over those blocks
  int arg;       // block of the largest (-1: none)
};

// Merge (best, second, err, arg) of another set of blocks into ours.
__device__ __forceinline__ void merge_part(float& b, float& s, float& e, int& a, float b2, float s2,
                                           float e2, int a2) {
  const float lo = fminf(b, b2);
  s = fmaxf(fmaxf(s, s2), lo);
  if (b2 > b || (b2 == b && a2 >= 0 && (a < 0 || a2 < a))) a = a2;
  b = fmaxf(b, b2);
  e = fmaxf(e, e2);
}

// grid (ntr, ceil(T / QG)), 256 threads: workgroup tr covers block tiles
// [tr * TPW, tr * TPW + TPW) of QG queries; wave w takes heads [16w, 16w+16).
// v_mfma_f32_16x16x32_bf16 with rows = blocks, columns = heads; lane l feeds
// block / head l % 16 with dims [32(l/16), 32(l/16) + 32) over the four K
// steps, and holds rows (blocks) 4(l/16) + e of column (head) l % 16 of the
// result, so that a head's maximum over a tile stays within its column.
// kb16 [M][2][128] holds the hi / lo split of every block mean; without it
// (cached means) the split is formed here from kbar.
// Settling and selection outputs of the single-pass form (see below).
struct RouteSettle {
  const float* w;
  const double* ksum;  // block sums (used when kbar is null)
  const double* tsum;  // each query's last-block sum
  int A;
  int32_t* heads;
  float* r_out;
  uint16_t* qr;
  float* wr;
};

// Exact q . m_b over this lane's 32 dims (32 g .. 32 g + 31) in float64; qa
// holds those dims of the head's q row, m_b = src[b] / div (block sums) or the
// cached mean, src rows of 128 values.
__device__ __forceinline__ double exact_part32(const bf16x8 (&qa)[4], const double* sum_row,
                                               const float* mean_row, int g) {
  double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const u32x4 qw = __builtin_bit_cast(u32x4, qa[s]);
    if (mean_row) {
      const f32x4* src = reinterpret_cast<const f32x4*>(mean_row + 32 * g + 8 * s);
      const f32x4 x0 = src[0], x1 = src[1];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = p < 2 ? x0[2 * p] : x1[2 * p - 4], b = p < 2 ? x0[2 * p + 1] : x1[2 * p - 3];
        acc0 = fma((double)bf16_bits_to_f32(qw[p] & 0xffffu), (double)a, acc0);
        acc1 = fma((double)bf16_bits_to_f32(qw[p] >> 16), (double)b, acc1);
      }
    } else {
      const f64x2* src = reinterpret_cast<const f64x2*>(sum_row + 32 * g + 8 * s);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f64x2 k2 = src[p];
        acc0 = fma((double)bf16_bits_to_f32(qw[p] & 0xffffu), k2[0], acc0);
        acc1 = fma((double)bf16_bits_to_f32(qw[p] >> 16), k2[1], acc1);
      }
    }
  }
  return acc0 + acc1;
}

// Sum over the four lanes col, col + 16, col + 32, col + 48 (every one receives it).
__device__ __forceinline__ double sum_groups(double v) {
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

// FUSED (every complete block of each query inside this workgroup's range,
// ntr == 1): instead of writing partial records, the workgroup places each
// head by a certified interval of r (the bf16 leader and its bound, and a
// float evaluation of the query's last block with its own bound): a head is in
// when fewer than A heads may beat it, out when at least A heads must, and
// only the heads left between are settled in float64 (the candidate block,
// all blocks for the rare head whose second-best bf16 score reaches the
// leader's bound, and the last block) and ranked among themselves, so the
// chosen set is the one the float64 router picks. It writes heads, r (every
// head exactly when asked for) and the packed q rows and weights of the
// chosen heads, as k_route_exact does.
template <int QG, int TPW, bool FUSED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_route_fast(const uint16_t* q, const int32_t* pos, int T, int H,
                                                    int L, int B, int ntr, const uint16_t* kb16,
                                                    const float* kbar, RoutePart* part, RouteSettle st) {
  // the last query groups (most visible blocks under a causal mask) start first
  const int tr = blockIdx.x, tq0 = (gridDim.y - 1 - blockIdx.y) * QG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int M = (int)(((long long)L + B - 1) / B);
  const int h_a = kFastTile * wv + col;
  int nfull[QG];  // complete blocks before each query's last block
  int nvis[QG];   // visible keys of each query
  float wq[QG];   // (single-pass form) head weight of this lane's head
  float wsel[QG];  // (single-pass form) weight of head tid (tid < 64): the packed weight if chosen
  bf16x8 qa[QG][4];
  // every input read is issued from an always-valid (clamped) address and
  // masked once it has arrived: a read under a condition is waited for inside
  // it, one memory round trip per query
  int pos_raw[QG];
  float wq_raw[QG];
  u32x4 q_raw[QG][4];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    const int tc = min(tq0 + i, T - 1), hc = min(h_a, H - 1);
    pos_raw[i] = pos[tc];
    wq_raw[i] = FUSED ? st.w[(size_t)tc * H + hc] : 0.f;
    // the packed weight of head tid if it is chosen (read here rather than
    // beside the final stores, which would then each wait for it)
    wsel[i] = FUSED ? st.w[(size_t)tc * H + min(tid & (kWave - 1), H - 1)] : 0.f;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)tc * H + hc) * kHeadDim + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) q_raw[i][s] = src[s];
  }
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    const int t = tq0 + i;
    const int n = t < T ? visible_len(pos_raw[i], L) : 0;
    const int Mt = (int)(((long long)n + B - 1) / B);
    nfull[i] = Mt > 0 ? Mt - 1 : 0;
    nvis[i] = n;
    const bool ok = t < T && h_a < H;
    wq[i] = ok ? wq_raw[i] : 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[i][s] = __builtin_bit_cast(bf16x8, ok ? q_raw[i][s] : u32x4{0u, 0u, 0u, 0u});
  }
  // blocks any query of the group can use: only those are staged and scored
  int mneed = 0;
#pragma unroll
  for (int i = 0; i < QG; ++i) mneed = max(mneed, nfull[i]);
  const int bend = min(M, mneed);
  // hi / lo bf16 parts of the workgroup's block means, staged once in LDS for
  // the four waves (rows padded by 16 bytes: conflict-free 16-byte reads)
  constexpr int NB = TPW * kFastTile;
  constexpr int RS = kHeadDim + 8;
  __shared__ __attribute__((aligned(16))) uint16_t smb[2 * NB * RS];
  uint16_t* const smh = smb;
  uint16_t* const sml = smb + NB * RS;
  {
    const int bstart = tr * NB;
    constexpr int NC = NB * 16 / 256;  // 16-byte chunks (8 dims) per thread
    u32x4 hv[NC], lv[NC];
    // every row is read from a valid block (clamped to the last one; M >= 1)
    // before any is used, and rows past bend are stored as zeros below (a read
    // under a condition would be waited for inside it, one round trip per row)
    if (kb16) {
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int c = tid + 256 * u, r = c >> 4, v = c & 15;
        const int blk = min(bstart + r, M - 1);
        hv[u] = reinterpret_cast<const u32x4*>(kb16 + (size_t)blk * 2 * kHeadDim)[v];
        lv[u] = reinterpret_cast<const u32x4*>(kb16 + (size_t)blk * 2 * kHeadDim + kHeadDim)[v];
      }
    } else {
      f32x4 xr[NC][2];
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int c = tid + 256 * u, r = c >> 4, v = c & 15;
        const f32x4* src = reinterpret_cast<const f32x4*>(kbar + (size_t)min(bstart + r, M - 1) * kHeadDim + 8 * v);
        xr[u][0] = src[0];
        xr[u][1] = src[1];
      }
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const f32x4 x0 = xr[u][0], x1 = xr[u][1];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t ha, la, hb, lb;
          split_bf16((double)(p < 2 ? x0[2 * p] : x1[2 * p - 4]), ha, la);
          split_bf16((double)(p < 2 ? x0[2 * p + 1] : x1[2 * p - 3]), hb, lb);
          hv[u][p] = ha | (hb << 16);
          lv[u][p] = la | (lb << 16);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      const int c = tid + 256 * u, r = c >> 4, v = c & 15;
      const bool ok = bstart + r < bend;
      *reinterpret_cast<u32x4*>(&smh[r * RS + 8 * v]) = ok ? hv[u] : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&sml[r * RS + 8 * v]) = ok ? lv[u] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // (single-pass form) each query's last-block sum, rounded to float, for the
  // certified interval of its tail term; and the weights of heads 0..63 (the
  // packed weights of the chosen heads, read from LDS at the end)
  __shared__ float tsh[FUSED ? QG : 1][kHeadDim];
  __shared__ float wsh[FUSED ? QG : 1][kWave];
  if constexpr (FUSED) {
    for (int x = tid; x < QG * kHeadDim; x += 256) {
      const int i = x / kHeadDim, d = x % kHeadDim;
      tsh[i][d] = (float)st.tsum[(size_t)min(tq0 + i, T - 1) * kHeadDim + d];
    }
    if (tid < kWave) {
#pragma unroll
      for (int i = 0; i < QG; ++i) wsh[i][tid] = wsel[i];
    }
  }
  __syncthreads();
  // running record of head 16 wv + col over the blocks of this lane's rows
  float best[QG], second[QG], err[QG];
  int arg[QG];
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    best[i] = -__builtin_huge_valf();
    second[i] = -__builtin_huge_valf();
    err[i] = 0.f;  // largest |q|.|hi| product, scaled to the bound after the loop
    arg[i] = -1;
  }

  for (int tt = 0; tt < TPW; ++tt) {
    const int b0 = (tr * TPW + tt) * kFastTile;
    if (b0 >= bend) break;  // uniform: no query of the group uses these blocks
    // A operands of this lane's block row b0 + col: hi, lo and |hi|, dims 32g .. 32g+31
    bf16x8 bh[4], bl[4], ba[4];
    const int rl = (tt * kFastTile + col) * RS + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 h4 = *reinterpret_cast<const u32x4*>(&smh[rl + 8 * s]);
      bh[s] = __builtin_bit_cast(bf16x8, h4);
      bl[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sml[rl + 8 * s]));
      ba[s] = __builtin_bit_cast(bf16x8, h4 & u32x4{0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu});
    }
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      if (b0 >= nfull[i]) continue;  // uniform: no complete block of this tile
      f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = ah, aa = ah;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        ah = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[s], qa[i][s], ah, 0, 0, 0);
        al = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl[s], qa[i][s], al, 0, 0, 0);
        const u32x4 qabs = __builtin_bit_cast(u32x4, qa[i][s]) & u32x4{0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu, 0x7fff7fffu};
        aa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba[s], __builtin_bit_cast(bf16x8, qabs), aa, 0, 0, 0);
      }
      // element e: block b0 + 4g + e of head 16 wv + col
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int blk = b0 + 4 * g + e;
        if (blk < nfull[i]) {
          const float v = ah[e] + al[e];
          second[i] = fmaxf(second[i], fminf(best[i], v));
          if (v > best[i]) arg[i] = blk;
          best[i] = fmaxf(best[i], v);
          err[i] = fmaxf(err[i], aa[e]);
        }
      }
    }
  }
  // the four row groups hold different blocks of the same head: merge across them,
  // after which every lane of column col holds its head's record
#pragma unroll
  for (int i = 0; i < QG; ++i) {
    // (a block was scored when a leader exists or a bound product is positive: an
    // overflowed screen can leave only NaN values, but |q|.|hi| is never NaN)
    err[i] = arg[i] >= 0 || err[i] > 0.f ? ldexpf(err[i], -14) + 1e-30f : 0.f;
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
      const float b2 = __shfl_xor(best[i], off, kWave), s2 = __shfl_xor(second[i], off, kWave);
      const float e2 = __shfl_xor(err[i], off, kWave);
      const int a2 = __shfl_xor(arg[i], off, kWave);
      merge_part(best[i], second[i], err[i], arg[i], b2, s2, e2, a2);
    }
  }
  if constexpr (!FUSED) {
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < QG; ++i) {
        const int t = tq0 + i;
        if (t >= T) break;
        RoutePart r;
        r.best = best[i];
        r.second = second[i];
        r.err = err[i];
        r.arg = arg[i];
        part[((size_t)t * ntr + tr) * kWave + h_a] = r;
      }
    }
    return;
  } else {
    // The staged means are dead after the tile loop: the settling reuses their LDS.
    struct Lds {
      float2 rb[QG][kWave];                   // certified bounds of r(t, h), rounded outward
      double rex[QG][kWave];                  // exact r of the heads evaluated
      int state[QG][kWave];                   // 0 out, 1 in, 2 evaluated exactly
      int slot_of[QG][kWave];
      uint16_t qrow[4][kHeadDim];             // per wave: one q row
    };
    static_assert(sizeof(Lds) <= sizeof(smb), "settling scratch fits the staging buffer");
    Lds& sh = *reinterpret_cast<Lds*>(smb);
    __syncthreads();  // every wave is past its last read of the staged means

    // Certified interval of r(t, h) = w * max(0, max_b rho) for this lane's head:
    // max_b rho over the complete blocks lies within err of the largest rho~
    // (the maximum is 1-Lipschitz in each term), and the last block's rho within
    // 2^-14 sum |q| |t| / n_tail of its float evaluation (float rounding of the
    // sum and of 34 accumulation steps stay below 2^-18.8 of that sum).
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      const int t = tq0 + i;
      const bool active = t < T && h_a < H;
      const int n = nvis[i];
      const int Mt = (int)(((long long)n + B - 1) / B);
      double lo = -__builtin_huge_val(), hi = -__builtin_huge_val();
      // a float term that overflowed certifies nothing (fmax would drop a NaN)
      bool wide = !__builtin_isfinite(err[i]);
      if (arg[i] >= 0) {
        lo = (double)best[i] - (double)err[i];
        hi = (double)best[i] + (double)err[i];
      }
      if (Mt > 0) {
        float a = 0.f, ab = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const u32x4 qw = __builtin_bit_cast(u32x4, qa[i][s2]);
          const f32x4* tp = reinterpret_cast<const f32x4*>(&tsh[i][32 * g + 8 * s2]);
          const f32x4 t0 = tp[0], t1 = tp[1];
#pragma unroll
          for (int p2 = 0; p2 < 4; ++p2) {
            const float x0 = bf16_bits_to_f32(qw[p2] & 0xffffu), x1 = bf16_bits_to_f32(qw[p2] >> 16);
            const float y0 = p2 < 2 ? t0[2 * p2] : t1[2 * p2 - 4], y1 = p2 < 2 ? t0[2 * p2 + 1] : t1[2 * p2 - 3];
            a = fmaf(x0, y0, a);
            a = fmaf(x1, y1, a);
            ab = fmaf(fabsf(x0), fabsf(y0), ab);
            ab = fmaf(fabsf(x1), fabsf(y1), ab);
          }
        }
        a += __shfl_xor(a, 16, kWave);
        a += __shfl_xor(a, 32, kWave);
        ab += __shfl_xor(ab, 16, kWave);
        ab += __shfl_xor(ab, 32, kWave);
        const double cnt = (double)(n - (Mt - 1) * B);
        const double tv = (double)a / cnt, te = ldexp((double)ab / cnt, -14);
        wide = wide || !(__builtin_isfinite(tv) && __builtin_isfinite(te));
        lo = fmax(lo, tv - te);
        hi = fmax(hi, tv + te);
      }
      const double mlo = fmax(lo, 0.0), mhi = fmax(hi, 0.0);
      const double wd = (double)wq[i];
      double rl = wd >= 0.0 ? wd * mlo : wd * mhi, rh = wd >= 0.0 ? wd * mhi : wd * mlo;
      // such a head is settled exactly
      if (wide) {
        rl = -__builtin_huge_val();
        rh = __builtin_huge_val();
      }
      if (!active) rl = rh = -__builtin_huge_val();
      if (g == 0) {
        float fl = (float)rl, fh = (float)rh;  // outward: below rl, above rh
        if ((double)fl > rl) fl = nextafterf(fl, -__builtin_huge_valf());
        if ((double)fh < rh) fh = nextafterf(fh, __builtin_huge_valf());
        sh.rb[i][h_a] = make_float2(fl, fh);
      }
    }
    __syncthreads();
    static_assert(QG * kWave <= 256, "one thread per (query, head)");
    if (tid < QG * kWave) {
      // head h of query i against every head: how many may beat it (upper bound
      // at or above its lower bound, ties going to the lower head) and how many
      // must (lower bound at or above its upper bound). In: fewer than A may;
      // out: at least A must; else evaluated exactly (every head when the
      // caller asks for r).
      const int i = tid >> 6, h = tid & 63;
      const float2 mine = sh.rb[i][h];
      int may = 0, must = 0;
#pragma unroll 8
      for (int o = 0; o < kWave; ++o) {
        const float2 b = sh.rb[i][o];
        may += o != h && (b.y > mine.x || (b.y == mine.x && o < h));
        must += b.x > mine.y || (b.x == mine.y && o < h);
      }
      const bool active = tq0 + i < T && h < H;
      sh.state[i][h] = !active ? 0 : st.r_out ? 2 : may < st.A ? 1 : must >= st.A ? 0 : 2;
    }
    __syncthreads();
    const double divb = kbar ? 1.0 : (double)B;
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      const bool need = sh.state[i][h_a] == 2;
      if (wave_ballot(need) == 0) continue;  // uniform over the wave
      const int t = tq0 + i;
      const int tc = t < T ? t : T - 1;
      // the head's candidate block, coded as -1 (no block can be positive), the
      // leader block, or the leader + 2^30 when the second best reaches the
      // leader's bound (every block evaluated)
      // (a bound that overflowed leaves the screen unusable: every complete block)
      const bool sure = __builtin_isfinite(err[i]);
      const float thr = best[i] - 2.f * err[i];
      const bool use = sure ? arg[i] >= 0 && best[i] + err[i] >= 0.f : nfull[i] > 0;
      const int c = use ? (max(arg[i], 0) | (!sure || second[i] >= thr ? (1 << 30) : 0)) : -1;
      const int b = c >= 0 ? (c & ((1 << 30) - 1)) : 0;  // (block 0 when there is none: unused)
      const double rho = sum_groups(exact_part32(qa[i], st.ksum + (size_t)b * kHeadDim,
                                                 kbar ? kbar + (size_t)b * kHeadDim : nullptr, g)) / divb;
      double m = c >= 0 && rho > 0.0 ? rho : 0.0;
      uint64_t ambm = wave_ballot(g == 0 && need && c >= 0 && (c >> 30) != 0);
      while (ambm) {
        // a head whose bf16 scores cannot separate its blocks: every complete block
        // in float64, the wave's 16 columns taking 16 blocks at a time
        const int hc = __builtin_ctzll(ambm);  // column (head 16 wv + hc) of the lane group 0 bit
        ambm &= ambm - 1;
        if (col == hc) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            *reinterpret_cast<u32x4*>(&sh.qrow[wv][32 * g + 8 * s2]) = __builtin_bit_cast(u32x4, qa[i][s2]);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the row is in LDS for the whole wave
        __builtin_amdgcn_wave_barrier();
        bf16x8 qh[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) qh[s2] = *reinterpret_cast<const bf16x8*>(&sh.qrow[wv][32 * g + 8 * s2]);
        double mb = 0.0;
        for (int b0 = 0; b0 < nfull[i]; b0 += 2 * kFastTile) {  // uniform over the query
          const int b1 = b0 + col, b2 = b0 + kFastTile + col;
          const int c1 = min(b1, nfull[i] - 1), c2 = min(b2, nfull[i] - 1);
          const double r1 = sum_groups(exact_part32(qh, st.ksum + (size_t)c1 * kHeadDim,
                                                    kbar ? kbar + (size_t)c1 * kHeadDim : nullptr, g)) / divb;
          const double r2 = sum_groups(exact_part32(qh, st.ksum + (size_t)c2 * kHeadDim,
                                                    kbar ? kbar + (size_t)c2 * kHeadDim : nullptr, g)) / divb;
          mb = r1 > mb ? r1 : mb;  // (c1, c2 are complete blocks of this query)
          mb = r2 > mb ? r2 : mb;
        }
        // largest over the 16 columns
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const double o = __shfl_xor(mb, off, kWave);
          mb = o > mb ? o : mb;
        }
        if (col == hc) m = mb > m ? mb : m;
        __builtin_amdgcn_wave_barrier();
      }
      const int n = nvis[i];
      const int Mt = (int)(((long long)n + B - 1) / B);
      if (Mt > 0) {
        // the query's own last block, exactly, from its float64 sum
        const double tq = exact_part32(qa[i], st.tsum + (size_t)tc * kHeadDim, nullptr, g);
        const double rho_t = sum_groups(tq) / (double)(n - (Mt - 1) * B);
        m = rho_t > m ? rho_t : m;
      }
      const double r = (double)wq[i] * m + 0.0;
      if (g == 0 && need) {
        sh.rex[i][h_a] = r;
        if (st.r_out) st.r_out[(size_t)t * H + h_a] = (float)r;
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // the chosen set: every head that is in, and the best of the exactly
      // evaluated heads, under (-r, h), up to A
      const int h = tid;
#pragma unroll
      for (int i = 0; i < QG; ++i) {
        const int t = tq0 + i;
        const int sth = sh.state[i][h];
        const int nin = __builtin_popcountll(wave_ballot(sth == 1));
        bool sel = sth == 1;
        if (wave_ballot(sth == 2) != 0) {  // uniform over the wave
          const double rh = sh.rex[i][h];
          int rank = 0;
          for (int o = 0; o < kWave; ++o) {
            if (sh.state[i][o] != 2) continue;  // uniform
            const double r2 = sh.rex[i][o];
            rank += (r2 > rh) || (r2 == rh && o < h);
          }
          sel = sel || (sth == 2 && rank < st.A - nin);
        }
        const uint64_t mask = wave_ballot(sel);
        const int slot = sel ? lanes_below(mask) : -1;
        sh.slot_of[i][h] = slot;
        if (sel) {
          if (st.heads) st.heads[(size_t)t * st.A + slot] = h;
          if (st.wr) st.wr[(size_t)t * st.A + slot] = wsh[i][h];
        }
      }
    }
    if (st.qr) {
      __syncthreads();
      // the lanes that hold a chosen head's q row write it to its slot
#pragma unroll
      for (int i = 0; i < QG; ++i) {
        const int slot = sh.slot_of[i][h_a];
        if (slot >= 0) {
          u32x4* dst = reinterpret_cast<u32x4*>(st.qr + ((size_t)(tq0 + i) * st.A + slot) * kHeadDim + 32 * g);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) dst[s2] = __builtin_bit_cast(u32x4, qa[i][s2]);
        }
      }
    }
  }
}

// Exact q . m_b in float64, q a 128-dim bf16 row in LDS (16-byte words) and
// m_b the block mean ksum[b] / B or kbar[b]; the whole row of m_b is requested
// at once.
constexpr int kQStride = kHeadDim / 8 + 1;  // 16-byte words per q row in LDS (one pad word)

// Dims [16 sub, 16 sub + 16) of rho(q, b) in float64; eight lanes (sub = 0..7) of one
// group together cover the head dimension and their partials are summed by the caller.
__device__ __forceinline__ double exact_rho_part(const u32x4* qrow, const double* ksum,
                                                 const float* kbar, int b, int B, int sub) {
  const u32x4 q0 = qrow[2 * sub], q1 = qrow[2 * sub + 1];
  double acc = 0.0;
  if (kbar) {
    const f32x4* src = reinterpret_cast<const f32x4*>(kbar + (size_t)b * kHeadDim + 16 * sub);
    f32x4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = src[i];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t qw = p < 4 ? q0[p] : q1[p - 4];
      const f32x4 xx = x[p >> 1];
      acc = fma((double)bf16_bits_to_f32(qw & 0xffffu), (double)xx[2 * (p & 1)], acc);
      acc = fma((double)bf16_bits_to_f32(qw >> 16), (double)xx[2 * (p & 1) + 1], acc);
    }
    return acc;
  }
  const f64x2* src = reinterpret_cast<const f64x2*>(ksum + (size_t)b * kHeadDim + 16 * sub);
  f64x2 k2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) k2[i] = src[i];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t qw = p < 4 ? q0[p] : q1[p - 4];
    acc = fma((double)bf16_bits_to_f32(qw & 0xffffu), k2[p][0], acc);
    acc = fma((double)bf16_bits_to_f32(qw >> 16), k2[p][1], acc);
  }
  return acc;
}

// Sum over the eight lanes of a group; every lane of the group receives the total.
__device__ __forceinline__ double group8_sum(double v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  return v;
}

// Settles one candidate (head hh, block b) with the eight lanes of a group.
__device__ __forceinline__ void settle_block(const u32x4* qs, const double* ksum, const float* kbar,
                                             int hh, int b, int B, int sub,
                                             unsigned long long* mbits) {
  double rho = group8_sum(exact_rho_part(&qs[hh * kQStride], ksum, kbar, b, B, sub));
  if (!kbar) rho = (B & (B - 1)) == 0 ? rho * (1.0 / (double)B) : rho / (double)B;
  if (sub == 0 && rho > 0.0) atomicMax(&mbits[hh], (unsigned long long)__double_as_longlong(rho));
}

// One workgroup of 256 threads per query: settles max_b ReLU(rho) of every
// head exactly, forms r(t,h) and keeps the first A heads under (-r, h).
// A block can hold a head's maximum only if its rho~ is within twice the
// head's bound of the largest rho~; such blocks are evaluated exactly: the
// recorded leader of a block range, or the whole range when its runner-up
// also comes that close. heads[t,:] is written in ascending order; with qr
// the routed q rows and weights are packed in slot order for the scoring
// kernel.
constexpr int kWorkCap = 1024;              // exact-product work items held in LDS

__global__ __launch_bounds__(256) void k_route_exact(const uint16_t* q, const float* w,
                                                    const int32_t* pos, int H, int L, int B, int A,
                                                    int ntr, int range_blocks, const RoutePart* part,
                                                    const double* ksum, const float* kbar,
                                                    const double* tsum, int32_t* heads,
                                                    float* r_out, uint16_t* qr, float* wr) {
  __shared__ u32x4 qs[kWave * kQStride];  // q[t, h, :] for every head
  __shared__ float pb[4][kWave], pe[4][kWave];
  __shared__ float gthr[kWave];           // per head: rho~ below this cannot be the maximum
  __shared__ double ts[kHeadDim];
  __shared__ double rs[kWave];
  __shared__ unsigned long long mbits[kWave];  // settled max_b ReLU(rho) (bits of a double >= 0)
  __shared__ int rank_part[4][kWave];
  __shared__ int work_h[kWorkCap], work_b[kWorkCap];  // (head, block) pairs to evaluate exactly
  __shared__ int n_work;
  const int t = blockIdx.x, tid = threadIdx.x, h = tid & 63, j = tid >> 6;
  const int n = visible_len(pos[t], L);
  const int Mt = (int)(((long long)n + B - 1) / B);
  const int nfull = Mt > 0 ? Mt - 1 : 0;
  const bool active = h < H;
  // everything independent of the partial results is requested first
  const float wt = active ? w[(size_t)t * H + h] : 0.f;
  if (tid < kHeadDim / 2)
    reinterpret_cast<f64x2*>(ts)[tid] = reinterpret_cast<const f64x2*>(tsum + (size_t)t * kHeadDim)[tid];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + (size_t)t * H * kHeadDim);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, row = i >> 4, v = i & 15;  // 64 rows of 16 words
      qs[row * kQStride + v] = row < H ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // global largest rho~ and bound per head
  float b = -__builtin_huge_valf(), e = 0.f;
  for (int c = j; c < ntr; c += 4) {
    const RoutePart p = part[((size_t)t * ntr + c) * kWave + h];
    b = fmaxf(b, p.best);
    e = fmaxf(e, p.err);
  }
  pb[j][h] = b;
  pe[j][h] = e;
  if (tid == 0) n_work = 0;
  if (j == 0) mbits[h] = 0ull;
  __syncthreads();
  if (j == 0) {
#pragma unroll
    for (int jj = 1; jj < 4; ++jj) {
      b = fmaxf(b, pb[jj][h]);
      e = fmaxf(e, pe[jj][h]);
    }
    // b + e < 0: every complete block has rho < 0 (nothing to evaluate); a bound
    // that overflowed (|q|.|hi| bounds every bf16 product) leaves the screen
    // unusable: -inf asks for every complete block
    const bool unsure = !__builtin_isfinite(e);
    gthr[h] = (active && nfull > 0 && (unsure || b + e >= 0.f)) ? (unsure ? -__builtin_huge_valf() : b - 2.f * e)
                                                               : __builtin_huge_valf();
  }
  __syncthreads();
  // candidate blocks of each head (thread j of head h scans ranges j, j+4, ...)
  const float thr = gthr[h];
  const bool every = thr == -__builtin_huge_valf();
  for (int c = j; c < ntr; c += 4) {
    const RoutePart p = part[((size_t)t * ntr + c) * kWave + h];
    if (every ? c * range_blocks < nfull : (p.arg >= 0 && p.best >= thr)) {
      const bool whole = every || p.second >= thr;
      const int first = whole ? c * range_blocks : p.arg;
      const int cnt = whole ? min(range_blocks, nfull - c * range_blocks) : 1;
      const int at = atomicAdd(&n_work, cnt);
      for (int k = 0; k < cnt && at + k < kWorkCap; ++k) {
        work_h[at + k] = h;
        work_b[at + k] = first + k;
      }
    }
  }
  __syncthreads();
  const int nw = n_work;
  const int grp = tid >> 3, sub = tid & 7;  // 32 groups of eight lanes
  if (nw <= kWorkCap) {
    for (int it = grp; it < nw; it += 32) settle_block(qs, ksum, kbar, work_h[it], work_b[it], B, sub, mbits);
  } else {
    // too many candidates to list: every complete block of every head
    for (int i = grp; i < H * nfull; i += 32) {
      const int hh = i / nfull;
      if (gthr[hh] != __builtin_huge_valf()) settle_block(qs, ksum, kbar, hh, i - hh * nfull, B, sub, mbits);
    }
  }
  __syncthreads();
  if (j == 0) {
    double m = __longlong_as_double((long long)mbits[h]);
    if (Mt > 0 && active) {
      // the query's own last block, always exactly
      double acc = 0.0;
      const u32x4* qrow = &qs[h * kQStride];
#pragma unroll 4
      for (int v = 0; v < 16; ++v) {
        const u32x4 qw = qrow[v];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc = fma((double)bf16_bits_to_f32(qw[p] & 0xffffu), ts[8 * v + 2 * p], acc);
          acc = fma((double)bf16_bits_to_f32(qw[p] >> 16), ts[8 * v + 2 * p + 1], acc);
        }
      }
      const double rho = acc / (double)(n - (Mt - 1) * B);
      m = rho > m ? rho : m;
    }
    const double r = active ? (double)wt * m + 0.0 : -__builtin_huge_val();
    if (r_out && active) r_out[(size_t)t * H + h] = (float)r;
    rs[h] = r;
  }
  __syncthreads();
  if (!heads) return;
  {
    // rank of head h: wave j compares it with heads [16j, 16j + 16)
    const double rh = rs[h];
    int c = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const double r2 = rs[16 * j + u];
      c += (r2 > rh) || (r2 == rh && 16 * j + u < h);
    }
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
      wr[(size_t)t * A + slot] = wt;
      u32x4* dst = reinterpret_cast<u32x4*>(qr + ((size_t)t * A + slot) * kHeadDim);
#pragma unroll
      for (int v = 0; v < kHeadDim / 8; ++v) dst[v] = qs[h * kQStride + v];
    }
  }
}

// ---------------------------------------------------------------------------

int route_fast_parts(int L, int B, int T) {
  (void)T;
  const int M = (int)(((long long)L + B - 1) / B);
  const int tiles = (M + kFastTile - 1) / kFastTile;
  return (tiles + 7) / 8;  // ranges of eight block tiles
}

size_t route_part_bytes() { return sizeof(RoutePart); }

bool route_fast_wins(int L, int B, int T) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int tiles = (M + kFastTile - 1) / kFastTile;
  return (long long)tiles * T > 4096;
}

hipError_t launch_route_heads(const LaunchCtx& cx, const uint16_t* q, const float* w, const int32_t* pos,
                              int T, int H, int L, int B, int A, const double* ksum, const uint16_t* kb16,
                              const float* kbar, const double* tsum, void* part, int32_t* heads,
                              float* r_out, uint16_t* qr, float* wr) {
  if (T == 0) return hipSuccess;
  const int ntr = route_fast_parts(L, B, T);
  RoutePart* pp = reinterpret_cast<RoutePart*>(part);
  const uint16_t* kb = kbar ? nullptr : kb16;
  const RouteSettle st{w, ksum, tsum, A, heads, r_out, qr, wr};
  const dim3 grid(ntr, (T + 1) / 2);  // split form: two queries and eight block tiles per workgroup
  if (ntr == 1)  // every block in one range: four queries, settled and selected in the same launch
    return cx.launch("route_fast", k_route_fast<4, 8, true>, dim3(1, (T + 3) / 4), dim3(256), 0, q, pos, T,
                     H, L, B, ntr, kb, kbar, pp, st);
  hipError_t e = cx.launch("route_fast", k_route_fast<2, 8, false>, grid, dim3(256), 0, q, pos, T, H, L, B,
                           ntr, kb, kbar, pp, st);
  if (e != hipSuccess) return e;
  return cx.launch("route_exact", k_route_exact, dim3(T), dim3(256), 0, q, w, pos, H, L, B, A, ntr,
                   8 * kFastTile, (const RoutePart*)pp, ksum, kbar, tsum, heads, r_out, qr, wr);
}

}  // namespace misa
