// Host-side launch plumbing shared by the kernel translation units and the
// C-ABI layer: every kernel goes through LaunchCtx::launch so that optional
// per-kernel timing (HIP events on the launch stream) wraps each launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace misa {

constexpr int kHeadDimHost = 128;  // the only head dim the kernels implement

// Profiling hook (implemented in api.hip): when profiling is enabled it
// creates a start/stop event pair for the launch named `name` and returns true.
bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

struct LaunchCtx {
  hipStream_t stream;

  template <typename... KArgs, typename... Args>
  hipError_t launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                    Args... args) const {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (prof_events(name, &e0, &e1)) {
      // hipExtLaunchKernel stamps the events with the kernel's own start/end
      std::tuple<KArgs...> tup(static_cast<KArgs>(args)...);
      void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
      fill_arg_ptrs(tup, ptrs, std::index_sequence_for<KArgs...>{});
      hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs,
                                        shmem, stream, e0, e1, 0);
      return e != hipSuccess ? e : hipGetLastError();
    }
    kernel<<<grid, block, shmem, stream>>>(static_cast<KArgs>(args)...);
    return hipGetLastError();
  }

 private:
  template <typename Tup, size_t... I>
  static void fill_arg_ptrs(Tup& tup, void** ptrs, std::index_sequence<I...>) {
    ((ptrs[I] = static_cast<void*>(&std::get<I>(tup))), ...);
  }
};

// Row stride (in elements) of internal [rows, n] buffers: a multiple of 128 so
// rows start 512-byte aligned, can be read with 16-byte vector loads, and hold
// whole 128-key score tiles (the scoring kernels write every column of a tile).
inline long long padded_ld(long long n) { return ((n + 127) / 128) * 128; }

// ---- router side (route_kernels.hip)
// Full-block key sums ksum[ceil(L/B), 128] (and optional means kbar) of blocks
// first_block .. ceil(L/B) - 1 and, when tsum is given, the sum of each query's
// last (possibly partial) block. max_pool: per-dimension maxima instead of the
// sums (ksum and tsum then hold max-pooled representatives; kbar, kb16 unused).
hipError_t launch_block_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                             int L, int B, double* ksum, float* kbar, int T, const int32_t* pos,
                             double* tsum, bool tails_only = false, uint16_t* kb16 = nullptr,
                             int first_block = 0, bool max_pool = false);
// MISA head routing with an exact result (route_fast.hip): bf16 block scores
// with proven error bounds, then float64 settling of every head's maximum.
// part: T * route_fast_parts(L, B, T) * 64 records of route_part_bytes();
// kb16 [M][2][128] bf16 hi / lo block means (from launch_block_sums), or kbar.
int route_fast_parts(int L, int B, int T);
// true when the two-pass router pays off (many queries times many block tiles)
bool route_fast_wins(int L, int B, int T);
size_t route_part_bytes();
hipError_t launch_route_heads(const LaunchCtx& cx, const uint16_t* q, const float* w, const int32_t* pos,
                              int T, int H, int L, int B, int A, const double* ksum, const uint16_t* kb16,
                              const float* kbar, const double* tsum, void* part, int32_t* heads,
                              float* r_out, uint16_t* qr, float* wr);
// Router tiles of 16 blocks.
int route_chunks(int L, int B);
// Router, one of two forms.
// Head ranking (beta null, heads or r_out set): the router tiles write the
// per-head maxima of the complete blocks before each query's last block into
// part[T, route_chunks(L, B), 64] (float64; every slot read is written, no
// clearing) and, with tsum, the last block's value into the T * 64 doubles
// after them (when tsum is null, which needs cached means kbar, an extra
// workgroup column of the router launch pools each query's last block from
// K / kscale into those slots instead); then one workgroup per query ranks the heads
// and writes heads[T,A] (ascending), optional r[T,H] and optionally the routed
// q rows qr[T,A,128] and weights wr[T,A] packed in slot order (so scoring
// needs no head indirection). ksum (or kbar) must hold the complete blocks.
// Block scores (beta set): HISA's beta from ksum / kbar and the query tails
// tsum; max_pool: ksum and tsum hold max-pooled representatives
// (launch_block_sums with max_pool), used as given.
// q_fp8: q holds E4M3FN codes with one scale per (query, head) in qscale (null:
// scale 1, for rows that already carry their scales; the head selection needs
// the scales). Packed rows of fp8 queries are codes with the scale's sign
// folded in, and their weights w * |scale|.
hipError_t launch_route(const LaunchCtx& cx, const void* q, bool q_fp8, const float* qscale, const float* w,
                        const int32_t* pos, int T, int H, int L, int B, int A, const double* ksum,
                        const float* kbar, const double* tsum, const void* K, const float* kscale, bool k_fp8,
                        double* part, int32_t* heads, float* r_out, float* beta, int beta_ld, void* qr, float* wr,
                        bool max_pool = false);
// Pack q rows and weights of given heads [T,A] in slot order (ids outside [0,H)
// give zero rows and weights).
hipError_t launch_gather_heads(const LaunchCtx& cx, const void* q, bool q_fp8, const float* qscale, const float* w,
                               const int32_t* heads, int T, int H, int A, void* qr, float* wr);
// true when launch_score_keys can score fp8 queries for this batch (decode
// shapes: every routed row of a query group in one workgroup)
bool score_fp8q_supported(int T, int A);

// ---- scoring (score_kernels.hip)
struct ScoreArgs {
  const void* q;         // [T,H,128] bf16, or E4M3FN codes (q_fp8); slot j < A of query t scores row j
  int q_fp8;             // q holds fp8 codes (keys must be fp8): fp8 x fp8 matrix products
  const float* qscale;   // q_fp8: [T,H] per-row scales (null: rows already carry the sign and
                         // the weights |scale|, as packed by the router)
  const float* w;        // [T,H]
  int A, H, T;           // A <= H rows of each query are scored (H is the row stride)
  const void* K;         // [L,128] bf16 or e4m3fn
  const float* kscale;   // [L] (fp8)
  int L;
  const int32_t* pos;    // [T]
  const int32_t* cand;   // gather mode: [T, cand_ld] key indices
  long long cand_ld;
  int cand_max;          // gather mode: bound on ncand[t]
  const int32_t* ncand;  // gather mode: [T] candidate counts
  // gather mode with a block list instead of cand/ncand: the candidates are the
  // visible keys of blocks[t, 0:nblocks[t]] (ascending, size B); their indices
  // and counts are written to cand_out [T, cand_ld] and ncand_out [T]
  const int32_t* blocks;
  long long blocks_ld;
  const int32_t* nblocks;
  int B;
  int32_t* cand_out;
  int32_t* ncand_out;
  float* S;              // output rows; launch_score_keys needs T + 1 rows (row T takes
                         // the writes of lanes without a query) and S_ld a multiple of 128
  long long S_ld;
  uint32_t* rmm;         // optional [nsplit, T, 2] per-split {min, max} score key of each row
  uint32_t* zero;        // optional buffer the workgroups clear (each a share) ...
  long long zero_n;      // ... (zero_n 32-bit words)
  int tiles_per_split;
  int ngroups;
  int reverse;
  int nsplit;
  int target_wgs;        // workgroups to aim for (0: default)
};
// Scores of every visible key over the first A rows of each query's q and w
// (the routed rows packed by the router, or all H heads for the dense indexer):
// S[t, s] = sum_{j<A} w[t,j] ReLU(q[t,j] . k[s]) for s < n_t; entries of a
// row past n_t (below S_ld) and row T may be overwritten. The number of key
// splits (rows of rmm) is returned in *nsplit_out.
int score_max_splits();
hipError_t launch_score_keys(const LaunchCtx& cx, ScoreArgs a, bool fp8, int* nsplit_out);
// Dense scores of gathered keys: S[t, j] = I_all(t, cand[t, j]) for j < ncand[t]
// (cand either given, or formed from a block list).
hipError_t launch_score_gather(const LaunchCtx& cx, ScoreArgs a, bool fp8);

// ---- selection (topk_kernels.hip)
struct TopkArgs {
  const float* S;          // score rows (16-byte aligned)
  long long S_ld;          // multiple of 4 and >= every row length: the kernels read whole
                           // 16-byte groups up to the one holding a row's last item
  const int32_t* row_n;    // [rows] explicit lengths, or null: n from pos
  const int32_t* pos;      // used when row_n == null: n = ceil(visible_len / n_div)
  int L;
  int n_div;
  const int32_t* row_idx;  // [rows, idx_ld] explicit key indices, or null (index = position)
  long long idx_ld;        // same rule as S_ld
  int rows;
  int k;
  int32_t* out_idx;        // [rows, out_ld]
  float* out_score;        // [rows, out_ld] or null
  long long out_ld;
  int32_t* out_count;      // [rows] or null
};
// Rows no longer than `cap` elements: one workgroup per row in LDS.
int topk_lds_cap();
hipError_t launch_topk_rows(const LaunchCtx& cx, const TopkArgs& a, int max_n);
// Long rows: coarse histogram, threshold bin with per-chunk counts and the
// bin's items, then exact rank inside that bin and ordered emission, each pass
// spread over many workgroups. Every [rows, *] array below has row stride
// topk_long_chunks(max_n) (per chunk) or topk_long_chunks(max_n) *
// topk_long_chunk() (per item).
struct TopkLongWs {
  const uint32_t* rmm; // [nmm, rows, 2] row key ranges written by the scoring kernel
  int nmm;
  uint32_t* ghist;     // [rows, topk_coarse_bins()] (zero on entry)
  void* rec;           // [rows] per-row records of topk_long_rec_bytes()
  int32_t* gcnt;       // [rows, nchunk] items above the threshold bin
  int32_t* bcnt;       // [rows, nchunk] threshold-bin items of each chunk
  uint32_t* bkeys;     // [rows, stride] threshold-bin keys, one region per chunk
};
int topk_long_chunks(int max_n);
int topk_long_chunk();
int topk_long_max_chunks();
size_t topk_long_rec_bytes();
int topk_coarse_bins();
// Rescoring of the kept items with every head, fused into the emission (rows
// whose item index is the key index, i.e. row_idx null): S[row, p] for each
// output position p < out_count[row] gets sum_h w[row,h] ReLU(q[row,h] . k_s)
// (times the key's scale for fp8 keys) of the key s emitted at p.
struct RerankArgs {
  const void* q;         // [rows, H, 128] bf16, or E4M3FN codes (q_fp8, fp8 keys only)
  bool q_fp8;
  const float* qscale;   // q_fp8: [rows, H] per-row scales
  const float* w;        // [rows, H]
  int H;                 // 1 <= H <= 64
  const void* K;         // [L, 128] bf16 or e4m3fn
  const float* kscale;   // [L] (fp8)
  bool fp8;
  float* S;              // [rows, S_ld]
  long long S_ld;        // multiple of 4
};
hipError_t launch_topk_long(const LaunchCtx& cx, const TopkArgs& a, const TopkLongWs& ws,
                            int max_n, const RerankArgs* rr = nullptr);
// Rows whose key range is not known yet: per-chunk ranges into rmm_out
// [topk_long_chunks(max_n), rows, 2] (and `zero` cleared).
hipError_t launch_topk_range(const LaunchCtx& cx, const TopkArgs& a, uint32_t* rmm_out,
                             uint32_t* zero, long long zero_n, int max_n);

hipError_t launch_fill_u32(const LaunchCtx& cx, uint32_t* p, size_t n, uint32_t v);


}  // namespace misa
