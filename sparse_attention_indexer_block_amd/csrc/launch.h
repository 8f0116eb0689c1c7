// Host-side launch plumbing shared by the kernel translation units and the
// C-ABI layer: every kernel goes through LaunchCtx::launch so that optional
// per-kernel timing (HIP events on the launch stream) wraps each launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

constexpr int kHeadDimHost = 128;  // the only head dim the kernels implement

// Profiling hooks (implemented in api.hip). prof_begin/prof_end record a pair
// of HIP events around one launch when profiling is enabled.
void prof_begin(const char* name, hipStream_t stream);
void prof_end(hipStream_t stream);

struct LaunchCtx {
  hipStream_t stream;

  template <typename... KArgs, typename... Args>
  hipError_t launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                    Args... args) const {
    prof_begin(name, stream);
    kernel<<<grid, block, shmem, stream>>>(static_cast<KArgs>(args)...);
    hipError_t e = hipGetLastError();
    prof_end(stream);
    return e;
  }
};

// ---- router side (route_kernels.hip)
hipError_t launch_block_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                             int L, int B, double* ksum, float* kbar);
hipError_t launch_tail_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                            int L, int B, int T, const int32_t* pos, double* tsum);
int route_chunks(int L, int B);
hipError_t launch_route(const LaunchCtx& cx, const uint16_t* q, const float* w, const int32_t* pos,
                        int T, int H, int L, int B, int A, const double* ksum, const double* tsum,
                        double* pmax, int32_t* heads, float* r_out, float* beta, int beta_ld);

// ---- scoring (score_kernels.hip)
struct ScoreArgs {
  const uint16_t* q;     // [T,H,128] bf16
  const float* w;        // [T,H]
  const int32_t* heads;  // [T,A] or null (slot j scores head j)
  int A, H, T;
  const void* K;         // [L,128] bf16 or e4m3fn
  const float* kscale;   // [L] (fp8)
  int L;
  const int32_t* pos;    // [T]
  const int32_t* cand;   // gather mode: [T, cand_ld] key indices
  long long cand_ld;
  const int32_t* ncand;  // gather mode: [T] candidate counts
  float* S;              // output rows
  long long S_ld;
  int tiles_per_split;
  int ngroups;
  int reverse;
};
// Routed (or dense with heads == null, A == H) scores of every visible key:
// S[t, s] = sum_j w[t,h_j] ReLU(q[t,h_j] . k[s]) for s < n_t.
hipError_t launch_score_keys(const LaunchCtx& cx, ScoreArgs a, bool fp8);
// Dense scores of gathered keys: S[t, j] = I_all(t, cand[t, j]) for j < ncand[t].
hipError_t launch_score_gather(const LaunchCtx& cx, ScoreArgs a, bool fp8);

// ---- selection (topk_kernels.hip)
struct TopkArgs {
  const float* S;          // score rows
  long long S_ld;
  const int32_t* row_n;    // [rows] explicit lengths, or null: n from pos
  const int32_t* pos;      // used when row_n == null: n = ceil(visible_len / n_div)
  int L;
  int n_div;
  const int32_t* row_idx;  // [rows, idx_ld] explicit key indices, or null (index = position)
  long long idx_ld;
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
// Long rows: histogram + filter over many workgroups, then per-row selection.
// Workspace of the long-row path; every [rows, *] array has row stride
// topk_long_chunks(max_n) * topk_long_chunk().
struct TopkLongWs {
  uint32_t* ghist;     // [rows, 4096]
  uint32_t* rkeys;     // [rows, stride] candidate keys (one region per chunk)
  int32_t* ridx;       // [rows, stride] candidate indices
  int32_t* rcnt;       // [rows, nchunk]
  uint32_t* gkeys;     // [rows, stride] ordered copy when candidates overflow LDS
  int32_t* gidx;       // [rows, stride]
};
int topk_long_chunks(int max_n);
int topk_long_chunk();
int topk_coarse_bins();
hipError_t launch_topk_long(const LaunchCtx& cx, const TopkArgs& a, const TopkLongWs& ws,
                            int max_n);

hipError_t launch_fill_u32(const LaunchCtx& cx, uint32_t* p, size_t n, uint32_t v);
hipError_t launch_expand_blocks(const LaunchCtx& cx, const int32_t* blocks, const int32_t* nblocks,
                                int m, const int32_t* pos, int L, int B, int T, int32_t* cand,
                                long long cand_ld, int32_t* ncand);

}  // namespace misa
