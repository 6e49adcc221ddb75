// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/absh.h"

struct absh_ctx {
  int T, Y, X, block;
  int N, nb, n_pad;
  int m;        // bits per axis of the enclosing Hilbert cube
  int device;
  int num_cus;        // compute units of the device (persistent launch size)
  int32_t* perm;      // [N] grid index of the r-th token in Hilbert order
  int32_t* inv;       // [N] Hilbert position of grid token n
  int32_t* counters;  // [16] tile-pull counters of the attention kernel (zero between launches)
};

namespace absh {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// Keys per block in the block-transposed value layout: blocks shorter than one
// 32-key MFMA step are padded with zero keys.
__host__ __device__ constexpr int vt_keys(int block) { return block < 32 ? 32 : block; }

// Round a float to bfloat16, nearest-even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Launchers (each returns hipGetLastError() of its launches).
int hilbert_chunks(int m);
hipError_t launch_hilbert_perm(const absh_ctx* c, int32_t* chunk_counts, int chunks, hipStream_t s);
// layout: ABSH_ROWS (bf16 rows), ABSH_VT (bf16, block-transposed) or ABSH_ROWS_F32 (float rows)
hipError_t launch_permute(const absh_ctx* c, const void* x, int x_is_f32, void* xh, int B, int H, int d,
                          int layout, hipStream_t s);
hipError_t launch_permute_pool(const absh_ctx* c, const void* x, int x_is_f32, void* xh, float* xbar, int B, int H,
                               int d, int layout, hipStream_t s);
hipError_t launch_unpermute(const absh_ctx* c, const void* oh, void* o, int B, int H, int d, hipStream_t s);
hipError_t launch_pool(const absh_ctx* c, const void* xh, int xh_is_f32, float* xbar, int B, int H, int d,
                       hipStream_t s);
hipError_t launch_scores(const absh_ctx* c, const float* qbar, const float* kbar, float* S, int BH, int d,
                         hipStream_t s);

struct RouteBuffers {
  const float* S;     // [tiles][nb] block scores, or NULL: computed on chip where needed
  const float* qbar;  // [tiles][d] block means of q (float32)
  const float* kbar;  // [tiles][d] block means of k
  int d;              // head dimension
  int32_t* counts;
  int16_t* kv_idx;    // [tiles][nb] ascending block ids, row-padded
  int16_t* order;     // [tiles][order_depth] importance-order prefix
  int32_t* work;
  float* L;
  int32_t* queue;
  int32_t* target;      // [tiles] slack-fill target counts
  int64_t* slack_info;  // [4] lambda, remainder, E, total
  int32_t* chunk_hist;  // [nb + 1][chunks] chunk histograms of counts, bin nb first (LPT queue)
  int32_t* scan_sums;   // [queue_scan_tiles] totals of the queue scan's tiles
  int32_t* slack_aux;   // [slack_aux_words] count histogram and per-chunk raised tiles (slack fill)
  int32_t* rank;        // [tiles]
  int32_t* sched;        // [10] queue segment bounds (one segment per XCD) and query blocks per unit
  uint32_t* unit_list;   // [units][nb] union lists of query-block groups
  int32_t* unit_cnt;     // [units]
  int32_t* unit_queue;   // [units] group units longest first within each XCD run (ABSH_SCHED_LPT)
  int32_t* owner;        // [B*H] rank of each head after migration (ABSH_SCHED_RANKS)
  int32_t* head_order;   // [B*H] heads by rank, ascending within a rank (ABSH_SCHED_RANKS)
  int64_t* budget;       // [8] SASA budgets E_r in retained blocks (ABSH_SCHED_RANKS)
  double* rank_info;     // [kRankInfo] rank-stage report (ABSH_SCHED_RANKS)
};
// Rank-stage parameters (ABSH_SCHED_RANKS): policy -1 = piecewise on rho with
// thresholds k1, k2; 0 = none; 1 = SASA only; 2 = RLB, then SASA; 3 = RLB only.
struct RankOpts {
  int policy;
  double k1, k2, n1, n2;
};
// unit_members > 1 (first selection from scores in memory only): the same pass also
// writes the union lists of the work units of that many query blocks (rb.unit_list,
// rb.unit_cnt), as launch_groups would from the written lists.
hipError_t launch_select(const absh_ctx* c, const RouteBuffers& rb, int tiles, double p, int k_floor,
                         int order_depth, int reselect, hipStream_t s, int unit_members = 0);
hipError_t launch_slack_plan(const absh_ctx* c, const RouteBuffers& rb, int tiles, double beta, hipStream_t s);
hipError_t launch_workload(const absh_ctx* c, const RouteBuffers& rb, int BH, hipStream_t s);
hipError_t launch_queue(const absh_ctx* c, const RouteBuffers& rb, int tiles, int lpt, hipStream_t s);
int unit_members(const absh_ctx* c, int schedule);  // query blocks per attention work unit
int unit_count(const absh_ctx* c, int BH, int members);
hipError_t launch_groups(const absh_ctx* c, const RouteBuffers& rb, int BH, int members, hipStream_t s);
hipError_t launch_segments(const absh_ctx* c, const RouteBuffers& rb, int BH, int schedule, hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
// unit_queue: the group units of each XCD run (sched bounds) by union length, descending, ties by unit
hipError_t launch_unit_lpt(const absh_ctx* c, const RouteBuffers& rb, int BH, hipStream_t s);
int queue_chunks(int tiles);
int queue_scan_tiles(int tiles, int nb);
int slack_aux_words(int tiles);
hipError_t launch_rank_stage(const absh_ctx* c, const RouteBuffers& rb, int BH, const RankOpts& o, hipStream_t s);
hipError_t launch_rank_fill(const absh_ctx* c, const RouteBuffers& rb, hipStream_t s);
hipError_t launch_rank_final(const RouteBuffers& rb, int BH, hipStream_t s);
hipError_t launch_window_anchor(const absh_ctx* c, const RouteBuffers& rb, int tiles, int window, int stride,
                                int offset, hipStream_t s);

// Work lists of the attention kernel. A unit is `members` neighbouring query
// blocks of one head (1: a single tile taken from the queue; 2 or 4: a group
// walking the union of its members' lists).
struct AttnLists {
  const int32_t* queue;       // single units: queue position -> tile
  const int32_t* counts;      // [tiles]
  const int16_t* kv_idx;      // [tiles][nb]
  const uint32_t* unit_list;  // group units: [units][nb] flagged union entries
  const int32_t* unit_cnt;    // [units]
  const int32_t* sched;       // [10] segment bounds + members (read by the kernel)
  int members;                // host copy of sched[9]
  const int32_t* head_order;  // group units: segment position p / per_head -> head (NULL: identity)
  int strict;                 // 1: a workgroup takes units from its own XCD's segment only
  const int32_t* unit_queue;  // group units: segment position -> unit (NULL: identity or head_order)
  int32_t* counters;          // [16] pull counters (NULL: the context's)
  uint64_t* wg_busy;          // [grid][2] start / end times per workgroup (NULL: none)
};
// Most resident workgroups per CU of any attention kernel (bounds wg_busy).
constexpr int kMaxAttnWgPerCu = 8;
// grid_out: oh is the caller's [B, N, H, d] output in grid order; output row r
// of head (b, h) goes to token perm[r] of batch b, and pad rows (r >= N) are not
// written. Else oh is [B, H, n_pad, d] in Hilbert order.
hipError_t launch_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B,
                            int H, int d, const AttnLists* lists, hipStream_t s, bool grid_out = false);
// Group units of 64- and 128-row query blocks (four and two members) run on the
// union kernel; single tiles and other block sizes on the tile kernel.
bool union_attention_supported(int d, int block, int members);
// vscale == NULL: vt in the bf16 ABSH_VT layout; else vt in the 8-bit ABSH_VT8
// layout with per-channel scales vscale [B*H][d].
hipError_t launch_union_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt,
                                  const float* vscale, void* oh, int B, int H, int d, const AttnLists* lists,
                                  hipStream_t s, bool grid_out = false);
// V quantization: vh [B*H][n_pad][d] bf16 -> vt8 (ABSH_VT8) and vscale [B*H][d].
hipError_t launch_quantize_v(const absh_ctx* c, const void* vh, void* vt8, float* vscale, int BH, int d,
                             hipStream_t s);

}  // namespace absh
