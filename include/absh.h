/*
 * absh.h — C ABI of the Hilbert-ordered Top-p block router and block-sparse
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method is the sparse-routing frontend and block-sparse execution of FVAttn
 * as described on the xllm-io review of FVAttn (section 三 "技术架构", Stage 1
 * "Sparse Mask Routing" and "Block-Sparse Attention Execution"; section 3.1) and
 * on the alanhou.org explainer of FVAttn ("Core Mechanism", layer 1; "Key
 * Concepts", Top-p routing with a safety floor). The multi-GPU runtime stages
 * (head migration, slack augmentation) appear here in their one-GPU form: a
 * longest-processing-time-first tile queue and a slack fill over tiles.
 *
 * Conventions shared by every call
 *  - All tensor, list and workspace pointers are DEVICE pointers on the context's
 *    device unless stated otherwise; the caller owns them. The library owns only
 *    the context and the Hilbert permutation inside it.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *    call except absh_create/absh_destroy only enqueues work on it: no host
 *    synchronisation, no device allocation.
 *  - Each call makes the context's device current while it runs and makes the
 *    caller's current device current again before it returns.
 *  - Grid order: token n = (t*Y + y)*X + x of the (T, Y, X) latent grid; caller
 *    tensors are [B, N, H, d], row-major.
 *  - Hilbert order: the library's own tensors hold tokens sorted along a 3-D
 *    Hilbert curve, in head-major form, with n_pad = nb*block rows per head;
 *    rows N..n_pad-1 are zero. nb = ceil(N / block) blocks of `block` tokens;
 *    block j holds Hilbert positions [j*block, min((j+1)*block, N)).
 *  - A tile is one (batch b, head h, query block i); its id is (b*H + h)*nb + i.
 *  - Attention calls (absh_sparse_attn, absh_sparse_attn_v8) take their work
 *    counters from lists->pull, so calls with different lists may overlap in
 *    time; calls that share one set of counters (the same lists, or dense mode
 *    and lists without pull, which use the context's own) must not. Every other
 *    call only reads the context and may run on another stream concurrently with
 *    any call on the same context.
 *  - Arguments are validated on the host before any HIP call; a failure returns
 *    ABSH_EINVAL / ABSH_EUNSUPPORTED / ABSH_EWORKSPACE and launches nothing.
 *    HIP failures return ABSH_EHIP. absh_last_error() gives the detail of the
 *    last failing call on this thread. Device faults surface at the caller's
 *    next synchronisation. Inputs must be finite.
 */
#ifndef ABSH_H
#define ABSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ABSH_OK = 0,
  ABSH_EINVAL = -1,       /* bad argument (null pointer, value out of range, shape mismatch) */
  ABSH_EUNSUPPORTED = -2, /* valid but not built: head dim, block size or nb outside the kernels */
  ABSH_EWORKSPACE = -3,   /* workspace smaller than absh_route_workspace_bytes() */
  ABSH_ENODEV = -4,       /* no HIP device, or the device index does not exist */
  ABSH_EHIP = -5          /* a HIP runtime call or a kernel launch failed */
} absh_status;

typedef enum { ABSH_BF16 = 0, ABSH_F32 = 1 } absh_dtype;

/* Layout of a tensor in Hilbert order written by absh_permute. */
typedef enum {
  ABSH_ROWS = 0, /* [B, H, n_pad, d] bf16: one row of d per token (queries, keys, outputs) */
  ABSH_VT = 1,   /* [B, H, nb, d, KB] bf16, KB = max(block, 32): each block transposed, keys
                    fastest, zero keys past `block` (values) */
  ABSH_VT8 = 2   /* [B, H, n_pad / 64, 64 * d] bytes, written by absh_quantize_v (values in
                    8-bit floating point): per 64-key step an image of 64*d bytes in which
                    byte e*32*d + 32*c + 16*(g ^ ((c >> 3) & 1)) + 8*a + i holds channel c
                    of key 32*e + 16*a + 8*g + i of the step (e, a, g in {0, 1}, i < 8),
                    as an OCP FP8 E4M3 code of the value divided by the channel's scale */,
  ABSH_ROWS_F32 = 3 /* [B, H, n_pad, d] float32 rows (bf16 inputs widened exactly, float32
                    inputs copied): queries and keys for routing from float32 (absh_route) */
} absh_layout;

typedef struct absh_ctx absh_ctx;

/* Tile schedules for absh_sparse_attn (the one-GPU readings of the xllm-io
 * review's runtime load balancing, section 三 Stage 2 and section 3.2). */
typedef enum {
  ABSH_SCHED_ORDER = 0, /* queue = tile ids in order, pulled by whichever CU is free          */
  ABSH_SCHED_LPT = 1,   /* queue = tiles by retained count, longest first (ties: lower id). With
                           blocks of 64 or 128 the attention work units are query-block groups
                           as for ABSH_SCHED_XCD, cut into the same eight runs, and each run
                           is taken longest first: unit_queue orders its units by union length,
                           descending, ties by unit index. With blocks of 16 the work units are
                           single tiles taken in queue order                                     */
  ABSH_SCHED_XCD = 2,   /* queue = tile ids in order, cut into eight runs of equal retained
                           cost, one per XCD (L2 cache); an XCD whose run is done takes tiles
                           from the next runs                                                  */
  ABSH_SCHED_RANKS = 3  /* the review's rank-level stages with the eight XCDs as the ranks
                           (核心公式 Eq. 2, 5-10; 3.2 RLB; 3.3 SASA and its piecewise policy):
                           XCD r runs the heads of rank r, which first holds the contiguous
                           heads floor(r*B*H/8) .. floor((r+1)*B*H/8)-1; by the policy on
                           rho = max/mean of the rank loads, RLB moves heads within the
                           review's pair topologies (3.2): the ranks are matched in pairs and
                           a pair moves at most one head each way (one send and one receive
                           per rank; a swap moves one each), the plan of least (max,
                           variance) of the new loads over all 105 matchings (exact search);
                           then SASA gives rank r E_r = floor(n1 * dW_r) extra blocks when
                           dW_r = W_max - W_r > n2 * W_max, filling the rank's lightest tiles
                           along their importance order. Work units are query-block groups as
                           for ABSH_SCHED_XCD. Needs B*H <= 1024 and B*H*nb*nb < 2^31.        */
} absh_schedule;

/* Routing options (xllm-io review of FVAttn, section 五 "关键超参数": Top-p
 * operating points 0.90 / 0.95; explainer "Key Concepts": the Top-k floor). */
typedef struct {
  double p;            /* Top-p threshold in (0, 1]; p == 1 keeps every block              */
  int32_t k_floor;     /* Top-k safety floor, >= 0; clamped to nb                         */
  double slack_frac;   /* slack-fill budget beta in [0, 1): E = floor(beta * sum counts)  */
  int32_t schedule;    /* an absh_schedule                                                */
  int32_t order_depth; /* 0..64: length of the importance-order prefix written to `order` */
  /* ABSH_SCHED_RANKS only (ignored otherwise): */
  int32_t rank_policy;  /* -1: by rho (below k1 nothing, below k2 SASA only, else RLB then
                           SASA); 0: nothing; 1: SASA only; 2: RLB then SASA; 3: RLB only     */
  int32_t strict_ranks; /* 1: an XCD takes work only from its own rank (as separate GPUs
                           would); 0: an XCD that is done takes work from the other ranks     */
  double k1, k2;        /* policy thresholds on rho, 0 < k1 <= k2 (the review's 1.05, 1.10)  */
  double n1, n2;        /* SASA coefficient in [0, 1) and trigger >= 0 (0.8, 0.07)           */
  /* The router: ABSH_ROUTER_TOPP, or ABSH_ROUTER_WINDOW_ANCHOR, the structured
   * pattern of the LVSA note (a local window plus global anchor blocks that
   * rotate with the diffusion step): query block i keeps the key blocks j with
   * |j - i| <= window and those with j mod anchor_stride == (step * anchor_shift)
   * mod anchor_stride (anchor_stride 0: no anchors). It reads neither qh nor kh
   * (both may be NULL); p and k_floor are not used; slack_frac and order_depth
   * must be 0, and the schedule ABSH_SCHED_ORDER, _LPT or _XCD. */
  int32_t router;
  int32_t window;        /* >= 0, in blocks on each side                                     */
  int32_t anchor_stride; /* >= 0                                                              */
  int32_t anchor_shift;  /* >= 0: anchor offset advance per diffusion step                    */
  int32_t step;          /* >= 0: the diffusion step                                          */
} absh_route_opts;

#define ABSH_ROUTER_TOPP 0
#define ABSH_ROUTER_WINDOW_ANCHOR 1

/* Routing outputs, caller-allocated device buffers (plus one host field).
 * nb, tiles = B*H*nb. */
typedef struct {
  int32_t* counts; /* [tiles] retained key blocks per tile (after floor and slack fill)        */
  int16_t* kv_idx; /* [tiles][nb] row-padded; the first counts[t] entries, ascending block id
                      (block ids < nb <= 2048 fit in int16)                                     */
  int16_t* order;  /* [tiles][order_depth] block ids, probability descending, ties by smaller
                      id; -1 past nb. May be NULL when order_depth == 0                         */
  int32_t* work;   /* [B*H] sum_i counts (the numerator of Eq. 1, exact)                        */
  float* L;        /* [B*H] L_h = work / nb, float32 division (Eq. 1)                           */
  int32_t* queue;  /* [tiles] tiles by retained count (ABSH_SCHED_LPT) or in order (others)       */
  int32_t* sched;  /* [10] bounds of the eight runs of the attention work queue, one per XCD,
                      then the query blocks per work unit (see absh_sparse_attn)                 */
  uint32_t* unit_list; /* [units][nb] for every schedule whose work units are query-block groups
                      (ABSH_SCHED_ORDER, _XCD, _RANKS, and _LPT with blocks of 64 or 128; else
                      unused, may be NULL; units = absh_lists_units()): the ascending union of
                      the retained lists of the M neighbouring query blocks qM .. qM+M-1 of a
                      head, entry = block id | (member m retains it) << (28 + m); M = 4
                      (block <= 64) or 2                                                        */
  int32_t* unit_cnt; /* [units] length of each union list (same condition as unit_list)         */
  int32_t schedule;  /* HOST field, written by absh_route: the absh_schedule the lists were made
                        for; absh_sparse_attn reads it                                           */
  int32_t* head_order; /* [B*H] ABSH_SCHED_RANKS: the heads by rank after migration (ranks
                        ascending, heads ascending within a rank); the queue segment of rank r
                        holds their work units in this order (else unused, may be NULL)          */
  double* rank_info;   /* [ABSH_RANK_INFO] ABSH_SCHED_RANKS: [0] rho before, [1] after migration,
                        [2] after augmentation; [3] policy taken (0 none, 1 SASA, 2 RLB + SASA, 3 RLB);
                        [4] number of moves; [5..12] rank loads W_r in retained blocks before,
                        [13..20] after migration, [21..28] after augmentation; [29..36] E_r;
                        [37..60] the moves as (head, from, to), by sending rank; [61] candidate
                        plans in the migration space (0 without RLB); [62] 0
                        (else unused, may be NULL)                                               */
  int32_t strict_ranks; /* HOST field, written by absh_route (opts->strict_ranks); absh_sparse_attn
                        reads it                                                                 */
  int32_t* unit_queue; /* [units] ABSH_SCHED_LPT with blocks of 64 or 128: the group units of each
                        of the eight runs (sched), by union length descending, ties by unit
                        index (else unused, may be NULL)                                         */
  int32_t* pull;       /* [ABSH_PULL_WORDS] work counters of the attention launches on these lists:
                        absh_route zeroes them and every attention launch leaves them zero. NULL:
                        attention uses the context's counters                                     */
  uint64_t* wg_busy;   /* optional [absh_attn_workgroups()][2], set by the caller (NULL: none): each
                        attention workgroup writes its start time and the time its last pull found
                        no work, in ticks of the 100 MHz constant clock (s_memrealtime), at index
                        2 * workgroup; entries of workgroups a launch does not have keep their
                        values. For the balance over workers (Eq. 2 over workgroups)            */
} absh_lists;

#define ABSH_PULL_WORDS 16

#define ABSH_RANK_INFO 64

/* Library version as major*10000 + minor*100 + patch. */
int absh_version(void);

/* Human-readable name of a status code. Never NULL. */
const char* absh_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). Valid
 * until the next call into the library on this thread. */
const char* absh_last_error(void);

/* Create a context for one (T, Y, X) grid and block size on `device`.
 * Builds the Hilbert permutation (xllm-io review of FVAttn, 3.1: blocks follow a
 * Hilbert curve so that neighbouring tokens share blocks) on the device: every
 * index of the enclosing 2^m cube is mapped to its cell, out-of-grid cells are
 * dropped, and the survivors are ranked in index order. Synchronises `stream`
 * once (set-up only). block must be 16, 64 or 128. On success *ctx owns device
 * memory for perm and inv (2 * N int32). */
absh_status absh_create(absh_ctx** ctx, int T, int Y, int X, int block, int device, void* stream);

/* Release a context (synchronises the device first). NULL is accepted. */
absh_status absh_destroy(absh_ctx* ctx);

/* Host outputs: token count N, block count nb, padded rows per head n_pad. Any
 * output pointer may be NULL. */
absh_status absh_dims(const absh_ctx* ctx, int* N, int* nb, int* n_pad);

/* Device pointers (owned by the context, valid until absh_destroy) to
 * perm[r] = grid index of the r-th token in Hilbert order, and inv = perm^-1;
 * both int32[N]. */
absh_status absh_perm(const absh_ctx* ctx, const int32_t** perm, const int32_t** inv);

/* Copy perm and inv (int32[N] each) into caller buffers (either may be NULL),
 * asynchronously on `stream`. */
absh_status absh_perm_copy(const absh_ctx* ctx, int32_t* perm_dst, int32_t* inv_dst, void* stream);

/* Gather a grid-order tensor x [B, N, H, d] (bf16, or f32 rounded to bf16 to
 * nearest-even) into Hilbert order, in the given layout, zero-filling pad rows.
 * ABSH_ROWS: xh holds B*H*n_pad*d bf16. ABSH_VT: xh holds B*H*nb*d*KB bf16 with
 * KB = max(block, 32) keys per block (keys past `block` are zero).
 * ABSH_ROWS_F32: xh holds B*H*n_pad*d float32, x unrounded (bf16 widened
 * exactly). d must be 64 or 128. */
absh_status absh_permute(absh_ctx* ctx, const void* x, absh_dtype xt, void* xh, int B, int H, int d,
                         absh_layout layout, void* stream);

/* Scatter a Hilbert-order output oh [B, H, n_pad, d] bf16 back to grid order
 * o [B, N, H, d] bf16 (pad rows are dropped). */
absh_status absh_unpermute(absh_ctx* ctx, const void* oh, void* o, int B, int H, int d, void* stream);

/* Block summaries: xbar[b, h, j, :] = mean of the rows of block j of xh
 * ([B, H, n_pad, d] bf16), summed in float64, divided by the block's true token
 * count in float64, rounded once to float32. xbar: float32 [B, H, nb, d]. */
absh_status absh_pool(absh_ctx* ctx, const void* xh, float* xbar, int B, int H, int d, void* stream);

/* absh_permute and absh_pool in one pass over x (the Hilbert reordering and the
 * block pooling of the xllm-io review's Stage 1): xh exactly as absh_permute
 * writes it in a rows layout (ABSH_ROWS: bf16 rows; ABSH_ROWS_F32: float32 rows),
 * and xbar[b, h, j, :] = the block means of the rows written to xh, bit-identical
 * to absh_pool over them (float64 sums in the same order, one float64 division by
 * the block's token count, rounded once to float32). Routing from these means
 * (absh_route_means) then reads no row a second time. xbar: float32 [B, H, nb, d];
 * x, xh and xbar 16-byte aligned. ABSH_VT is refused with ABSH_EINVAL. */
absh_status absh_permute_pool(absh_ctx* ctx, const void* x, absh_dtype xt, void* xh, float* xbar, int B, int H,
                              int d, absh_layout layout, void* stream);

/* Block scores s[b, h, i, j] = qbar_i . kbar_j / sqrt(d), products and sums in
 * float64, rounded once to float32 (the routing-stage similarity of the xllm-io
 * review's Stage 1). qbar, kbar: float32 [B, H, nb, d]; s: float32 [B, H, nb, nb]. */
absh_status absh_block_scores(absh_ctx* ctx, const float* qbar, const float* kbar, float* s, int B, int H,
                              int d, void* stream);

/* Number of attention work units absh_route makes for this shape and schedule
 * (the row count of absh_lists.unit_list and unit_queue): B*H*ceil(nb/M) with M
 * query blocks per unit, M = 1 for ABSH_SCHED_LPT with blocks of 16, else 4
 * (block <= 64) or 2 (block 128). Every schedule, ABSH_SCHED_RANKS included. 0
 * on a bad argument. */
int absh_lists_units(const absh_ctx* ctx, int B, int H, int schedule);

/* Device bytes of every buffer of absh_lists for this shape, sized for any
 * schedule (units = the largest absh_lists_units()), each buffer 256-byte
 * aligned, in field order: what one arena for absh_lists_carve must hold. 0 on a
 * bad argument (order_depth outside 0..64). */
size_t absh_lists_bytes(const absh_ctx* ctx, int B, int H, int order_depth);

/* Point every device buffer of *out into `arena` (a caller-owned device
 * allocation of at least absh_lists_bytes(), 256-byte aligned): counts, kv_idx,
 * order (NULL when order_depth == 0), work, L, queue, sched, unit_list,
 * unit_cnt, head_order, rank_info, unit_queue. The host fields are reset (schedule
 * -1, strict_ranks 0). Touches no device memory. */
absh_status absh_lists_carve(const absh_ctx* ctx, int B, int H, int order_depth, void* arena, size_t arena_bytes,
                             absh_lists* out);

/* An upper bound on the workgroups of one attention launch on this context (its
 * compute units times the most resident workgroups per compute unit of any
 * attention kernel): the rows of absh_lists.wg_busy. 0 for a NULL context. */
int absh_attn_workgroups(const absh_ctx* ctx);

/* Device workspace needed by absh_route for this shape, in bytes. */
size_t absh_route_workspace_bytes(const absh_ctx* ctx, int B, int H, int d);

/* Device workspace the library's calls need for this shape, in bytes: absh_route's
 * (the attention calls need none). The same value as absh_route_workspace_bytes. */
size_t absh_workspace_bytes(const absh_ctx* ctx, int B, int H, int d);

/* Stage-1 routing (xllm-io review of FVAttn, Stage 1; explainer, "Key Concepts"):
 * from Hilbert-order qh, kh ([B, H, n_pad, d]; qk_type ABSH_BF16: bf16 rows,
 * ABSH_ROWS; ABSH_F32: float32 rows, ABSH_ROWS_F32; 16-byte aligned):
 *   block means -> float32 block scores (through the workspace) -> softmax over
 *   key blocks (float64) ->
 *   Top-p: the fewest blocks, by probability descending (ties: smaller id),
 *   whose cumulative probability reaches p -> floor count' = max(c, min(k, nb))
 *   -> optional slack fill of E = floor(beta * sum count') blocks raising the
 *   lightest tiles along their own importance order -> Eq. 1 workloads
 *   work_h and L_h -> the tile queue (longest first for ABSH_SCHED_LPT), the
 *   work units, and the pull counters (out->pull, if set) zeroed.
 * nb must be <= 2048. Writes every field of *out (order only if
 * opts->order_depth > 0). ws must hold absh_route_workspace_bytes(); its
 * contents are scratch. No host synchronisation. */
absh_status absh_route(absh_ctx* ctx, const void* qh, const void* kh, absh_dtype qk_type, int B, int H, int d,
                       const absh_route_opts* opts, absh_lists* out, void* ws, size_t ws_bytes, void* stream);

/* absh_route from block means the caller already holds (absh_permute_pool, or
 * absh_pool of qh and kh; xllm-io review of FVAttn, Stage 1): qbar, kbar float32
 * [B, H, nb, d], 16-byte aligned. Everything after the pooling is absh_route's,
 * with the same options, workspace size and outputs, so the lists are
 * bit-identical to absh_route's on the rows the means were taken from. Top-p
 * router only (the window/anchor router reads no means: ABSH_EINVAL). */
absh_status absh_route_means(absh_ctx* ctx, const float* qbar, const float* kbar, int B, int H, int d,
                             const absh_route_opts* opts, absh_lists* out, void* ws, size_t ws_bytes, void* stream);

/* The whole path in one call (the pages' drop-in use of the method: grid-order
 * q, k, v in, grid-order attention output out): absh_permute_pool of q and k,
 * absh_permute of v into ABSH_VT, absh_route_means (Top-p router, opts as for
 * absh_route, lists written as absh_route writes them), then
 * absh_sparse_attn_grid over those lists, which writes o in grid order. q, k, v:
 * [B, N, H, d] bf16 or float32 (xt; float32 is rounded to bf16, and routing uses
 * the means of the rounded rows); o: [B, N, H, d] bf16. The Hilbert-order q, k,
 * V^T and the routing scratch live in ws (absh_forward_workspace_bytes(), 256-byte
 * aligned, contents scratch). The same arithmetic in the same order as the
 * separate calls (absh_sparse_attn then absh_unpermute), so o is bit-identical
 * to theirs. */
absh_status absh_forward(absh_ctx* ctx, const void* q, const void* k, const void* v, absh_dtype xt, void* o, int B,
                         int H, int d, const absh_route_opts* opts, absh_lists* lists, void* ws, size_t ws_bytes,
                         void* stream);

/* Device workspace absh_forward needs for this shape, in bytes (0 on a bad argument). */
size_t absh_forward_workspace_bytes(const absh_ctx* ctx, int B, int H, int d);

/* absh_route for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same routing,
 * same arguments and bit-identical outputs, with the block scores computed on chip
 * inside the selection (no score matrix) and the rest of the workspace (block means,
 * slack and queue scratch) taken from a static device array
 * of ABSH_STATIC_SCRATCH_BYTES that the library holds on each GPU until the process
 * ends (its address is looked up by absh_create). The call allocates nothing. A
 * shape whose absh_route_workspace_bytes() exceeds the maximum returns
 * ABSH_EWORKSPACE and launches nothing (720p at 40 heads, about 50 MB, fits; 720p
 * at 64 heads, about 78 MB, does not). All calls on one GPU share the array:
 * calls that overlap in time on one GPU (other streams, other threads, other
 * contexts on the same device) race and must be serialised by the caller. The
 * kernels write every scratch word they read within the call, so nothing carries
 * over from the previous call. */
#define ABSH_STATIC_SCRATCH_BYTES (64u << 20)
absh_status absh_route_static(absh_ctx* ctx, const void* qh, const void* kh, absh_dtype qk_type, int B, int H,
                              int d, const absh_route_opts* opts, absh_lists* out, void* stream);

/* Block-sparse attention (xllm-io review of FVAttn, "Block-Sparse Attention
 * Execution"): for every tile (b, h, i) in lists->queue order,
 *   O_i = softmax(Q_i K_R^T / sqrt(d)) V_R
 * over the tokens of its retained key blocks R (lists->kv_idx, ascending), with
 * the pad keys of a partial last block masked. lists == NULL runs dense
 * attention over every block with the same kernel. qh, kh: [B, H, n_pad, d]
 * bf16 (ABSH_ROWS); vt: ABSH_VT layout; oh: [B, H, n_pad, d] bf16 out (pad rows
 * hold unspecified values). Scores and softmax in float32, probabilities rounded
 * to bf16 for the value product, float32 accumulation. Work is pulled by a
 * persistent grid (one workgroup per CU slot) following lists->sched. A work
 * unit is a group of neighbouring query blocks walking the union of their lists
 * (lists->unit_list), so each staged K/V block serves all of them, taken in unit
 * order (ABSH_SCHED_LPT: lists->unit_queue order within each run); under
 * ABSH_SCHED_LPT with blocks of 16 it is one tile, in lists->queue order. Dense mode
 * uses groups split evenly over the XCDs. Every query row is computed the same way whatever
 * the schedule (same blocks, same ascending order), so outputs do not depend on
 * it. */
absh_status absh_sparse_attn(absh_ctx* ctx, const void* qh, const void* kh, const void* vt, int B, int H,
                             int d, const absh_lists* lists, void* oh, void* stream);

/* V quantization (xllm-io review of FVAttn, "Block-Sparse Attention Execution"
 * and section 3.4, which quantize V before the sparse attention): from
 * Hilbert-order values vh ([B, H, n_pad, d] bf16, ABSH_ROWS) write
 *   vscale[b, h, c] = 2^e, e the smallest integer with max_r |v[b, h, r, c]| * 2^-e <= 448
 *                     (1 for an all-zero channel), float32 [B, H, d];
 *   vt8 = E4M3 codes (OCP FP8: bias 7, largest 448, round to nearest, ties to
 *         even) of v / vscale in the ABSH_VT8 layout, B*H*n_pad*d bytes.
 * The division by a power of two is exact, so the encoding is the only rounding.
 * block must be 64 or 128 (n_pad a multiple of 64); d 64 or 128. vscale's memory
 * serves as scratch during the call. No host synchronisation. */
absh_status absh_quantize_v(absh_ctx* ctx, const void* vh, int B, int H, int d, void* vt8, float* vscale,
                            void* stream);

/* absh_sparse_attn with 8-bit values: vt8 and vscale from absh_quantize_v, the
 * rest as absh_sparse_attn. The value product runs in fp8 (E4M3) with float32
 * accumulation: each probability, scaled by a power of two so that the row's
 * reference maximum maps to at least 2^6 and none exceeds 2^8, is rounded to
 * E4M3, and the row sum adds the same rounded values; the output is multiplied
 * by the channel scales before its bf16 rounding. Scores and softmax as in
 * absh_sparse_attn. Block 64 or 128 (every schedule, or lists == NULL for
 * dense). ABSH_EUNSUPPORTED otherwise. */
absh_status absh_sparse_attn_v8(absh_ctx* ctx, const void* qh, const void* kh, const void* vt8,
                                const float* vscale, int B, int H, int d, const absh_lists* lists, void* oh,
                                void* stream);

/* The attention with the inverse of the Hilbert reordering (xllm-io review of
 * FVAttn, 3.1) folded into its output write: absh_sparse_attn
 * (vscale == NULL; vt in ABSH_VT) or absh_sparse_attn_v8 (vscale and vt8 from
 * absh_quantize_v; block 64 or 128, else ABSH_EUNSUPPORTED), same lists, same
 * arithmetic, but output row r of head (b, h) is stored at o[b, perm[r], h, :]
 * of the caller's grid-order o ([B, N, H, d] bf16, 16-byte aligned), where
 * perm[r] is the grid index of the r-th token in Hilbert order. Pad rows are not
 * written. o is therefore bit-identical to absh_unpermute of the Hilbert-order
 * output, without the Hilbert-order buffer or the extra pass over it. */
absh_status absh_sparse_attn_grid(absh_ctx* ctx, const void* qh, const void* kh, const void* vt,
                                  const float* vscale, int B, int H, int d, const absh_lists* lists, void* o,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ABSH_H */
