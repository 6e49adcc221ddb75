// Block-sparse attention over retained key blocks (xllm-io review of FVAttn,
// "Block-Sparse Attention Execution"; alanhou.org explainer, "Core Mechanism":
// each head attends only to its selected KV blocks), for gfx950.
//
// Persistent kernel: one workgroup per (CU, occupancy slot). A workgroup pulls
// work units one at a time, with an atomic counter per segment of the unit
// queue. The queue is cut into eight segments, one per XCD; a workgroup pulls
// from its own XCD's segment first and then steals from the others in turn. With
// one segment holding every unit this is plain list scheduling in queue order
// (the longest-first order for the LPT tile queue); with the eight-way
// cost-balanced split it keeps the units that run together on one XCD (one L2)
// contiguous in Hilbert order, so they share K/V.
//
// A unit is one tile (b, h, query block i) taken from the tile queue, or a group
// of MEMBERS neighbouring query blocks of one head that walk the union of their
// retained lists together: every staged K/V block serves all members that retain
// it, which divides the K/V traffic per flop by up to MEMBERS. The workgroup has
// GROUPS wave groups; group g holds members 2g and 2g+1, one wave per 16 query
// rows of each, so every K/V operand fragment read from LDS serves two members.
// A member that does not retain a block skips its MFMAs for it.
//
// For every key block j of the unit's list, in ascending order, in sub-blocks of
// at most 64 keys:
//   S^T = K_j Q_i^T         16x16x32 bf16 MFMA, fp32 accumulate
//   online softmax          fp32, base-2 exponent, lazy rescale of O
//   row sums                bf16 dot2 of P against ones (the same rounded P as below)
//   O^T += V_j^T P^T        16x16x32 bf16 MFMA, P rounded to bf16
// K_j (rows of d) and V_j^T (rows of keys, block-transposed by the permute step)
// stream straight from global memory into LDS (buffer loads with the lds bit, 16
// bytes per lane) through a ring of NS stages: NS - 1 blocks are in flight while
// one is computed.
//
// Lane layout (wave of 64, n = lane % 16, g = lane / 16): for a 16x16x32 MFMA the
// A operand of lane (row n, group g) and the B operand of lane (column n,
// group g) carry the same eight k indices, and accumulator element r of lane
// (n, g) is (row 4g + r, column n). Computing S^T puts one query row per lane
// (column n) and lets the accumulator feed the value product directly: within
// each group of 32 keys the A rows of S^T are permuted so that lane group g ends
// up holding the eight consecutive keys 8g..8g+7 of that group, which is exactly
// the k slice its B operand of the value product needs.
//
// LDS layout: rows are stored unpadded (the direct loads write 1 KB runs) and the
// sixteen-byte chunks of a row are XOR-swizzled by a function of the row, chosen
// so that the sixteen rows one quarter-wave reads land on distinct banks.
#include <atomic>
#include <type_traits>

#include "absh_internal.h"

namespace absh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSegments = 8;             // XCDs of an MI355X: one queue segment each
constexpr int kFlagShift = 28;           // list entry: block id | (member m retains it) << (28 + m)
constexpr uint32_t kBlockMask = (1u << kFlagShift) - 1;
constexpr float kLazy = 8.0f;            // base-2 headroom before the softmax reference max moves

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int D, int BLK, int GROUPS>
struct Cfg {
  static constexpr int KB = vt_keys(BLK);   // keys per staged block (16-key blocks padded to 32)
  static constexpr int SB = cmin(KB, 64);   // keys per compute sub-block
  static constexpr int WAVES = BLK / 16;    // waves per query block (16 rows each)
  static constexpr int TW = GROUPS * WAVES; // waves per workgroup
  static constexpr int THREADS = TW * 64;
  static constexpr int MEMBERS = 2 * GROUPS;
  static constexpr int K_ROW = D * 2;       // bytes per K row
  static constexpr int V_ROW = KB * 2;      // bytes per V^T row
  static constexpr int K_BYTES = KB * K_ROW;
  static constexpr int V_BYTES = D * V_ROW;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  // LDS for the stage ring: 8-wave workgroups run one per CU, smaller ones two or more
  static constexpr int LDS_BUDGET = TW >= 8 ? 156 * 1024 : (TW >= 4 ? 78 * 1024 : 38 * 1024);
  static constexpr int NS = cmax(2, cmin(4, LDS_BUDGET / STAGE));
  static constexpr int KT = SB / 16;  // 16-key tiles of S^T per sub-block
  static constexpr int DT = D / 16;   // 16-channel tiles of O^T
  static constexpr int DS = D / 32;   // k steps of Q K^T
  static constexpr int KS = SB / 32;  // k steps of P V per sub-block
  static constexpr int HALVES = KB / SB;
  static constexpr int K_SLICES = BLK * K_ROW / 1024;  // 1 KB direct-load slices per K block
  static constexpr int V_SLICES = V_BYTES / 1024;
  static constexpr int K_PER_WAVE = K_SLICES / TW;
  static constexpr int V_PER_WAVE = V_SLICES / TW;
  static constexpr int LPS = K_PER_WAVE + V_PER_WAVE;  // direct loads per wave per stage
  static_assert(K_SLICES % TW == 0 && V_SLICES % TW == 0, "slices must tile the waves");
  static_assert(NS * STAGE <= 160 * 1024, "stage ring exceeds LDS");
};

// Chunk swizzle of a K row (16-byte chunks): the sixteen rows read by one
// quarter-wave (krow below) map to distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if (D == 128) return (r & 3) | (((r >> 3) & 3) << 2);
  return ((r >> 1) & 1) | (((r >> 3) & 3) << 1);
}
// Which of a lane's K direct-load offsets serves slice w + TW*k: the K swizzle
// depends on bits 1-2 (d = 128) or 0-1 (d = 64) of the slice index, and only the
// bits above log2(TW) vary with k.
template <int D, int TW>
__host__ __device__ constexpr int k_slot(int k) {
  return ((TW * k) >> (D == 128 ? 1 : 0)) & 3;
}
// Chunk swizzle of a V^T row of KB keys.
template <int KB>
__device__ __forceinline__ int v_swz(int r) {
  return (r / (128 / KB)) % (KB / 8);
}

// 16 bytes per lane from a buffer (per-lane offset + wave-uniform offset) straight
// into LDS: lane i lands at lds_dst + 16 i. The buffer's size bounds every read
// (reads past it return zero).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, uint32_t wave_off,
                                           char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void __attribute__((address_space(3)))*)lds_dst, 16, lane_off,
                                           wave_off, 0, 0);
}

constexpr int kRawBufferFlags = 0x00020000;  // raw buffer descriptor, 32-bit data format

// s_waitcnt vmcnt(N) with the other counters left alone (N < 64).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Wait until this wave's loads of the stage about to be computed have landed,
// given that `later` more stages were issued after it.
template <int LPS, int NS>
__device__ __forceinline__ void wait_stage(int later) {
  static_assert((NS - 2) * LPS < 64, "vmcnt range");
  if (NS >= 4 && later >= 2) wait_vm<(NS >= 4 ? 2 * LPS : 0)>();
  else if (NS >= 3 && later >= 1) wait_vm<(NS >= 3 ? LPS : 0)>();
  else wait_vm<0>();
}

// The queue, counts and lists are read-only while the kernel runs: reading them
// through the constant address space lets wave-uniform reads be scalar loads.
typedef const int32_t __attribute__((address_space(4)))* const_i32;
__device__ __forceinline__ const_i32 as_const(const int32_t* p) { return (const_i32)p; }

// Pull the next queue position for this workgroup (thread 0 only); -1 when
// every segment is exhausted. `dead` remembers exhausted segments.
__device__ __forceinline__ int pull(int32_t* counters, const int32_t* bounds, int units, int xcd, unsigned& dead,
                                    int strict) {
  for (int k = 0; k < (strict ? 1 : kSegments); ++k) {
    const int seg = (xcd + k) & (kSegments - 1);
    if (dead & (1u << seg)) continue;
    const int lo = bounds ? bounds[seg] : (int)((int64_t)units * seg / kSegments);
    const int hi = bounds ? bounds[seg + 1] : (int)((int64_t)units * (seg + 1) / kSegments);
    const int idx = atomicAdd(&counters[seg], 1);
    if (lo + idx < hi) return lo + idx;
    dead |= 1u << seg;
  }
  return -1;
}

template <int D, int BLK, int GROUPS>
__global__ __launch_bounds__((Cfg<D, BLK, GROUPS>::THREADS)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_kernel(const bf16_t* __restrict__ qh, const bf16_t* __restrict__ kh, const bf16_t* __restrict__ vt,
                 bf16_t* __restrict__ oh, AttnLists L, int32_t* __restrict__ counters, int units, int nb,
                 int n_pad, int N, float scale_log2, const int32_t* __restrict__ operm, int H) {
  using C = Cfg<D, BLK, GROUPS>;
  constexpr int NS = C::NS;
  __shared__ __attribute__((aligned(1024))) char ring[NS * C::STAGE];
  __shared__ int s_next[2];  // next unit, double-buffered: read one slot while the other is written
  // The output map is needed only after each unit's last step: parked in LDS, it
  // is not held in scalar registers across the step loop.
  __shared__ const int32_t* s_operm;
  __shared__ int s_heads;

  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();  // for the optional busy record
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) {
    s_operm = operm;
    s_heads = H;
  }
  const int grp = wave / C::WAVES;  // this wave's member pair: 2 grp, 2 grp + 1
  const int rw = wave % C::WAVES;   // this wave's 16-row slice of each member
  const int n = lane & 15;
  const int g = lane >> 4;
  const int xcd = blockIdx.x & (kSegments - 1);
  const bool dense = L.counts == nullptr;
  const int members = dense ? C::MEMBERS : L.members;
  const int per_head = (nb + members - 1) / members;

  if (BLK < C::KB) {  // padding keys of every stage stay zero: the loads never write them
    for (int e = tid * 4; e < NS * C::STAGE; e += C::THREADS * 4) *reinterpret_cast<uint32_t*>(ring + e) = 0u;
  }

  // Direct loads: wave w stages the 1 KB slices s = w + TW*k of a K block and of a
  // V^T block (lane i lands at slice base + 16 i). The swizzle reads only a few
  // bits of the slice index, so a lane's source offset minus the slice base takes
  // at most two values over k for K (indexed by k_slot) and one for V^T.
  uint32_t k_lane[4], v_lane;
#pragma unroll
  for (int k = 0; k < C::K_PER_WAVE; ++k) {
    const int sl = wave + C::TW * k;
    const int at = sl * 1024 + lane * 16;
    const int row = at / C::K_ROW, phys = (at % C::K_ROW) / 16;
    k_lane[k_slot<D, C::TW>(k)] = (uint32_t)(row * C::K_ROW + ((phys ^ k_swz<D>(row)) * 16) - sl * 1024);
  }
  {
    const int at = wave * 1024 + lane * 16;
    const int row = at / C::V_ROW, phys = (at % C::V_ROW) / 16;
    v_lane = (uint32_t)(row * C::V_ROW + ((phys ^ v_swz<C::KB>(row)) * 16) - wave * 1024);
  }
  // Per-lane LDS read offsets. S^T step s of key tile t reads K row krow(t, n),
  // logical chunk 4s + g; the t-dependent part of krow is lane-independent.
  int k_rd[C::DS];
  const int krow0 = 8 * (n >> 2) + (n & 3);
#pragma unroll
  for (int s = 0; s < C::DS; ++s) k_rd[s] = krow0 * C::K_ROW + (((4 * s + g) ^ k_swz<D>(krow0)) * 16);
  // The value product, channel tile t and key step u, reads V^T row 16t + n,
  // logical chunk 4u + g; the swizzle of rows 16t + n does not depend on t.
  int v_rd[C::SB / 32 * C::HALVES];
#pragma unroll
  for (int u = 0; u < C::SB / 32 * C::HALVES; ++u)
    v_rd[u] = C::K_BYTES + n * C::V_ROW + (((4 * u + g) ^ v_swz<C::KB>(n)) * 16);

  const int32_t* bounds = dense ? nullptr : L.sched;
  unsigned dead = 0;
  if (tid == 0) s_next[0] = pull(counters, bounds, units, xcd, dead, L.strict);

  for (int parity = 0;; parity ^= 1) {
    __syncthreads();  // s_next[parity] is published; every wave is done with the previous unit
    // wave-uniform values (readfirstlane) so that queue and list reads are scalar loads
    const int pos = __builtin_amdgcn_readfirstlane(s_next[parity]);
    if (pos < 0) break;
    int bh, qb0, cnt;
    const int16_t* plain = nullptr;  // single unit: plain ascending block ids
    const_i32 flagged = nullptr;  // group unit: flagged union entries
    if (members == 1) {
      const int tile = __builtin_amdgcn_readfirstlane(as_const(L.queue)[pos]);
      bh = tile / nb;
      qb0 = tile - bh * nb;
      cnt = as_const(L.counts)[tile];
      plain = L.kv_idx + (size_t)tile * nb;
    } else {
      // segment position -> unit: through unit_queue, or head_order (segments
      // following ranks), or in order
      int unit;
      if (L.unit_queue) {
        unit = __builtin_amdgcn_readfirstlane(as_const(L.unit_queue)[pos]);
      } else {
        const int slot = pos / per_head;
        const int bh_ = L.head_order ? __builtin_amdgcn_readfirstlane(as_const(L.head_order)[slot]) : slot;
        unit = bh_ * per_head + (pos - slot * per_head);
      }
      bh = unit / per_head;
      qb0 = (unit - bh * per_head) * members;
      cnt = dense ? nb : as_const(L.unit_cnt)[unit];
      if (!dense) flagged = as_const(reinterpret_cast<const int32_t*>(L.unit_list) + (size_t)unit * nb);
    }
    // member m of the unit exists when it is below `members` and below nb
    uint32_t present = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (m < members && qb0 + m < nb) present |= 1u << (kFlagShift + m);
    // entry k of the unit's list: block id | membership flags
    auto entry = [&](int k) __attribute__((always_inline)) -> uint32_t {
      if (flagged) return (uint32_t)flagged[k];
      if (plain) return (uint32_t)plain[k] | (1u << kFlagShift);
      return (uint32_t)k | present;
    };

    // this head's K rows and V^T blocks as buffers
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kh + (size_t)bh * n_pad * D), (short)0, n_pad * C::K_ROW, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vt + (size_t)bh * nb * D * C::KB), (short)0, nb * C::V_BYTES, kRawBufferFlags);
    auto issue = [&](int stage, uint32_t e) __attribute__((always_inline)) {
      const uint32_t j = e & kBlockMask;
      char* st = ring + stage * C::STAGE;
#pragma unroll
      for (int k = 0; k < C::K_PER_WAVE; ++k) {
        const int sl = wave + C::TW * k;
        load_lds16(krs, k_lane[k_slot<D, C::TW>(k)], j * (uint32_t)(BLK * C::K_ROW) + sl * 1024, st + sl * 1024);
      }
#pragma unroll
      for (int k = 0; k < C::V_PER_WAVE; ++k) {
        const int sl = wave + C::TW * k;
        load_lds16(vrs, v_lane, j * (uint32_t)C::V_BYTES + sl * 1024, st + C::K_BYTES + sl * 1024);
      }
    };

    // this wave's two members: query rows as the B operand of S^T = K Q^T
    const int m0 = 2 * grp;
    const bool have0 = (present >> (kFlagShift + m0)) & 1u;
    const bool have1 = (present >> (kFlagShift + m0 + 1)) & 1u;
    bf16x8 qf[2][C::DS];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      if (mm == 0 ? have0 : have1) {
        const int qrow = (qb0 + m0 + mm) * BLK + rw * 16 + n;
        const bf16_t* qsrc = qh + ((size_t)bh * n_pad + qrow) * D;
#pragma unroll
        for (int s = 0; s < C::DS; ++s) qf[mm][s] = *reinterpret_cast<const bf16x8*>(qsrc + 32 * s + 8 * g);
      }
    }
    // ring prologue: entries 0 .. NS-2 in flight; entry NS-1 read ahead
    uint32_t ent[NS];
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
      ent[k] = k < cnt ? entry(k) : 0u;
      if (k < cnt) issue(k, ent[k]);
    }
    uint32_t e_ahead = NS - 1 < cnt ? entry(NS - 1) : 0u;
    if (tid == 0) s_next[parity ^ 1] = pull(counters, bounds, units, xcd, dead, L.strict);  // the next unit

    f32x4 o[2][C::DT];
    float l_run[2];  // this lane's share of the row's running sum of (bf16) probabilities
    float m_run[2];  // reference max of this lane's row, base-2 scaled
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
      for (int t = 0; t < C::DT; ++t) o[mm][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run[mm] = 0.f;
      m_run[mm] = -INFINITY;
    }

    // Keys past a block's true length are masked. With BLK < KB every staged block
    // has padding keys; otherwise only the last block of a head can be short, and
    // lists are ascending, so only a unit's final entry can need the mask.
    const bool tail_partial =
        cnt > 0 && ((entry(cnt - 1) & kBlockMask) == (uint32_t)(nb - 1)) && (N - (nb - 1) * BLK < C::KB);

    // One staged key block for this wave's members in MASK (bit 0: 2 grp, bit 1: 2 grp + 1).
    auto compute = [&](const char* cur, int j, auto members_c, auto masked_c) __attribute__((always_inline)) {
      constexpr int MASK = decltype(members_c)::value;
      constexpr bool MASKED = decltype(masked_c)::value;
      const int nj = min(BLK, N - j * BLK);
#pragma unroll
      for (int h = 0; h < C::HALVES; ++h) {
        f32x4 sacc[2][C::KT];
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
          sacc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          sacc[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int tt = h * C::KT + t;
          const int trow = 32 * (tt >> 1) + 4 * (tt & 1);  // lane-independent part of krow
#pragma unroll
          for (int s = 0; s < C::DS; ++s) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + k_rd[s] + trow * C::K_ROW);
            if (MASK & 1) sacc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][s], sacc[0][t], 0, 0, 0);
            if (MASK & 2) sacc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][s], sacc[1][t], 0, 0, 0);
          }
        }
        bf16x8 pf[2][C::KS];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          if (!((MASK >> mm) & 1)) continue;
          if (MASKED) {
            // element r of tile t is key 64h + 32(t/2) + 8g + 4(t%2) + r of the block
            const int lim = nj - 8 * g - 64 * h;
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (32 * (t >> 1) + 4 * (t & 1) + r >= lim) sacc[mm][t][r] = -INFINITY;
          }
          float mx = -INFINITY;
#pragma unroll
          for (int t = 0; t < C::KT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[mm][t][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          // The reference max moves only when a row's block max exceeds it by more
          // than kLazy (base 2): probabilities then stay below 2^kLazy, and O and its
          // row sums are rescaled far less often. The result is the same softmax.
          const float m_blk = mx * scale_log2;
          if (__any(m_blk > m_run[mm] + kLazy)) {
            const float m_new = fmaxf(m_run[mm], m_blk);
            const float alpha = __builtin_amdgcn_exp2f(m_run[mm] - m_new);
#pragma unroll
            for (int t = 0; t < C::DT; ++t) o[mm][t] *= alpha;
            l_run[mm] *= alpha;
            m_run[mm] = m_new;
          }
          const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
          for (int u = 0; u < C::KS; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pf[mm][u][r] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[mm][2 * u][r], scale_log2, -m_run[mm]));
              pf[mm][u][4 + r] =
                  (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[mm][2 * u + 1][r], scale_log2, -m_run[mm]));
            }
            // row sum of the same bf16 probabilities that enter the value product
#pragma unroll
            for (int r = 0; r < 8; r += 2)
              l_run[mm] =
                  __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[mm][u][r], pf[mm][u][r + 1]}, one2, l_run[mm], false);
          }
        }
#pragma unroll
        for (int t = 0; t < C::DT; ++t) {
#pragma unroll
          for (int u = 0; u < C::KS; ++u) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8*>(cur + v_rd[h * C::KS + u] + 16 * t * C::V_ROW);
            if (MASK & 1) o[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[0][u], o[0][t], 0, 0, 0);
            if (MASK & 2) o[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[1][u], o[1][t], 0, 0, 0);
          }
        }
      }
    };

    // One step of the ring: wait for this stage, refill the stage freed by the
    // previous step, then compute.
    auto step = [&](int it, auto stage_c) __attribute__((always_inline)) {
      constexpr int K = decltype(stage_c)::value;
      wait_stage<C::LPS, NS>(min(NS - 2, cnt - 1 - it));
      __syncthreads();
      const uint32_t e = ent[K];
      if (it + NS - 1 < cnt) {
        ent[(K + NS - 1) % NS] = e_ahead;
        issue((K + NS - 1) % NS, e_ahead);
        e_ahead = it + NS < cnt ? entry(it + NS) : 0u;
      }
      const char* cur = ring + K * C::STAGE;
      const int j = (int)(e & kBlockMask);
      const uint32_t mine = (e >> (kFlagShift + m0)) & 3u;
      using T = std::true_type;
      using F = std::false_type;
      using M1 = std::integral_constant<int, 1>;
      using M2 = std::integral_constant<int, 2>;
      using M3 = std::integral_constant<int, 3>;
      if (BLK < C::KB || (tail_partial && it == cnt - 1)) {
        if (mine == 3) compute(cur, j, M3(), T());
        else if (mine == 1) compute(cur, j, M1(), T());
        else if (mine == 2) compute(cur, j, M2(), T());
      } else {
        if (mine == 3) compute(cur, j, M3(), F());
        else if (mine == 1) compute(cur, j, M1(), F());
        else if (mine == 2) compute(cur, j, M2(), F());
      }
    };

    for (int it = 0; it < cnt; it += NS) {
      step(it, std::integral_constant<int, 0>());
      if (it + 1 < cnt) step(it + 1, std::integral_constant<int, 1 % NS>());
      if (NS > 2 && it + 2 < cnt) step(it + 2, std::integral_constant<int, 2 % NS>());
      if (NS > 3 && it + 3 < cnt) step(it + 3, std::integral_constant<int, 3 % NS>());
    }

#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      if (!(mm == 0 ? have0 : have1)) continue;
      float l = l_run[mm] + __shfl_xor(l_run[mm], 16);
      l += __shfl_xor(l, 32);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int qrow = (qb0 + m0 + mm) * BLK + rw * 16 + n;
      // Hilbert order (every padded row), or the caller's grid order: row r of
      // head (b, h) is token perm[r] of batch b, and pad rows are not written
      const int32_t* om = s_operm;
      const int nh = s_heads;
      const bool keep = om == nullptr || qrow < N;
      const size_t out_row = om == nullptr ? (size_t)bh * n_pad + qrow
                                           : ((size_t)(bh / nh) * N + (keep ? om[qrow] : 0)) * nh + bh % nh;
      bf16_t* orow = oh + out_row * D;
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(o[mm][t][0] * inv) | ((uint32_t)f32_to_bf16(o[mm][t][1] * inv) << 16);
        w.y = (uint32_t)f32_to_bf16(o[mm][t][2] * inv) | ((uint32_t)f32_to_bf16(o[mm][t][3] * inv) << 16);
        if (keep) *reinterpret_cast<uint2*>(orow + 16 * t + 4 * g) = w;
      }
    }
  }

  // The last workgroup to finish resets the pull counters for the next launch.
  if (tid == 0) {
    if (L.wg_busy) {
      L.wg_busy[2 * blockIdx.x] = t_start;
      L.wg_busy[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
    }
    __threadfence();
    if (atomicAdd(&counters[kSegments], 1) == (int)gridDim.x - 1) {
      for (int s = 0; s <= kSegments; ++s) atomicExch(&counters[s], 0);
      __threadfence();
    }
  }
}

template <int D, int BLK, int GROUPS>
hipError_t launch(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B, int H,
                  const AttnLists& L, bool dense, hipStream_t s, bool grid_out) {
  using C = Cfg<D, BLK, GROUPS>;
  // resident workgroups per CU for this instantiation (one gfx950 value; computed once,
  // an atomic so that concurrent first calls from several threads are well defined)
  static std::atomic<int> occupancy{0};
  int per_cu = occupancy.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<D, BLK, GROUPS>, C::THREADS, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    occupancy.store(per_cu, std::memory_order_relaxed);
  }
  const int members = dense ? C::MEMBERS : L.members;
  const int units = B * H * ((c->nb + members - 1) / members);
  const int grid = c->num_cus * per_cu;
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  AttnLists Lk = L;
  if (dense) Lk = AttnLists{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, C::MEMBERS};
  if (grid > c->num_cus * kMaxAttnWgPerCu) return hipErrorInvalidConfiguration;  // wg_busy's bound
  int32_t* counters = Lk.counters ? Lk.counters : c->counters;
  attn_kernel<D, BLK, GROUPS><<<grid, C::THREADS, 0, s>>>(
      reinterpret_cast<const bf16_t*>(qh), reinterpret_cast<const bf16_t*>(kh), reinterpret_cast<const bf16_t*>(vt),
      reinterpret_cast<bf16_t*>(oh), Lk, counters, units, c->nb, c->n_pad, c->N, scale_log2,
      grid_out ? c->perm : nullptr, H);
  return hipGetLastError();
}

// Wave groups per workgroup for a unit of `members` query blocks: single tiles
// and pairs use one group, quads two.
template <int D, int BLK>
hipError_t dispatch(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B, int H,
                    const AttnLists* lists, hipStream_t s, bool grid_out) {
  const int members = lists ? lists->members : (BLK >= 128 ? 2 : 4);
  AttnLists L = lists ? *lists : AttnLists{};
  if (members == 4) return launch<D, BLK, (BLK >= 128 ? 1 : 2)>(c, qh, kh, vt, oh, B, H, L, !lists, s, grid_out);
  return launch<D, BLK, 1>(c, qh, kh, vt, oh, B, H, L, !lists, s, grid_out);
}

}  // namespace

int attention_members(const absh_ctx* c, const AttnLists* lists) {
  return lists ? lists->members : (c->block >= 128 ? 2 : 4);
}

hipError_t launch_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B,
                            int H, int d, const AttnLists* lists, hipStream_t s, bool grid_out) {
  const int members = lists ? lists->members : (c->block >= 128 ? 2 : 4);
  if (union_attention_supported(d, c->block, members))
    return launch_union_attention(c, qh, kh, vt, nullptr, oh, B, H, d, lists, s, grid_out);
#define ABSH_ATTN(DD, BB) \
  if (d == DD && c->block == BB) return dispatch<DD, BB>(c, qh, kh, vt, oh, B, H, lists, s, grid_out);
  ABSH_ATTN(64, 16)
  ABSH_ATTN(64, 64)
  ABSH_ATTN(64, 128)
  ABSH_ATTN(128, 16)
  ABSH_ATTN(128, 64)
  ABSH_ATTN(128, 128)
#undef ABSH_ATTN
  return hipErrorInvalidValue;
}

}  // namespace absh
