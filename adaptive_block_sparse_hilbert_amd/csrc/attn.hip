// Block-sparse attention over retained key blocks (xllm-io review of FVAttn,
// "Block-Sparse Attention Execution"; alanhou.org explainer, "Core Mechanism":
// each head attends only to its selected KV blocks), for gfx950.
//
// Persistent kernel: one workgroup per (CU, occupancy slot). A workgroup pulls
// work units one at a time, with an atomic counter per segment of the unit
// queue. The queue is cut into eight segments, one per XCD; a workgroup pulls
// from its own XCD's segment first and then steals from the others in turn. With
// one segment holding every unit this is plain list scheduling in queue order
// (the longest-first order for the LPT queue); with the eight-way cost-balanced
// split it keeps the units that run together on one XCD (one L2) contiguous in
// Hilbert order, so they share K/V.
//
// A unit is either one tile (b, h, query block i), taken from the tile queue, or
// a pair of neighbouring query blocks (2p, 2p+1) of one head that walk the union
// of their retained lists together: each staged K/V block, and each K/V operand
// fragment read from LDS, then serves both blocks, which halves the K/V traffic
// per flop; a block retained by only one member skips the other's MFMAs.
//
// Per unit, one wave per 16 query rows of each member. For every key block j of
// the unit's list, in ascending order:
//   S^T = K_j Q_i^T         16x16x32 bf16 MFMA, fp32 accumulate
//   online softmax          fp32, base-2 exponent, lazy rescale of O
//   O^T += V_j^T P^T        16x16x32 bf16 MFMA, P rounded to bf16
// K_j (rows of d) and V_j^T (rows of keys, block-transposed by the permute step)
// stream straight from global memory into LDS (global_load_lds, 16 bytes per
// lane), double-buffered: block j+1 is in flight while block j is computed.
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
#include <type_traits>

#include "absh_internal.h"

namespace absh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSegments = 8;  // XCDs of an MI355X: one queue segment each
constexpr uint32_t kInFirst = 1u << 30;   // list entry flag: the unit's first query block retains it
constexpr uint32_t kInSecond = 1u << 31;  // list entry flag: the second query block retains it
constexpr uint32_t kBlockMask = kInFirst - 1;

template <int D, int BLK>
struct Cfg {
  static constexpr int KB = vt_keys(BLK);  // keys per staged block (16-key blocks padded to 32)
  static constexpr int WAVES = BLK / 16;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int K_ROW = D * 2;   // bytes per K row
  static constexpr int V_ROW = KB * 2;  // bytes per V^T row
  static constexpr int K_BYTES = KB * K_ROW;
  static constexpr int V_BYTES = D * V_ROW;
  static constexpr int KT = KB / 16;  // 16-key tiles of S^T
  static constexpr int DT = D / 16;   // 16-channel tiles of O^T
  static constexpr int DS = D / 32;   // k steps of Q K^T
  static constexpr int KS = KB / 32;  // k steps of P V
  static constexpr int K_SLICES = BLK * K_ROW / 1024;  // 1 KB direct-load slices per K block
  static constexpr int V_SLICES = V_BYTES / 1024;
  static constexpr int K_PER_WAVE = K_SLICES / WAVES;
  static constexpr int V_PER_WAVE = V_SLICES / WAVES;
  static_assert(K_SLICES % WAVES == 0 && V_SLICES % WAVES == 0, "slices must tile the waves");
};

// Chunk swizzle of a K row (16-byte chunks): the sixteen rows read by one
// quarter-wave (krow below) map to distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if (D == 128) return (r & 3) | (((r >> 3) & 3) << 2);
  return ((r >> 1) & 1) | (((r >> 3) & 3) << 1);
}
// Chunk swizzle of a V^T row of KB keys.
template <int KB>
__device__ __forceinline__ int v_swz(int r) {
  return (r / (128 / KB)) % (KB / 8);
}

__device__ __forceinline__ void load_lds16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// The queue, counts and lists are read-only while the kernel runs: reading them
// through the constant address space lets wave-uniform reads be scalar loads.
typedef const int32_t __attribute__((address_space(4)))* const_i32;
__device__ __forceinline__ const_i32 as_const(const int32_t* p) { return (const_i32)p; }

// Pull the next queue position for this workgroup (thread 0 only); -1 when
// every segment is exhausted. `dead` remembers exhausted segments.
__device__ __forceinline__ int pull(int32_t* counters, const int32_t* bounds, int tiles, int xcd, unsigned& dead) {
  for (int k = 0; k < kSegments; ++k) {
    const int seg = (xcd + k) & (kSegments - 1);
    if (dead & (1u << seg)) continue;
    const int lo = bounds ? bounds[seg] : (int)((int64_t)tiles * seg / kSegments);
    const int hi = bounds ? bounds[seg + 1] : (int)((int64_t)tiles * (seg + 1) / kSegments);
    const int idx = atomicAdd(&counters[seg], 1);
    if (lo + idx < hi) return lo + idx;
    dead |= 1u << seg;
  }
  return -1;
}

template <int D, int BLK>
__global__ __launch_bounds__((Cfg<D, BLK>::THREADS)) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_kernel(
    const bf16_t* __restrict__ qh, const bf16_t* __restrict__ kh, const bf16_t* __restrict__ vt,
    bf16_t* __restrict__ oh, AttnLists L, int32_t* __restrict__ counters, int units, int nb, int n_pad, int N,
    float scale_log2) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char stage0[C::K_BYTES + C::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[C::K_BYTES + C::V_BYTES];
  __shared__ int s_next;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int xcd = blockIdx.x & (kSegments - 1);
  const int npairs = (nb + 1) >> 1;
  const bool dense = L.counts == nullptr;
  const bool pairs = dense || L.kind == kUnitPair;

  if (BLK < C::KB) {  // padding keys of both stages stay zero: the loads never write them
    for (int e = tid * 4; e < C::K_BYTES + C::V_BYTES; e += C::THREADS * 4) {
      *reinterpret_cast<uint32_t*>(stage0 + e) = 0u;
      *reinterpret_cast<uint32_t*>(stage1 + e) = 0u;
    }
  }

  // Per-lane byte offsets of this wave's direct-load pieces within a K block and a
  // V^T block (the LDS side is the wave's 1 KB slice; lane i lands at +16 i).
  int k_src[C::K_PER_WAVE], v_src[C::V_PER_WAVE];
#pragma unroll
  for (int u = 0; u < C::K_PER_WAVE; ++u) {
    const int at = (wave * C::K_PER_WAVE + u) * 1024 + lane * 16;
    const int row = at / C::K_ROW, phys = (at % C::K_ROW) / 16;
    k_src[u] = row * C::K_ROW + ((phys ^ k_swz<D>(row)) * 16);
  }
#pragma unroll
  for (int u = 0; u < C::V_PER_WAVE; ++u) {
    const int at = (wave * C::V_PER_WAVE + u) * 1024 + lane * 16;
    const int row = at / C::V_ROW, phys = (at % C::V_ROW) / 16;
    v_src[u] = row * C::V_ROW + ((phys ^ v_swz<C::KB>(row)) * 16);
  }
  // Per-lane LDS read offsets. S^T step s of key tile t reads K row krow(t, n),
  // logical chunk 4s + g; the t-dependent part of krow is lane-independent.
  int k_rd[C::DS];
  const int krow0 = 8 * (n >> 2) + (n & 3);
#pragma unroll
  for (int s = 0; s < C::DS; ++s) k_rd[s] = krow0 * C::K_ROW + (((4 * s + g) ^ k_swz<D>(krow0)) * 16);
  // The value product, channel tile t and key step u, reads V^T row 16t + n,
  // logical chunk 4u + g; the swizzle of rows 16t + n does not depend on t.
  int v_rd[C::KS];
#pragma unroll
  for (int u = 0; u < C::KS; ++u) v_rd[u] = C::K_BYTES + n * C::V_ROW + (((4 * u + g) ^ v_swz<C::KB>(n)) * 16);

  const int32_t* bounds = dense ? nullptr : L.sched;
  unsigned dead = 0;
  if (tid == 0) s_next = pull(counters, bounds, units, xcd, dead);
  __syncthreads();

  for (;;) {
    // wave-uniform values (readfirstlane) so that queue and list reads are scalar loads
    const int pos = __builtin_amdgcn_readfirstlane(s_next);
    if (pos < 0) break;
    int tile0, tile1, cnt;
    const_i32 plain = nullptr;     // single unit: plain ascending block ids
    const_i32 flagged = nullptr;   // pair unit: flagged union entries
    if (pairs) {
      const int bh = pos / npairs;
      const int pr = pos - bh * npairs;
      tile0 = bh * nb + 2 * pr;
      tile1 = 2 * pr + 1 < nb ? tile0 + 1 : -1;
      cnt = dense ? nb : as_const(L.pair_cnt)[pos];
      if (!dense) flagged = as_const(reinterpret_cast<const int32_t*>(L.pair_list) + (size_t)pos * nb);
    } else {
      tile0 = __builtin_amdgcn_readfirstlane(as_const(L.queue)[pos]);
      tile1 = -1;
      cnt = as_const(L.counts)[tile0];
      plain = as_const(L.kv_idx + (size_t)tile0 * nb);
    }
    const int bh = tile0 / nb;
    const int qb0 = tile0 - bh * nb;
    const bool two = tile1 >= 0;
    const uint32_t both = two ? (kInFirst | kInSecond) : kInFirst;
    // entry k of the unit's list: block id | membership flags
    auto entry = [&](int k) __attribute__((always_inline)) -> uint32_t {
      if (flagged) return (uint32_t)flagged[k];
      if (plain) return (uint32_t)plain[k] | kInFirst;
      return (uint32_t)k | both;
    };
    const char* kbase = reinterpret_cast<const char*>(kh + (size_t)bh * n_pad * D);
    const char* vbase = reinterpret_cast<const char*>(vt + (size_t)bh * nb * D * C::KB);

    auto issue = [&](char* st, uint32_t e) __attribute__((always_inline)) {
      const int j = (int)(e & kBlockMask);
      const char* ks = kbase + (size_t)j * BLK * C::K_ROW;
      const char* vs = vbase + (size_t)j * C::V_BYTES;
#pragma unroll
      for (int u = 0; u < C::K_PER_WAVE; ++u) load_lds16(ks + k_src[u], st + (wave * C::K_PER_WAVE + u) * 1024);
#pragma unroll
      for (int u = 0; u < C::V_PER_WAVE; ++u)
        load_lds16(vs + v_src[u], st + C::K_BYTES + (wave * C::V_PER_WAVE + u) * 1024);
    };

    // list entries: the current one, the next (whose loads are issued one block
    // ahead) and the one after (read one block ahead of its use)
    uint32_t e_cur = entry(0);
    uint32_t e_nxt = cnt > 1 ? entry(1) : 0u;
    issue(stage0, e_cur);
    // each member's query rows as the B operand of S^T = K Q^T: channels 32s + 8g .. +8
    bf16x8 qf[2][C::DS];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m == 1 && !two) break;
      const int qrow = (qb0 + m) * BLK + wave * 16 + n;
      const bf16_t* qsrc = qh + ((size_t)bh * n_pad + qrow) * D;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) qf[m][s] = *reinterpret_cast<const bf16x8*>(qsrc + 32 * s + 8 * g);
    }
    __syncthreads();  // every thread has read s_next
    if (tid == 0) s_next = pull(counters, bounds, units, xcd, dead);  // next unit, read after the loop
    wait_vm0();
    __syncthreads();

    f32x4 o[2][C::DT];
    float m_run[2], l_run[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int t = 0; t < C::DT; ++t) o[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[m] = -INFINITY;  // running max of this lane's row, base-2 scaled
      l_run[m] = 0.f;        // this lane's share of the row's running sum
    }

    // One key block for the members in `mask` (bit 0 first, bit 1 second).
    auto block = [&](const char* cur, char* nxt, int it, auto members) __attribute__((always_inline)) {
      constexpr int MASK = decltype(members)::value;
      const int j = (int)(e_cur & kBlockMask);
      const uint32_t e_after = it + 2 < cnt ? entry(it + 2) : 0u;
      if (it + 1 < cnt) issue(nxt, e_nxt);
      f32x4 sacc[2][C::KT];
#pragma unroll
      for (int t = 0; t < C::KT; ++t) {
        sacc[0][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        sacc[1][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int trow = 32 * (t >> 1) + 4 * (t & 1);  // lane-independent part of krow
#pragma unroll
        for (int s = 0; s < C::DS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + k_rd[s] + trow * C::K_ROW);
          if (MASK & 1) sacc[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][s], sacc[0][t], 0, 0, 0);
          if (MASK & 2) sacc[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][s], sacc[1][t], 0, 0, 0);
        }
      }
      // accumulator element r of tile t is key 32*(t/2) + 8g + 4*(t%2) + r of this block
      const int nj = min(BLK, N - j * BLK);
      bf16x8 pf[2][C::KS];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (!((MASK >> m) & 1)) continue;
        if (nj < C::KB) {
#pragma unroll
          for (int t = 0; t < C::KT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (32 * (t >> 1) + 8 * g + 4 * (t & 1) + r >= nj) sacc[m][t][r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < C::KT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[m][t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[m], mx * scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[m] - m_new);
        float rowsum = 0.f;
#pragma unroll
        for (int u = 0; u < C::KS; ++u) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[m][2 * u][r], scale_log2, -m_new));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[m][2 * u + 1][r], scale_log2, -m_new));
            rowsum += p0 + p1;
            pf[m][u][r] = (__bf16)p0;
            pf[m][u][4 + r] = (__bf16)p1;
          }
        }
        l_run[m] = l_run[m] * alpha + rowsum;
        if (__any(m_new != m_run[m])) {
#pragma unroll
          for (int t = 0; t < C::DT; ++t) o[m][t] *= alpha;
        }
        m_run[m] = m_new;
      }
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
#pragma unroll
        for (int u = 0; u < C::KS; ++u) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + v_rd[u] + 16 * t * C::V_ROW);
          if (MASK & 1) o[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[0][u], o[0][t], 0, 0, 0);
          if (MASK & 2) o[1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[1][u], o[1][t], 0, 0, 0);
        }
      }
      e_cur = e_nxt;
      e_nxt = e_after;
      wait_vm0();
      __syncthreads();
    };
    auto step = [&](const char* cur, char* nxt, int it) __attribute__((always_inline)) {
      const uint32_t f = e_cur & (kInFirst | kInSecond);
      if (f == (kInFirst | kInSecond))
        block(cur, nxt, it, std::integral_constant<int, 3>());
      else if (f == kInFirst)
        block(cur, nxt, it, std::integral_constant<int, 1>());
      else
        block(cur, nxt, it, std::integral_constant<int, 2>());
    };

    for (int it = 0; it < cnt; it += 2) {
      step(stage0, stage1, it);
      if (it + 1 < cnt) step(stage1, stage0, it + 1);
    }

#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m == 1 && !two) break;
      float l = l_run[m] + __shfl_xor(l_run[m], 16);
      l += __shfl_xor(l, 32);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int qrow = (qb0 + m) * BLK + wave * 16 + n;
      bf16_t* orow = oh + ((size_t)bh * n_pad + qrow) * D;
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(o[m][t][0] * inv) | ((uint32_t)f32_to_bf16(o[m][t][1] * inv) << 16);
        w.y = (uint32_t)f32_to_bf16(o[m][t][2] * inv) | ((uint32_t)f32_to_bf16(o[m][t][3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * t + 4 * g) = w;
      }
    }
  }

  // The last workgroup to finish resets the pull counters for the next launch.
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(&counters[kSegments], 1) == (int)gridDim.x - 1) {
      for (int s = 0; s <= kSegments; ++s) atomicExch(&counters[s], 0);
      __threadfence();
    }
  }
}

template <int D, int BLK>
hipError_t launch(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B, int H,
                  const AttnLists* lists, hipStream_t s) {
  using C = Cfg<D, BLK>;
  static int per_cu = 0;  // resident workgroups per CU for this instantiation
  if (per_cu == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<D, BLK>, C::THREADS, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
  }
  AttnLists L = lists ? *lists : AttnLists{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, kUnitPair};
  const int npairs = (c->nb + 1) / 2;
  const int units = (lists && L.kind == kUnitSingle) ? B * H * c->nb : B * H * npairs;
  const int grid = c->num_cus * per_cu;
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  attn_kernel<D, BLK><<<grid, C::THREADS, 0, s>>>(
      reinterpret_cast<const bf16_t*>(qh), reinterpret_cast<const bf16_t*>(kh), reinterpret_cast<const bf16_t*>(vt),
      reinterpret_cast<bf16_t*>(oh), L, c->counters, units, c->nb, c->n_pad, c->N, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B,
                            int H, int d, const AttnLists* lists, hipStream_t s) {
#define ABSH_ATTN(DD, BB) \
  if (d == DD && c->block == BB) return launch<DD, BB>(c, qh, kh, vt, oh, B, H, lists, s);
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
