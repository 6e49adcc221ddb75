// Block-sparse attention over retained key blocks (xllm-io review of FVAttn,
// "Block-Sparse Attention Execution"; alanhou.org explainer, "Core Mechanism":
// each head attends only to its selected KV blocks), for gfx950.
//
// Persistent kernel: one workgroup per (CU, occupancy slot). A workgroup pulls
// tiles (b, h, query block i) from the tile queue, one at a time, with an atomic
// counter per segment of the queue. The queue is cut into eight segments, one per
// XCD; a workgroup pulls from its own XCD's segment first and then steals from
// the others in turn. With one segment holding every tile this is plain list
// scheduling in queue order (the longest-first order when the queue is LPT);
// with the eight-way cost-balanced split of the queue it keeps the tiles that run
// together on one XCD (one L2) contiguous in Hilbert order, so they share K/V.
//
// Per tile, one wave per 16 query rows. For every retained key block j, in
// ascending order:
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
#include "absh_internal.h"

namespace absh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSegments = 8;  // XCDs of an MI355X: one queue segment each

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
__global__ __launch_bounds__((Cfg<D, BLK>::THREADS)) void attn_kernel(
    const bf16_t* __restrict__ qh, const bf16_t* __restrict__ kh, const bf16_t* __restrict__ vt,
    bf16_t* __restrict__ oh, const int32_t* __restrict__ queue, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ bounds, int32_t* __restrict__ counters,
    int tiles, int nb, int n_pad, int N, float scale_log2) {
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

  unsigned dead = 0;
  if (tid == 0) s_next = pull(counters, bounds, tiles, xcd, dead);
  __syncthreads();

  for (;;) {
    // wave-uniform values (readfirstlane) so that queue and list reads are scalar loads
    const int pos = __builtin_amdgcn_readfirstlane(s_next);
    if (pos < 0) break;
    const int tile = __builtin_amdgcn_readfirstlane(queue ? as_const(queue)[pos] : pos);
    const int bh = tile / nb;
    const int qb = tile - bh * nb;
    const int cnt = counts ? as_const(counts)[tile] : nb;
    const const_i32 list = counts ? as_const(kv_idx + (size_t)tile * nb) : nullptr;
    const char* kbase = reinterpret_cast<const char*>(kh + (size_t)bh * n_pad * D);
    const char* vbase = reinterpret_cast<const char*>(vt + (size_t)bh * nb * D * C::KB);

    auto issue = [&](char* st, int j) {
      const char* ks = kbase + (size_t)j * BLK * C::K_ROW;
      const char* vs = vbase + (size_t)j * C::V_BYTES;
#pragma unroll
      for (int u = 0; u < C::K_PER_WAVE; ++u) load_lds16(ks + k_src[u], st + (wave * C::K_PER_WAVE + u) * 1024);
#pragma unroll
      for (int u = 0; u < C::V_PER_WAVE; ++u)
        load_lds16(vs + v_src[u], st + C::K_BYTES + (wave * C::V_PER_WAVE + u) * 1024);
    };

    // block ids: the current one, the next (whose loads are issued one block
    // ahead) and the one after (read one block ahead of its use)
    int j_cur = list ? list[0] : 0;
    int j_nxt = cnt > 1 ? (list ? list[1] : 1) : 0;
    issue(stage0, j_cur);
    // this lane's query row as the B operand of S^T = K Q^T: channels 32s + 8g .. +8
    const int qrow = qb * BLK + wave * 16 + n;
    const bf16_t* qsrc = qh + ((size_t)bh * n_pad + qrow) * D;
    bf16x8 qf[C::DS];
#pragma unroll
    for (int s = 0; s < C::DS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qsrc + 32 * s + 8 * g);
    __syncthreads();  // every thread has read s_next
    if (tid == 0) s_next = pull(counters, bounds, tiles, xcd, dead);  // next tile, read after the loop
    wait_vm0();
    __syncthreads();

    f32x4 o[C::DT];
#pragma unroll
    for (int t = 0; t < C::DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of this lane's row, base-2 scaled
    float l_run = 0.f;        // this lane's share of the row's running sum

    auto block = [&](const char* cur, char* nxt, int it) {
      const int j = j_cur;
      const int j_after = it + 2 < cnt ? (list ? list[it + 2] : it + 2) : 0;
      if (it + 1 < cnt) issue(nxt, j_nxt);
      f32x4 sacc[C::KT];
#pragma unroll
      for (int t = 0; t < C::KT; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int trow = 32 * (t >> 1) + 4 * (t & 1);  // lane-independent part of krow
#pragma unroll
        for (int s = 0; s < C::DS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + k_rd[s] + trow * C::K_ROW);
          sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[t], 0, 0, 0);
        }
      }
      // accumulator element r of tile t is key 32*(t/2) + 8g + 4*(t%2) + r of this block
      const int nj = min(BLK, N - j * BLK);
      if (nj < C::KB) {
#pragma unroll
        for (int t = 0; t < C::KT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (32 * (t >> 1) + 8 * g + 4 * (t & 1) + r >= nj) sacc[t][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < C::KT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[t][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);

      bf16x8 pf[C::KS];
      float rowsum = 0.f;
#pragma unroll
      for (int u = 0; u < C::KS; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * u][r], scale_log2, -m_new));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[2 * u + 1][r], scale_log2, -m_new));
          rowsum += p0 + p1;
          pf[u][r] = (__bf16)p0;
          pf[u][4 + r] = (__bf16)p1;
        }
      }
      l_run = l_run * alpha + rowsum;
      if (__any(m_new != m_run)) {
#pragma unroll
        for (int t = 0; t < C::DT; ++t) o[t] *= alpha;
      }
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
#pragma unroll
        for (int u = 0; u < C::KS; ++u) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(cur + v_rd[u] + 16 * t * C::V_ROW);
          o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[u], o[t], 0, 0, 0);
        }
      }
      j_cur = j_nxt;
      j_nxt = j_after;
      wait_vm0();
      __syncthreads();
    };

    for (int it = 0; it < cnt; it += 2) {
      block(stage0, stage1, it);
      if (it + 1 < cnt) block(stage1, stage0, it + 1);
    }

    float l = l_run + __shfl_xor(l_run, 16);
    l += __shfl_xor(l, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16_t* orow = oh + ((size_t)bh * n_pad + qrow) * D;
#pragma unroll
    for (int t = 0; t < C::DT; ++t) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16(o[t][0] * inv) | ((uint32_t)f32_to_bf16(o[t][1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16(o[t][2] * inv) | ((uint32_t)f32_to_bf16(o[t][3] * inv) << 16);
      *reinterpret_cast<uint2*>(orow + 16 * t + 4 * g) = w;
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
                  const int32_t* queue, const int32_t* counts, const int32_t* kv_idx, const int32_t* bounds,
                  hipStream_t s) {
  using C = Cfg<D, BLK>;
  static int per_cu = 0;  // resident workgroups per CU for this instantiation
  if (per_cu == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<D, BLK>, C::THREADS, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
  }
  const int tiles = B * H * c->nb;
  const int grid = c->num_cus * per_cu;
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  attn_kernel<D, BLK><<<grid, C::THREADS, 0, s>>>(
      reinterpret_cast<const bf16_t*>(qh), reinterpret_cast<const bf16_t*>(kh), reinterpret_cast<const bf16_t*>(vt),
      reinterpret_cast<bf16_t*>(oh), queue, counts, kv_idx, bounds, c->counters, tiles, c->nb, c->n_pad, c->N,
      scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B,
                            int H, int d, const int32_t* queue, const int32_t* counts, const int32_t* kv_idx,
                            const int32_t* bounds, hipStream_t s) {
#define ABSH_ATTN(DD, BB) \
  if (d == DD && c->block == BB) return launch<DD, BB>(c, qh, kh, vt, oh, B, H, queue, counts, kv_idx, bounds, s);
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
