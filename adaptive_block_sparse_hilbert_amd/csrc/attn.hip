// Block-sparse attention over retained key blocks (xllm-io review of FVAttn,
// "Block-Sparse Attention Execution"; alanhou.org explainer, "Core Mechanism":
// each head attends only to its selected KV blocks), for gfx950.
//
// One workgroup per tile (b, h, query block i), taken in queue order; one wave
// per 16 query rows. For every retained key block j, in ascending order:
//   S^T = K_j Q_i^T         16x16x32 bf16 MFMA, fp32 accumulate
//   online softmax          fp32, base-2 exponent, lazy rescale of O
//   O^T += V_j^T P^T        16x16x32 bf16 MFMA, P rounded to bf16
// K_j (rows of d) and V_j^T (rows of keys, written pre-transposed by the
// permute step) are staged in LDS, double-buffered, with the next block's global
// loads issued before the current block's MFMAs.
//
// Lane layout (wave of 64, n = lane % 16, g = lane / 16): for a 16x16x32 MFMA the
// A operand of lane (row m = n, group g) and the B operand of lane (column n,
// group g) carry the same eight k indices, and accumulator element r of lane
// (n, g) is (row 4g + r, column n). Computing S^T puts one query row per lane
// (column n) and lets the accumulator feed the value product directly: within
// each group of 32 keys the A rows of S^T are permuted so that lane group g ends
// up holding the eight consecutive keys 8g..8g+7 of that group, which is exactly
// the k slice its B operand of the value product needs.
#include "absh_internal.h"

namespace absh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D, int BLK>
struct Cfg {
  static constexpr int KB = BLK < 32 ? 32 : BLK;  // keys per staged block (a 16-key block is padded to 32)
  static constexpr int WAVES = BLK / 16;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KSTR = D + 8;   // LDS row stride of K, bf16 elements
  static constexpr int VSTR = KB + 8;  // LDS row stride of V^T
  static constexpr int K_ELEMS = KB * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int KT = KB / 16;  // 16-key tiles of S^T
  static constexpr int DT = D / 16;   // 16-channel tiles of O^T
  static constexpr int DS = D / 32;   // k steps of Q K^T
  static constexpr int KS = KB / 32;  // k steps of P V
  static constexpr int LOAD_K = BLK * D / 8;  // 16-byte pieces per K block
  static constexpr int LOAD_V = D * BLK / 8;  // 16-byte pieces per V^T block
  static constexpr int PK = (LOAD_K + THREADS - 1) / THREADS;
  static constexpr int PV = (LOAD_V + THREADS - 1) / THREADS;
};

// Global -> register half of the K / V^T staging: each thread takes PK (PV)
// 16-byte pieces of the block, strided by the workgroup size.
template <int D, int BLK>
__device__ __forceinline__ void global_load(const bf16_t* kbase, const bf16_t* vbase, int j, int tid,
                                            u32x4 (&pk)[Cfg<D, BLK>::PK], u32x4 (&pv)[Cfg<D, BLK>::PV]) {
  using C = Cfg<D, BLK>;
  const u32x4* ks = reinterpret_cast<const u32x4*>(kbase + (size_t)j * BLK * D);
  const u32x4* vs = reinterpret_cast<const u32x4*>(vbase + (size_t)j * D * BLK);
#pragma unroll
  for (int u = 0; u < C::PK; ++u) pk[u] = ks[tid + u * C::THREADS];
#pragma unroll
  for (int u = 0; u < C::PV; ++u) pv[u] = vs[tid + u * C::THREADS];
}

// Register -> LDS half: K rows of d (stride KSTR), V^T rows of keys (stride VSTR).
template <int D, int BLK>
__device__ __forceinline__ void lds_store(bf16_t* lds, int buf, int tid, const u32x4 (&pk)[Cfg<D, BLK>::PK],
                                          const u32x4 (&pv)[Cfg<D, BLK>::PV]) {
  using C = Cfg<D, BLK>;
  bf16_t* K = lds + buf * C::STAGE;
  bf16_t* V = K + C::K_ELEMS;
#pragma unroll
  for (int u = 0; u < C::PK; ++u) {
    const int idx = tid + u * C::THREADS;
    *reinterpret_cast<u32x4*>(K + (idx / (D / 8)) * C::KSTR + (idx % (D / 8)) * 8) = pk[u];
  }
#pragma unroll
  for (int u = 0; u < C::PV; ++u) {
    const int idx = tid + u * C::THREADS;
    *reinterpret_cast<u32x4*>(V + (idx / (BLK / 8)) * C::VSTR + (idx % (BLK / 8)) * 8) = pv[u];
  }
}

template <int D, int BLK>
__global__ __launch_bounds__((Cfg<D, BLK>::THREADS)) void attn_kernel(
    const bf16_t* __restrict__ qh, const bf16_t* __restrict__ kh, const bf16_t* __restrict__ vt,
    bf16_t* __restrict__ oh, const int32_t* __restrict__ queue, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ kv_idx, int nb, int n_pad, int N, float scale_log2) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  const int tile = queue ? queue[blockIdx.x] : (int)blockIdx.x;
  const int bh = tile / nb;
  const int qb = tile - bh * nb;
  const int cnt = counts ? counts[tile] : nb;
  const int32_t* list = counts ? kv_idx + (size_t)tile * nb : nullptr;
  const bf16_t* kbase = kh + (size_t)bh * n_pad * D;
  const bf16_t* vbase = vt + (size_t)bh * nb * D * BLK;

  // This lane's query row, as the B operand of S^T = K Q^T: channels 32s + 8g .. +8.
  const int qrow = qb * BLK + wave * 16 + n;
  const bf16_t* qsrc = qh + ((size_t)bh * n_pad + qrow) * D;
  bf16x8 qf[C::DS];
#pragma unroll
  for (int s = 0; s < C::DS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qsrc + 32 * s + 8 * g);

  if (BLK < C::KB) {  // zero the padding keys of both stages once; loads never touch them
    for (int e = tid; e < 2 * C::STAGE; e += C::THREADS) lds[e] = 0;
    __syncthreads();
  }

  static_assert(C::LOAD_K % C::THREADS == 0 && C::LOAD_V % C::THREADS == 0, "loads must tile the workgroup");
  u32x4 pk[C::PK], pv[C::PV];

  f32x4 o[C::DT];
#pragma unroll
  for (int t = 0; t < C::DT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of this lane's row, base-2 scaled
  float l_run = 0.f;        // this lane's share of the row's running sum

  if (cnt > 0) {
    global_load<D, BLK>(kbase, vbase, list ? list[0] : 0, tid, pk, pv);
    lds_store<D, BLK>(lds, 0, tid, pk, pv);
  }
  __syncthreads();

  for (int it = 0; it < cnt; ++it) {
    const int j = list ? list[it] : it;
    const int stage = it & 1;
    if (it + 1 < cnt) global_load<D, BLK>(kbase, vbase, list ? list[it + 1] : it + 1, tid, pk, pv);
    const bf16_t* K = lds + stage * C::STAGE;
    const bf16_t* V = K + C::K_ELEMS;

    f32x4 sacc[C::KT];
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int krow = 32 * (t >> 1) + 8 * (n >> 2) + 4 * (t & 1) + (n & 3);
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(K + krow * C::KSTR + 32 * s + 8 * g);
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
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(V + (16 * t + n) * C::VSTR + 32 * u + 8 * g);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[u], o[t], 0, 0, 0);
      }
    }
    if (it + 1 < cnt) lds_store<D, BLK>(lds, stage ^ 1, tid, pk, pv);
    __syncthreads();
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

template <int D, int BLK>
hipError_t launch(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B, int H,
                  const int32_t* queue, const int32_t* counts, const int32_t* kv_idx, hipStream_t s) {
  using C = Cfg<D, BLK>;
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  const unsigned grid = (unsigned)((uint64_t)B * H * c->nb);
  attn_kernel<D, BLK><<<grid, C::THREADS, 0, s>>>(
      reinterpret_cast<const bf16_t*>(qh), reinterpret_cast<const bf16_t*>(kh), reinterpret_cast<const bf16_t*>(vt),
      reinterpret_cast<bf16_t*>(oh), queue, counts, kv_idx, c->nb, c->n_pad, c->N, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt, void* oh, int B,
                            int H, int d, const int32_t* queue, const int32_t* counts, const int32_t* kv_idx,
                            hipStream_t s) {
#define ABSH_ATTN(DD, BB) \
  if (d == DD && c->block == BB) return launch<DD, BB>(c, qh, kh, vt, oh, B, H, queue, counts, kv_idx, s);
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
