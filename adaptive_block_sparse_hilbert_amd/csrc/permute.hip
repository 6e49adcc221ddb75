// Gather between grid order and Hilbert order (the reordering half of the
// xllm-io review's Stage 1, "Hilbert curve block reordering").
//
// All three kernels move whole 16-byte pieces of rows, so every wave reads and
// writes contiguous runs of at least d*2 bytes (one token's row of one head).
#include "absh_internal.h"

namespace absh {
namespace {

constexpr int kThreads = 256;

struct alignas(16) Pack8 {
  uint32_t w[4];
};

__device__ __forceinline__ Pack8 load8(const void* base, size_t elem, int is_f32) {
  Pack8 out;
  if (is_f32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    out.w[0] = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    out.w[1] = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    out.w[2] = (uint32_t)f32_to_bf16(b.x) | ((uint32_t)f32_to_bf16(b.y) << 16);
    out.w[3] = (uint32_t)f32_to_bf16(b.z) | ((uint32_t)f32_to_bf16(b.w) << 16);
  } else {
    out = *reinterpret_cast<const Pack8*>(reinterpret_cast<const bf16_t*>(base) + elem);
  }
  return out;
}

// xh[b, h, r, :] = x[b, perm[r], h, :] for r < N, zero for N <= r < n_pad.
// One thread per 8 output elements; consecutive threads cover one row, then the
// next Hilbert position of the same head.
__global__ __launch_bounds__(kThreads) void gather_rows(const void* __restrict__ x, int is_f32,
                                                        bf16_t* __restrict__ xh, const int32_t* __restrict__ perm,
                                                        int N, int n_pad, int H, int d, uint64_t pieces) {
  const uint64_t id = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= pieces) return;
  const int per_row = d >> 3;
  const int e = (int)(id % per_row);
  const uint64_t row = id / per_row;          // (b*H + h)*n_pad + r
  const int r = (int)(row % n_pad);
  const uint64_t bh = row / n_pad;
  const int h = (int)(bh % H);
  const uint64_t b = bh / H;
  Pack8 v = {{0u, 0u, 0u, 0u}};
  if (r < N) v = load8(x, ((b * N + perm[r]) * H + h) * d + (size_t)e * 8, is_f32);
  *reinterpret_cast<Pack8*>(xh + row * d + (size_t)e * 8) = v;
}

// The same gather with float rows out: bf16 inputs widen exactly, float inputs
// are copied unchanged (routing from float queries and keys).
__global__ __launch_bounds__(kThreads) void gather_rows_f32(const void* __restrict__ x, int is_f32,
                                                            float* __restrict__ xh, const int32_t* __restrict__ perm,
                                                            int N, int n_pad, int H, int d, uint64_t pieces) {
  const uint64_t id = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= pieces) return;
  const int per_row = d >> 2;
  const int e = (int)(id % per_row);
  const uint64_t row = id / per_row;  // (b*H + h)*n_pad + r
  const int r = (int)(row % n_pad);
  const uint64_t bh = row / n_pad;
  const int h = (int)(bh % H);
  const uint64_t b = bh / H;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r < N) {
    const size_t elem = ((b * N + perm[r]) * H + h) * d + (size_t)e * 4;
    if (is_f32) {
      v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + elem);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(x) + elem);
      v = make_float4(bf16_to_f32((bf16_t)(w.x & 0xFFFFu)), bf16_to_f32((bf16_t)(w.x >> 16)),
                      bf16_to_f32((bf16_t)(w.y & 0xFFFFu)), bf16_to_f32((bf16_t)(w.y >> 16)));
    }
  }
  *reinterpret_cast<float4*>(xh + row * d + (size_t)e * 4) = v;
}

// vt[b, h, j, c, k] = x[b, perm[j*blk + k], h, c] for k < blk, with KB = vt_keys(blk)
// keys per block (keys blk..KB-1 and pad tokens are zero): one workgroup per
// (b, h, j) stages the block's rows in LDS and writes them back transposed.
template <int D, int BLK>
__global__ __launch_bounds__(kThreads) void gather_vt(const void* __restrict__ x, int is_f32,
                                                      bf16_t* __restrict__ vt, const int32_t* __restrict__ perm,
                                                      int N, int nb, int H) {
  constexpr int KB = vt_keys(BLK);
  constexpr int kStride = KB + 2;  // keys per LDS row (+2 breaks bank aliasing of the column writes)
  __shared__ bf16_t tile[D * kStride];
  if (KB > BLK) {
    for (int e = threadIdx.x; e < D * kStride; e += kThreads) tile[e] = 0;
    __syncthreads();
  }
  const int j = blockIdx.x % nb;
  const uint64_t bh = blockIdx.x / nb;
  const int h = (int)(bh % H);
  const uint64_t b = bh / H;
  // Load: piece p = (key k, 8 channels starting at c8*8).
  for (int p = threadIdx.x; p < BLK * (D / 8); p += kThreads) {
    const int k = p / (D / 8);
    const int c8 = p % (D / 8);
    const int r = j * BLK + k;
    Pack8 v = {{0u, 0u, 0u, 0u}};
    if (r < N) v = load8(x, ((b * N + perm[r]) * H + h) * D + (size_t)c8 * 8, is_f32);
    const bf16_t* vv = reinterpret_cast<const bf16_t*>(&v);
    for (int q = 0; q < 8; ++q) tile[(c8 * 8 + q) * kStride + k] = vv[q];
  }
  __syncthreads();
  // Store: piece p = (channel c, 8 keys starting at k8*8).
  bf16_t* out = vt + (bh * nb + j) * (size_t)(D * KB);
  for (int p = threadIdx.x; p < D * (KB / 8); p += kThreads) {
    const int c = p / (KB / 8);
    const int k8 = p % (KB / 8);
    Pack8 v;
    bf16_t* vv = reinterpret_cast<bf16_t*>(&v);
    for (int q = 0; q < 8; ++q) vv[q] = tile[c * kStride + k8 * 8 + q];
    *reinterpret_cast<Pack8*>(out + (size_t)c * KB + k8 * 8) = v;
  }
}

// The rows gather fused with the block means of the rows it writes (the pooling
// of the xllm-io review's Stage 1, done in the same pass over x): one workgroup
// per (b, h, block j). Thread t moves the 16-byte output piece t % PIECES of rows
// t / PIECES, + ROWS, ... of the block and sums those of its rows that hold tokens
// in float64; the row groups' partial sums are then added in order and divided by
// the block's token count in float64, rounded once to float32. That is the
// order of the pooling kernel over the same rows, so the means are bit-identical
// to pooling xh afterwards. TO: bf16_t (bf16 rows) or float (float32 rows).
template <int D, typename TO>
__global__ __launch_bounds__(kThreads) void gather_pool(const void* __restrict__ x, int is_f32, TO* __restrict__ xh,
                                                        float* __restrict__ xbar, const int32_t* __restrict__ perm,
                                                        int N, int n_pad, int nb, int blk, int H) {
  constexpr int EPP = 16 / (int)sizeof(TO);  // channels per 16-byte output piece
  constexpr int PIECES = D / EPP;
  constexpr int ROWS = kThreads / PIECES;
  __shared__ double part[ROWS][D + 1];
  const int j = blockIdx.x % nb;
  const uint64_t bh = blockIdx.x / nb;
  const int h = (int)(bh % H);
  const uint64_t b = bh / H;
  const int piece = threadIdx.x % PIECES;
  const int r0 = threadIdx.x / PIECES;
  const int n = min(blk, N - j * blk);  // rows of the block that hold tokens
  double acc[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
  for (int r = r0; r < blk; r += ROWS) {
    const int row = j * blk + r;  // Hilbert position
    const size_t src = ((b * N + (r < n ? perm[row] : 0)) * H + h) * D + (size_t)piece * EPP;
    TO* dst = xh + (bh * n_pad + row) * D + (size_t)piece * EPP;
    if constexpr (sizeof(TO) == 2) {
      Pack8 v = {{0u, 0u, 0u, 0u}};
      if (r < n) {
        v = load8(x, src, is_f32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)bf16_to_f32((bf16_t)(v.w[e] & 0xFFFFu));
          acc[2 * e + 1] += (double)bf16_to_f32((bf16_t)(v.w[e] >> 16));
        }
      }
      *reinterpret_cast<Pack8*>(dst) = v;
    } else {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < n) {
        if (is_f32) {
          v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + src);
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(x) + src);
          v = make_float4(bf16_to_f32((bf16_t)(w.x & 0xFFFFu)), bf16_to_f32((bf16_t)(w.x >> 16)),
                          bf16_to_f32((bf16_t)(w.y & 0xFFFFu)), bf16_to_f32((bf16_t)(w.y >> 16)));
        }
        acc[0] += (double)v.x;
        acc[1] += (double)v.y;
        acc[2] += (double)v.z;
        acc[3] += (double)v.w;
      }
      *reinterpret_cast<float4*>(dst) = v;
    }
  }
#pragma unroll
  for (int e = 0; e < EPP; ++e) part[r0][piece * EPP + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += kThreads) {
    double sum = 0.0;
    for (int r = 0; r < ROWS; ++r) sum += part[r][c];
    xbar[(bh * nb + j) * D + c] = __double2float_rn(sum / (double)n);
  }
}

// o[b, n, h, :] = oh[b, h, inv[n], :]: one thread per 8 output elements.
__global__ __launch_bounds__(kThreads) void scatter_rows(const bf16_t* __restrict__ oh, bf16_t* __restrict__ o,
                                                         const int32_t* __restrict__ inv, int N, int n_pad, int H,
                                                         int d, uint64_t pieces) {
  const uint64_t id = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= pieces) return;
  const int per_row = d >> 3;
  const int e = (int)(id % per_row);
  const uint64_t row = id / per_row;  // (b*N + n)*H + h
  const int h = (int)(row % H);
  const uint64_t bn = row / H;
  const int n = (int)(bn % N);
  const uint64_t b = bn / N;
  const Pack8 v = *reinterpret_cast<const Pack8*>(oh + ((b * H + h) * n_pad + inv[n]) * d + (size_t)e * 8);
  *reinterpret_cast<Pack8*>(o + row * d + (size_t)e * 8) = v;
}

template <int D, int BLK>
void launch_vt(const void* x, int is_f32, bf16_t* vt, const int32_t* perm, int N, int nb, int H, int B,
               hipStream_t s) {
  gather_vt<D, BLK><<<(unsigned)((uint64_t)B * H * nb), kThreads, 0, s>>>(x, is_f32, vt, perm, N, nb, H);
}

}  // namespace

hipError_t launch_permute(const absh_ctx* c, const void* x, int x_is_f32, void* xh, int B, int H, int d,
                          int layout, hipStream_t s) {
  bf16_t* out = reinterpret_cast<bf16_t*>(xh);
  if (layout == ABSH_ROWS_F32) {
    const uint64_t pieces = (uint64_t)B * H * c->n_pad * (d / 4);
    const unsigned grid = (unsigned)((pieces + kThreads - 1) / kThreads);
    gather_rows_f32<<<grid, kThreads, 0, s>>>(x, x_is_f32, reinterpret_cast<float*>(xh), c->perm, c->N, c->n_pad,
                                              H, d, pieces);
    return hipGetLastError();
  }
  if (layout == ABSH_ROWS) {
    const uint64_t pieces = (uint64_t)B * H * c->n_pad * (d / 8);
    const unsigned grid = (unsigned)((pieces + kThreads - 1) / kThreads);
    gather_rows<<<grid, kThreads, 0, s>>>(x, x_is_f32, out, c->perm, c->N, c->n_pad, H, d, pieces);
    return hipGetLastError();
  }
#define ABSH_VT_CASE(DD, BB)                                                  \
  if (d == DD && c->block == BB) {                                            \
    launch_vt<DD, BB>(x, x_is_f32, out, c->perm, c->N, c->nb, H, B, s);       \
    return hipGetLastError();                                                 \
  }
  ABSH_VT_CASE(64, 16)
  ABSH_VT_CASE(64, 64)
  ABSH_VT_CASE(64, 128)
  ABSH_VT_CASE(128, 16)
  ABSH_VT_CASE(128, 64)
  ABSH_VT_CASE(128, 128)
#undef ABSH_VT_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_permute_pool(const absh_ctx* c, const void* x, int x_is_f32, void* xh, float* xbar, int B, int H,
                               int d, int layout, hipStream_t s) {
  const unsigned grid = (unsigned)((uint64_t)B * H * c->nb);
  const bool f32 = layout == ABSH_ROWS_F32;
  if (layout != ABSH_ROWS && !f32) return hipErrorInvalidValue;
#define ABSH_GP(DD, TT)                                                                                       \
  gather_pool<DD, TT><<<grid, kThreads, 0, s>>>(x, x_is_f32, reinterpret_cast<TT*>(xh), xbar, c->perm, c->N, \
                                                c->n_pad, c->nb, c->block, H)
  if (d == 64 && !f32)
    ABSH_GP(64, bf16_t);
  else if (d == 128 && !f32)
    ABSH_GP(128, bf16_t);
  else if (d == 64)
    ABSH_GP(64, float);
  else if (d == 128)
    ABSH_GP(128, float);
  else
    return hipErrorInvalidValue;
#undef ABSH_GP
  return hipGetLastError();
}

hipError_t launch_unpermute(const absh_ctx* c, const void* oh, void* o, int B, int H, int d, hipStream_t s) {
  const uint64_t pieces = (uint64_t)B * c->N * H * (d / 8);
  const unsigned grid = (unsigned)((pieces + kThreads - 1) / kThreads);
  scatter_rows<<<grid, kThreads, 0, s>>>(reinterpret_cast<const bf16_t*>(oh), reinterpret_cast<bf16_t*>(o), c->inv,
                                         c->N, c->n_pad, H, d, pieces);
  return hipGetLastError();
}

}  // namespace absh
