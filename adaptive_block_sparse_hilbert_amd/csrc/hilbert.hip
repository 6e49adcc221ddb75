// Hilbert permutation of the (T, Y, X) latent grid (xllm-io review of FVAttn,
// 3.1: blocks follow a Hilbert curve so that spatially adjacent tokens share
// blocks). Set-up only: it runs once per context.
//
// Every Hilbert index of the enclosing 2^m cube is mapped to its cell with the
// index-to-axes direction of Skilling's transform (J. Skilling, "Programming the
// Hilbert curve", AIP Conf. Proc. 707, 2004): de-interleave the index into the
// transposed form (bit l of axis i is index bit 3l + 2 - i, axes (t, y, x)),
// Gray-decode, then undo the per-level reflections and exchanges from the
// lowest level up. Cells outside the grid are dropped; the survivors keep index
// order, which is the Hilbert order of the grid.
#include "absh_internal.h"

namespace absh {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;
constexpr int kChunk = kThreads * kPerThread;

__device__ __forceinline__ void index_to_cell(uint32_t index, int m, uint32_t& t, uint32_t& y, uint32_t& x) {
  uint32_t a[3] = {0u, 0u, 0u};
  for (int l = 0; l < m; ++l)
    for (int i = 0; i < 3; ++i) a[i] |= ((index >> (3 * l + 2 - i)) & 1u) << l;
  // Gray decode across the axes: each axis takes the XOR of the ones before it;
  // axis 0 takes the last axis shifted down by one level.
  uint32_t carry = a[2] >> 1;
  a[2] ^= a[1];
  a[1] ^= a[0];
  a[0] ^= carry;
  // Undo the reflections (invert the lower bits of axis 0) and exchanges (swap
  // the lower bits of axis 0 and axis i), level by level from the bottom.
  for (uint32_t level = 2; level != (2u << (m - 1)); level <<= 1) {
    const uint32_t low = level - 1;
    for (int i = 2; i >= 0; --i) {
      if (a[i] & level) {
        a[0] ^= low;
      } else {
        const uint32_t diff = (a[0] ^ a[i]) & low;
        a[0] ^= diff;
        a[i] ^= diff;
      }
    }
  }
  t = a[0];
  y = a[1];
  x = a[2];
}

__device__ __forceinline__ bool in_grid(uint32_t index, int m, int T, int Y, int X, int32_t& rowmajor) {
  uint32_t t, y, x;
  index_to_cell(index, m, t, y, x);
  if (t >= (uint32_t)T || y >= (uint32_t)Y || x >= (uint32_t)X) return false;
  rowmajor = (int32_t)((t * (uint32_t)Y + y) * (uint32_t)X + x);
  return true;
}

// Pass 1: number of in-grid cells per chunk of kChunk consecutive indices.
__global__ __launch_bounds__(kThreads) void count_kernel(int m, int T, int Y, int X, uint64_t total,
                                                         int32_t* chunk_counts) {
  __shared__ int32_t partial[kThreads / 64];
  const uint64_t base = (uint64_t)blockIdx.x * kChunk + (uint64_t)threadIdx.x * kPerThread;
  int mine = 0;
  for (int e = 0; e < kPerThread; ++e) {
    const uint64_t idx = base + e;
    int32_t rm;
    if (idx < total && in_grid((uint32_t)idx, m, T, Y, X, rm)) ++mine;
  }
  for (int off = 32; off > 0; off >>= 1) mine += __shfl_xor(mine, off);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kThreads / 64; ++w) s += partial[w];
    chunk_counts[blockIdx.x] = s;
  }
}

// Pass 2: exclusive scan of the chunk counts in place (one workgroup).
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* chunk_counts, int chunks) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < chunks; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < chunks ? chunk_counts[i] : 0;
    buf[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < chunks) chunk_counts[i] = carry + buf[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
}

// Pass 3: rank in-grid cells in index order and scatter perm / inv.
__global__ __launch_bounds__(kThreads) void scatter_kernel(int m, int T, int Y, int X, uint64_t total,
                                                           const int32_t* chunk_offsets, int32_t* perm,
                                                           int32_t* inv) {
  __shared__ int32_t scan[kThreads];
  const uint64_t base = (uint64_t)blockIdx.x * kChunk + (uint64_t)threadIdx.x * kPerThread;
  int32_t rm[kPerThread];
  unsigned flags = 0;
  int mine = 0;
  for (int e = 0; e < kPerThread; ++e) {
    const uint64_t idx = base + e;
    if (idx < total && in_grid((uint32_t)idx, m, T, Y, X, rm[e])) {
      flags |= 1u << e;
      ++mine;
    }
  }
  scan[threadIdx.x] = mine;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  int pos = chunk_offsets[blockIdx.x] + scan[threadIdx.x] - mine;
  for (int e = 0; e < kPerThread; ++e) {
    if (flags & (1u << e)) {
      perm[pos] = rm[e];
      inv[rm[e]] = pos;
      ++pos;
    }
  }
}

}  // namespace

hipError_t launch_hilbert_perm(const absh_ctx* c, int32_t* chunk_counts, int chunks, hipStream_t s) {
  const uint64_t total = 1ull << (3 * c->m);
  count_kernel<<<chunks, kThreads, 0, s>>>(c->m, c->T, c->Y, c->X, total, chunk_counts);
  scan_kernel<<<1, 1024, 0, s>>>(chunk_counts, chunks);
  scatter_kernel<<<chunks, kThreads, 0, s>>>(c->m, c->T, c->Y, c->X, total, chunk_counts, c->perm, c->inv);
  return hipGetLastError();
}

int hilbert_chunks(int m) {
  const uint64_t total = 1ull << (3 * m);
  return (int)((total + kChunk - 1) / kChunk);
}

}  // namespace absh
