// Stage-1 routing kernels (xllm-io review of FVAttn, section 三 Stage 1 and 3.1;
// alanhou.org explainer of FVAttn, "Key Concepts": Top-p with a Top-k floor),
// the Eq. 1 workloads, and the one-GPU runtime stages: a slack fill over tiles
// (the review's SASA steps, read for one GPU) and a longest-first tile queue
// (the review's RLB, read for one GPU).
//
// Precision: a routing decision is an integer decided by floating point, so it
// is taken in a precision the checker can reproduce exactly: block means are
// float64 sums of bf16 rows (exact) divided in float64 and rounded to float32;
// scores are float64 dot products rounded to float32; the softmax, cumulative
// sums and the comparison with p are float64.
#include <math.h>

#include "absh_internal.h"

namespace absh {
namespace {

// ------------------------------------------------------------------ pooling

// xbar[bh, j, c] = (sum over the block's true rows of xh[bh, r, c]) / n_j.
// One workgroup per (bh, j). Each thread reads 16-byte pieces (8 bf16 or 4 float
// channels) of every ROWS-th row and keeps float64 partial sums; the partials of
// a channel are then added in LDS. Sums of bf16 values in float64 are exact for
// any operands whose exponents lie within 45 binades of each other, so the order
// of the additions does not change the result (float values: within 29 binades).
constexpr int kPoolThreads = 256;

template <int D, typename T>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const T* __restrict__ xh, float* __restrict__ xbar,
                                                            int N, int n_pad, int nb, int blk) {
  constexpr int EPP = 16 / (int)sizeof(T);  // channels per 16-byte piece
  constexpr int PIECES = D / EPP;
  constexpr int ROWS = kPoolThreads / PIECES;
  __shared__ double part[ROWS][D + 1];
  const int j = blockIdx.x % nb;
  const uint64_t bh = blockIdx.x / nb;
  const int piece = threadIdx.x % PIECES;
  const int r0 = threadIdx.x / PIECES;
  const int n = min(blk, N - j * blk);
  const T* src = xh + (bh * n_pad + (size_t)j * blk) * D + piece * EPP;
  double acc[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
#pragma unroll 4
  for (int r = r0; r < n; r += ROWS) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + (size_t)r * D);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_to_f32((bf16_t)(u[e] & 0xFFFFu));
        acc[2 * e + 1] += (double)bf16_to_f32((bf16_t)(u[e] >> 16));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(u[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPP; ++e) part[r0][piece * EPP + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += kPoolThreads) {
    double sum = 0.0;
    for (int r = 0; r < ROWS; ++r) sum += part[r][c];
    xbar[(bh * nb + j) * D + c] = __double2float_rn(sum / (double)n);
  }
}

// ------------------------------------------------------------------ scores

// S[bh, i, j] = float32( sum_c double(qbar[bh,i,c]) * double(kbar[bh,j,c]) / sqrt_d ).
// 128 x 128 output tile per workgroup; wave w takes the 64 x 64 quadrant (w / 2, w % 2)
// as 4 x 4 tiles of the float64 MFMA D(16x16) += A(16x4) B(4x16), with A = block means
// of q (rows i, channels) and B = block means of k (channels, columns j). Channels
// are staged in LDS sixteen at a time as float64. Each float32 product is exact in
// float64; only the order of the additions is the kernel's.
// MFMA operand layout (lane l): A[l % 16][l / 16], B[l / 16][l % 16]; result element
// v of lane l is D[4 v + l / 16][l % 16].
constexpr int kTile = 128;
constexpr int kDepth = 16;
constexpr int kLdsRow = kTile + 4;  // doubles per staged channel (padding spreads the four lane groups)

typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                     float* __restrict__ S, int nb, int d, double sqrt_d,
                                                     int tiles_per_side) {
  __shared__ double qs[kDepth][kLdsRow];
  __shared__ double ks[kDepth][kLdsRow];
  const int per_head = tiles_per_side * tiles_per_side;
  const uint64_t bh = blockIdx.x / per_head;
  const int tile = blockIdx.x % per_head;
  const int i0 = (tile / tiles_per_side) * kTile;
  const int j0 = (tile % tiles_per_side) * kTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;
  const int r16 = lane & 15, k4 = lane >> 4;
  const float* qb = qbar + bh * nb * (size_t)d;
  const float* kb = kbar + bh * nb * (size_t)d;
  f64x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
  // loader: thread -> (row lr, 8 channels at lc)
  const int lr = threadIdx.x / 2, lc = (threadIdx.x % 2) * 8;
  for (int c0 = 0; c0 < d; c0 += kDepth) {
    float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0, k0 = q0, k1 = q0;
    if (i0 + lr < nb) {
      const float4* p = reinterpret_cast<const float4*>(qb + (size_t)(i0 + lr) * d + c0 + lc);
      q0 = p[0];
      q1 = p[1];
    }
    if (j0 + lr < nb) {
      const float4* p = reinterpret_cast<const float4*>(kb + (size_t)(j0 + lr) * d + c0 + lc);
      k0 = p[0];
      k1 = p[1];
    }
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qs[lc + e][lr] = qv[e];
      ks[lc + e][lr] = kv[e];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kDepth; c += 4) {
      double a[4], b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = qs[c + k4][wr + 16 * t + r16];
        b[t] = ks[c + k4][wc + 16 * t + r16];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[u], b[v], acc[u][v], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + wr + 16 * u + 4 * e + k4;
      if (i >= nb) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = j0 + wc + 16 * v + r16;
        if (j < nb) S[(bh * nb + i) * (size_t)nb + j] = __double2float_rn(acc[u][v][e] / sqrt_d);
      }
    }
}

// ------------------------------------------------------------------ Top-p select

// Reductions over the wave as a butterfly on the DPP and lane-swap paths, with no
// LDS round trip: partners 1 and 2 apart within each quad, then the mirrors of 8
// and 16 lanes (each half meets the other half's equal partial), then rows 16 and
// half-waves 32 apart by the gfx950 lane swaps. At every step the two partners
// combine the same two values in the same order, so every lane ends with the same
// bits. The wave must be fully active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;  // lane i of each 8 <- lane 7 - i
constexpr int kMirror = 0x140;      // lane i of each 16 <- lane 15 - i

template <typename T>
struct LaneBits;
template <>
struct LaneBits<float> {
  static constexpr int W = 1;
  __device__ static void split(float v, uint32_t* u) { u[0] = __float_as_uint(v); }
  __device__ static float join(const uint32_t* u) { return __uint_as_float(u[0]); }
};
template <>
struct LaneBits<double> {
  static constexpr int W = 2;
  __device__ static void split(double v, uint32_t* u) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    u[0] = (uint32_t)b;
    u[1] = (uint32_t)(b >> 32);
  }
  __device__ static double join(const uint32_t* u) {
    return __longlong_as_double((long long)(((uint64_t)u[1] << 32) | u[0]));
  }
};
template <>
struct LaneBits<uint64_t> {
  static constexpr int W = 2;
  __device__ static void split(uint64_t v, uint32_t* u) {
    u[0] = (uint32_t)v;
    u[1] = (uint32_t)(v >> 32);
  }
  __device__ static uint64_t join(const uint32_t* u) { return ((uint64_t)u[1] << 32) | u[0]; }
};

template <int CTRL, typename T>
__device__ __forceinline__ T dpp_partner(T v) {
  using LB = LaneBits<T>;
  uint32_t u[LB::W];
  LB::split(v, u);
#pragma unroll
  for (int w = 0; w < LB::W; ++w) u[w] = dpp_move<CTRL>(u[w]);
  return LB::join(u);
}
// Combine with the lane 16 (R16) or 32 apart: the swap hands each lane its own
// value and its partner's, ordered by lane group, so both partners see (a, b).
template <bool R16, typename T, typename Op>
__device__ __forceinline__ T swap_combine(T v, Op op) {
  using LB = LaneBits<T>;
  uint32_t u[LB::W], a[LB::W], b[LB::W];
  LB::split(v, u);
#pragma unroll
  for (int w = 0; w < LB::W; ++w) {
    const auto sw = R16 ? __builtin_amdgcn_permlane16_swap(u[w], u[w], false, false)
                        : __builtin_amdgcn_permlane32_swap(u[w], u[w], false, false);
    a[w] = sw[0];
    b[w] = sw[1];
  }
  return op(LB::join(a), LB::join(b));
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_partner<kQuadXor1>(v));
  v = op(v, dpp_partner<kQuadXor2>(v));
  v = op(v, dpp_partner<kHalfMirror>(v));
  v = op(v, dpp_partner<kMirror>(v));
  v = swap_combine<true>(v, op);
  return swap_combine<false>(v, op);
}
__device__ __forceinline__ double wave_sum(double v) {
  return wave_reduce(v, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  return wave_reduce(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }
__device__ __forceinline__ uint64_t lanes_below(int lane) { return lane == 0 ? 0ull : (~0ull >> (64 - lane)); }

// Monotone map of a finite float to uint32 (a < b  <=>  key(a) < key(b)).
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per tile row. Lane l holds key blocks j = l + 64 t, t < J.
//
// The importance order is probability descending, ties by smaller id. A block's
// probability is exp(s_j - max s) / Z, so for blocks of non-zero probability the
// order is the order of the scores; blocks whose probability underflows to zero
// all tie. Each block gets a 32-bit key, larger = more important: 0 for zero
// probability, else ordered_bits(s_j) + 1. Equal keys then mean equal
// probabilities, and ties resolve by block id exactly as in the definition.
//
// Top-p: the largest key tau whose upper set {key >= tau} carries mass >= p is
// found bit by bit from the top; the count is #{key > tau} plus as many of the
// tied blocks at tau (each of the same probability) as the running sum needs to
// reach p. The floor then asks for count' = max(c, min(k, nb)) blocks, and the
// retained set is the top count' blocks, found the same way by counting.
// wanted counts up to this take the arg-max route
constexpr int kArgmaxWant = 16;

// RS: re-selection to the counts in `target` (keys only), as its own instance.
// One wave, the scores of tile `row` at srow[0 .. nb - 1] (in LDS).
// Returns the retained blocks as bit t for block lane + 64 t (0 for a re-selection
// row that needs no new block).
template <int J, bool RS>
__device__ __forceinline__ uint32_t select_row(const float* srow, int row, int nb, double p, int k_floor,
                                           int order_depth, const int32_t* __restrict__ target,
                                           int32_t* __restrict__ counts, int16_t* __restrict__ kv_idx,
                                           int16_t* __restrict__ order) {
  const int lane = threadIdx.x & 63;
  int want = 0;
  if (RS) {
    want = target[row];
    if (want <= counts[row]) return 0u;
  }
  float s[J];
  bool valid[J];
#pragma unroll
  for (int t = 0; t < J; ++t) {
    const int j = lane + 64 * t;
    valid[t] = j < nb;
    s[t] = valid[t] ? srow[j] : -INFINITY;
  }
  float smax = -INFINITY;
#pragma unroll
  for (int t = 0; t < J; ++t) smax = fmaxf(smax, s[t]);
  smax = wave_max(smax);
  // Probabilities. The float64 softmax is the definition; a float32 one (the
  // exponent s - smax in float32, v_exp_f32, the row sum per lane then across the
  // wave) carries a relative error below 2e-6 per block plus 1.8e-7 times
  // |s - smax|, so any mass it sums is within 5.4e-6 of the exact one (the mean of
  // |s - smax| under the softmax is at most ln nb < 7.7). Decisions further than
  // kBand from p are therefore the float64 ones; closer ones, and ties at the
  // threshold, take the float64 probabilities, computed for the row on first need.
  // A block's key is 0 only where its float64 probability underflows to 0, which
  // cannot happen within 700 of the row's max (exp > 9.8e-305, row sum <= 2048);
  // rows with a block further down take the float64 path from the start.
  constexpr double kBand = 2e-5;
  double P[J];
  float P32[J];
  uint32_t key[J];
  bool have64 = false;
  auto exact = [&]() __attribute__((always_inline)) {
    double z = 0.0;
#pragma unroll
    for (int t = 0; t < J; ++t) {
      P[t] = valid[t] ? exp((double)s[t] - (double)smax) : 0.0;
      z += P[t];
    }
    z = wave_sum(z);
#pragma unroll
    for (int t = 0; t < J; ++t) P[t] = P[t] / z;
    have64 = true;
  };
  bool far = false;
#pragma unroll
  for (int t = 0; t < J; ++t) far = far || (valid[t] && (double)s[t] - (double)smax <= -700.0);
  if (__any(far)) {
    exact();
#pragma unroll
    for (int t = 0; t < J; ++t) {
      key[t] = (valid[t] && P[t] != 0.0) ? ordered_bits(s[t]) + 1u : 0u;
      P32[t] = (float)P[t];
    }
  } else {
#pragma unroll
    for (int t = 0; t < J; ++t) key[t] = valid[t] ? ordered_bits(s[t]) + 1u : 0u;
    if (!RS) {  // a re-selection needs only the keys
      float z32 = 0.f;
#pragma unroll
      for (int t = 0; t < J; ++t) {
        P32[t] = valid[t] ? __builtin_amdgcn_exp2f((s[t] - smax) * 1.44269504f) : 0.f;
        z32 += P32[t];
      }
      const float inv = 1.f / wave_sum_f32(z32);
#pragma unroll
      for (int t = 0; t < J; ++t) P32[t] *= inv;
    }
  }

  // the Top-p threshold, when the count c came from it (then a count of exactly c
  // has the same threshold: every key above it and the first ties at it)
  uint32_t tau_p = 0;
  bool tau_p_set = false;
  // Both threshold searches below fix the bits of the answer from the top. After
  // a bit is fixed the answer lies in [tau, tau + 2^bit); the searches count the
  // keys at or above each candidate on the way, so they know how many keys that
  // interval holds, and when it holds one, that key is the answer (the property
  // holds at tau, hence at the one key above it in the interval, and fails at the
  // interval's end): the remaining steps would only spell it out bit by bit.
  int n_keys = 0;  // keys >= 1 (every key of a block with a non-zero probability)
#pragma unroll
  for (int t = 0; t < J; ++t) n_keys += popc64(__ballot(key[t] != 0u));
  // smallest key >= lo over the wave
  auto min_key_from = [&](uint32_t lo) __attribute__((always_inline)) -> uint32_t {
    uint64_t best = 0;
#pragma unroll
    for (int t = 0; t < J; ++t) {
      const uint64_t inv = (uint64_t)(~key[t]);
      best = key[t] >= lo && inv > best ? inv : best;
    }
    return ~(uint32_t)wave_max_u64(best);
  };
  if (!RS) {
    int c = nb;
    if (p < 1.0) {
      // each step: is the mass of {key >= cand} at least p?
      uint32_t tau = 0;
      int n_lo = n_keys, n_hi = 0;  // keys >= tau (tau >= 1 once set), keys >= the interval's end
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        float f32 = 0.f;
        int n_c = 0;
#pragma unroll
        for (int t = 0; t < J; ++t) {
          const bool ge = key[t] >= cand;
          f32 += ge ? P32[t] : 0.f;
          n_c += popc64(__ballot(ge));
        }
        const double m32 = (double)wave_sum_f32(f32);
        bool take = m32 >= p;
        if (fabs(m32 - p) <= kBand) {
          if (!have64) exact();
          double f = 0.0;
#pragma unroll
          for (int t = 0; t < J; ++t) f += key[t] >= cand ? P[t] : 0.0;
          take = wave_sum(f) >= p;
        }
        if (take) {
          tau = cand;
          n_lo = n_c;
        } else {
          n_hi = n_c;
        }
        if (n_lo - n_hi == 1 && tau != 0u) {
          tau = min_key_from(tau);
          break;
        }
      }
      int n_above = 0, n_at = 0;
      float f32 = 0.f;
#pragma unroll
      for (int t = 0; t < J; ++t) {
        const bool gt = valid[t] && key[t] > tau;
        const bool eq = valid[t] && key[t] == tau;
        f32 += (gt || eq) ? P32[t] : 0.f;
        n_above += popc64(__ballot(gt));
        n_at += popc64(__ballot(eq));
      }
      const double f_tau32 = (double)wave_sum_f32(f32);
      if (n_at == 1 && fabs(f_tau32 - p) > kBand) {
        // one block at the threshold: the count is n_above + 1 when the mass reaches p
        if (f_tau32 >= p) {
          c = n_above + 1;
          tau_p = tau;
          tau_p_set = true;
        }
      } else {
        if (!have64) exact();
        double above = 0.0, at = 0.0, f_tau = 0.0;
#pragma unroll
        for (int t = 0; t < J; ++t) {
          const bool gt = valid[t] && key[t] > tau;
          const bool eq = valid[t] && key[t] == tau;
          above += gt ? P[t] : 0.0;
          at = eq ? P[t] : at;
          f_tau += (gt || eq) ? P[t] : 0.0;
        }
        above = wave_sum(above);
        f_tau = wave_sum(f_tau);
        // every tied block has the same probability; take it from any lane holding one
        const uint64_t holders = __ballot(at != 0.0);
        const double tied = holders ? __shfl(at, __ffsll((long long)holders) - 1) : 0.0;
        if (f_tau >= p) {
          int m = 1;
          double run = above + tied;
          while (run < p && m < n_at) {
            run += tied;
            ++m;
          }
          c = n_above + m;
          tau_p = tau;
          tau_p_set = true;
        }
      }
    }
    want = max(c, min(k_floor, nb));
    tau_p_set = tau_p_set && want == c;
  }

  // Top-`want` blocks by (key desc, id asc), as bit t of `takebits` for block
  // lane + 64 t. A small `want` (the floor, a few slack blocks) takes the arg-max
  // of (key, -id) want times. Otherwise a count search on the key finds the
  // want-th key; when the floor did not raise the Top-p count the search would end
  // at the Top-p threshold (n_above < want <= n_above + n_at there), so it is skipped.
  uint32_t takebits = 0;
  if (!tau_p_set && want <= kArgmaxWant) {
    for (int r = 0; r < want; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int t = 0; t < J; ++t) {
        const uint64_t cand = ((uint64_t)key[t] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * t));
        best = (valid[t] && !((takebits >> t) & 1u) && cand > best) ? cand : best;
      }
      best = wave_max_u64(best);
      const int j = (int)(0xFFFFFFFFu - (uint32_t)best);
      if ((j & 63) == lane) takebits |= 1u << (j >> 6);
    }
  } else {
    uint32_t tau = tau_p_set ? tau_p : 0u;
    int n_lo = n_keys, n_hi = 0;
    for (int bit = 31; bit >= 0 && !tau_p_set; --bit) {
      const uint32_t cand = tau | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < J; ++t) cnt += popc64(__ballot(valid[t] && key[t] >= cand));
      if (cnt >= want) {
        tau = cand;
        n_lo = cnt;
      } else {
        n_hi = cnt;
      }
      if (n_lo - n_hi == 1 && tau != 0u) {
        tau = min_key_from(tau);
        break;
      }
    }
    int n_above = 0;
#pragma unroll
    for (int t = 0; t < J; ++t) n_above += popc64(__ballot(valid[t] && key[t] > tau));
    const int ties_needed = want - n_above;
    int ties_seen = 0;
    const uint64_t below = lanes_below(lane);
#pragma unroll
    for (int t = 0; t < J; ++t) {
      const bool gt = valid[t] && key[t] > tau;
      const bool eq = valid[t] && key[t] == tau;
      const uint64_t eq_mask = __ballot(eq);
      if (gt || (eq && ties_seen + popc64(eq_mask & below) < ties_needed)) takebits |= 1u << t;
      ties_seen += popc64(eq_mask);
    }
  }
  // the list in ascending block id
  int16_t* out = kv_idx + (size_t)row * nb;
  int written = 0;
  const uint64_t below = lanes_below(lane);
#pragma unroll
  for (int t = 0; t < J; ++t) {
    const bool take = (takebits >> t) & 1u;
    const uint64_t take_mask = __ballot(take);
    if (take) out[written + popc64(take_mask & below)] = (int16_t)(lane + 64 * t);
    written += popc64(take_mask);
  }
  if (lane == 0) counts[row] = want;

  // Importance-order prefix: repeated arg-max of (key, -id) over the blocks not yet taken.
  if (!RS && order_depth > 0) {
    uint32_t taken = 0;
    int16_t* ord = order + (size_t)row * order_depth;
    for (int r = 0; r < order_depth; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int t = 0; t < J; ++t) {
        if (valid[t] && !(taken & (1u << t))) {
          const uint64_t cand = ((uint64_t)key[t] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * t));
          best = cand > best ? cand : best;
        }
      }
      best = wave_max_u64(best);
      const int j = best ? (int)(0xFFFFFFFFu - (uint32_t)best) : -1;
      if (j >= 0 && (j & 63) == lane) taken |= 1u << (j >> 6);
      if (lane == 0) ord[r] = (int16_t)j;
    }
  }
  return takebits;
}

// Selection from scores in memory: one wave per tile row. The searches are
// latency-bound, so rows of up to 1,280 blocks are held to three waves per SIMD's
// worth of registers (wider rows would spill).
template <int J, bool RS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(J <= 20 ? 3 : 1))) void select_kernel(const float* __restrict__ S, int nb, int tiles, double p,
                                                     int k_floor, int order_depth,
                                                     const int32_t* __restrict__ target, int32_t* __restrict__ counts,
                                                     int16_t* __restrict__ kv_idx, int16_t* __restrict__ order) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= tiles) return;
  select_row<J, RS>(S + (size_t)row * nb, row, nb, p, k_floor, order_depth, target, counts, kv_idx, order);
}

// The first selection with the work units' union lists built in the same pass, for
// routing whose counts do not change afterwards (no slack fill, no rank stage). A
// workgroup takes 4 / M units of M neighbouring query blocks of one head (M = 4 or
// 2), one wave per member row. Each wave selects its row as select_kernel does and
// keeps the bit mask of its retained blocks; a unit's union is the OR of its
// members' masks, so its entries (block id | member m's flag << (28 + m)) come out
// in ascending block id: the list group_merge_kernel builds from the written lists.
// The member rows' searches take different numbers of steps, so the unit's last
// wave to finish builds the union (counted in LDS) and the others leave at once,
// freeing their registers, instead of waiting at a barrier.
template <int J>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(J <= 20 ? 3 : 1))) void select_units_kernel(
    const float* __restrict__ S, int nb, int members, int per_head, int units, double p, int k_floor,
    int order_depth, int32_t* __restrict__ counts, int16_t* __restrict__ kv_idx, int16_t* __restrict__ order,
    uint32_t* __restrict__ unit_list, int32_t* __restrict__ unit_cnt) {
  __shared__ uint32_t taken[4][64];
  __shared__ int finished[4];  // member waves done, per unit of the workgroup
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int slot = w / members;
  const int u = blockIdx.x * (4 / members) + slot;
  const int m = w % members;
  const int bh = u / per_head;
  const int qb = (u - bh * per_head) * members + m;
  if (threadIdx.x < 4) finished[threadIdx.x] = 0;
  __syncthreads();
  if (u >= units) return;  // every wave of this unit slot leaves here
  uint32_t bits = 0u;
  if (qb < nb) {
    const int row = bh * nb + qb;
    bits = select_row<J, false>(S + (size_t)row * nb, row, nb, p, k_floor, order_depth, nullptr, counts, kv_idx,
                                order);
  }
  taken[w][lane] = bits;
  __threadfence_block();  // this wave's mask is in LDS before it counts itself done
  int before = 0;
  if (lane == 0) before = atomicAdd(&finished[slot], 1);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before != members - 1) return;
  __threadfence_block();  // the other members' masks, written before their counts
  const int w0 = slot * members;
  uint32_t mine[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) mine[k] = k < members ? taken[w0 + k][lane] : 0u;
  uint32_t* out = unit_list + (size_t)u * nb;
  const uint64_t below = lanes_below(lane);
  int n = 0;
#pragma unroll
  for (int t = 0; t < J; ++t) {
    uint32_t flags = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) flags |= ((mine[k] >> t) & 1u) << k;
    const uint64_t in = __ballot(flags != 0u);
    if (flags) out[n + popc64(in & below)] = (uint32_t)(lane + 64 * t) | (flags << 28);
    n += popc64(in);
  }
  if (lane == 0) unit_cnt[u] = n;
}

// Block scores and selection in one kernel, for routing without a score matrix in
// memory. A workgroup takes kSelRows consecutive query blocks i0 .. of one head. Its
// four waves first compute their scores against every key block on the float64 MFMA
// D(16x16) += A(16x4) B(4x16) (A: the rows' block means of q, B: block means of k),
// divide by sqrt(d), round to float32 and keep them in LDS (ld floats per row, nb
// rounded up to 16); then each wave runs the selection on rows w, w + 4, ... The k
// index of lane group g = l / 16 at k-step t is channel 4 t + g and the steps go in
// order, as in scores_kernel, so the scores are the same float32 values bit for bit.
// Re-selection (RS) rows that need no new block skip the work, and a workgroup whose
// rows all do skips the scores too.
constexpr int kSelRows = 16;

template <int J, bool RS, int D>
__global__ __launch_bounds__(256) void score_select_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar, int nb, int groups,
                                                           double sqrt_d, double p, int k_floor, int order_depth,
                                                           const int32_t* __restrict__ target,
                                                           int32_t* __restrict__ counts, int16_t* __restrict__ kv_idx,
                                                           int16_t* __restrict__ order) {
  constexpr int KS = D / 4;  // k-steps of the float64 MFMA
  extern __shared__ float srows[];  // [kSelRows][ld]
  const int ld = (nb + 15) & ~15;
  const int bh = blockIdx.x / groups;
  const int i0 = (blockIdx.x - bh * groups) * kSelRows;
  const int nrows = min(kSelRows, nb - i0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile0 = bh * nb + i0;
  if (RS) {
    int need = 0;
    for (int r = 0; r < nrows; ++r) need |= target[tile0 + r] > counts[tile0 + r];
    if (!need) return;  // uniform over the workgroup
  }
  const int r16 = lane & 15, g = lane >> 4;
  // lane group g's element of the four channels 4 t .. 4 t + 3
  auto pick = [&](const float4& v) __attribute__((always_inline)) -> double {
    return (double)(g == 0 ? v.x : g == 1 ? v.y : g == 2 ? v.z : v.w);
  };
  // A operand: row i0 + r16, channel 4 t + g at k-step t (zero past the head's last block)
  double a[KS];
  {
    const float4* q4 = reinterpret_cast<const float4*>(qbar + ((size_t)tile0 + r16) * D);
    const bool in = r16 < nrows;
#pragma unroll
    for (int t = 0; t < KS; ++t) a[t] = in ? pick(q4[t]) : 0.0;
  }
  const float* kb = kbar + (size_t)bh * nb * D;
  const int col_tiles = (nb + 15) / 16;
  for (int ct = wave; ct < col_tiles; ct += 4) {
    const int j = ct * 16 + r16;
    const float4* k4 = reinterpret_cast<const float4*>(kb + (size_t)j * D);
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int t = 0; t < KS; ++t)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[t], j < nb ? pick(k4[t]) : 0.0, acc, 0, 0, 0);
    // element e of lane l is row 4 e + l / 16, column l % 16 of the tile
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * e + g;
      if (r < nrows && j < nb) srows[r * ld + j] = __double2float_rn(acc[e] / sqrt_d);
    }
  }
  __syncthreads();
  for (int r = wave; r < nrows; r += 4)
    select_row<J, RS>(srows + r * ld, tile0 + r, nb, p, k_floor, order_depth, target, counts, kv_idx, order);
}

// ------------------------------------------------------------------ workloads (Eq. 1)

__global__ __launch_bounds__(256) void workload_kernel(const int32_t* __restrict__ counts, int nb,
                                                       int32_t* __restrict__ work, float* __restrict__ L) {
  __shared__ int partial[4];
  const int32_t* c = counts + (size_t)blockIdx.x * nb;
  int sum = 0;
  for (int i = threadIdx.x; i < nb; i += 256) sum += c[i];
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int w = partial[0] + partial[1] + partial[2] + partial[3];
    work[blockIdx.x] = w;
    L[blockIdx.x] = __fdiv_rn((float)w, (float)nb);
  }
}

// ------------------------------------------------------------------ block-wide scans (1024 threads)

// Exclusive prefix sum over the 1024 threads of the workgroup (integer types, so
// the result does not depend on the order of the additions) and the total: an
// inclusive scan within each wave by shuffles, then the 16 wave totals through
// buf[0..15]. Every thread of the workgroup must call it.
template <typename T>
__device__ T block_exclusive_scan(T v, T* buf, T& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  T base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const T t = buf[w];
    base += w < wave ? t : (T)0;
    all += t;
  }
  total = all;
  __syncthreads();  // buf is free again for the next call
  return base + incl - v;
}

// ------------------------------------------------------------------ slack fill plan

// E = floor(beta * sum counts) extra blocks; the water level is the largest
// lambda with need(lambda) = sum_t max(0, lambda - c_t) <= E (tiles at nb never
// rise); every tile at or below lambda rises to lambda, and the first
// E - need(lambda) of them by tile id take one more. target[t] is the result.
// Four passes: a histogram of the counts over chunks of kQChunk tiles, the plan
// (lambda and the remainder) in one workgroup, the chunks' numbers of tiles at or
// below lambda, and the targets with each tile's rank among those tiles.
constexpr int kMaxBins = 2049;
constexpr int kQChunk = 256;

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// One workgroup per chunk: an LDS histogram, then one global add per non-empty bin
// (a chunk's tiles often share one count, e.g. the floor).
__global__ __launch_bounds__(kQChunk) void slack_hist_kernel(const int32_t* __restrict__ counts, int tiles, int nb,
                                                             int32_t* __restrict__ hist_g) {
  __shared__ int32_t hist[kMaxBins];
  for (int b = threadIdx.x; b <= nb; b += kQChunk) hist[b] = 0;
  __syncthreads();
  const int t = blockIdx.x * kQChunk + threadIdx.x;
  if (t < tiles) atomicAdd(&hist[counts[t]], 1);
  __syncthreads();
  for (int b = threadIdx.x; b <= nb; b += kQChunk)
    if (hist[b]) atomicAdd(&hist_g[b], hist[b]);
}

__global__ __launch_bounds__(1024) void slack_plan_kernel(const int32_t* __restrict__ hist_g, int nb, double beta,
                                                          int64_t* __restrict__ info) {
  __shared__ int64_t buf[1024];
  __shared__ int64_t cnt_lt_s[kMaxBins + 1];
  __shared__ int64_t sum_lt_s[kMaxBins + 1];
  // exclusive prefix over bins of hist[c] and c*hist[c]: each thread owns a run of bins
  const int bins = nb + 1;
  const int per = (bins + 1023) / 1024;
  const int b0 = threadIdx.x * per;
  int64_t my_cnt = 0, my_sum = 0;
  for (int b = b0; b < min(bins, b0 + per); ++b) {
    my_cnt += hist_g[b];
    my_sum += (int64_t)b * hist_g[b];
  }
  int64_t tot_cnt, tot_sum;
  int64_t run_cnt = block_exclusive_scan<int64_t>(my_cnt, buf, tot_cnt);
  int64_t run_sum = block_exclusive_scan<int64_t>(my_sum, buf, tot_sum);
  for (int b = b0; b < min(bins, b0 + per); ++b) {
    cnt_lt_s[b] = run_cnt;
    sum_lt_s[b] = run_sum;
    run_cnt += hist_g[b];
    run_sum += (int64_t)b * hist_g[b];
  }
  __syncthreads();
  const int64_t E = (int64_t)floor(beta * (double)tot_sum);
  // need(lambda) = lambda * #(c < lambda) - sum(c < lambda) is non-decreasing: count lambdas with need <= E
  int64_t ok = 0;
  for (int lam = threadIdx.x; lam <= nb; lam += 1024) ok += ((int64_t)lam * cnt_lt_s[lam] - sum_lt_s[lam]) <= E;
  int64_t n_ok;
  block_exclusive_scan<int64_t>(ok, buf, n_ok);
  if (threadIdx.x == 0) {
    const int64_t lam = n_ok - 1;
    info[0] = lam;
    info[1] = E - (lam * cnt_lt_s[lam] - sum_lt_s[lam]);
    info[2] = E;
    info[3] = tot_sum;
  }
}

// Tiles of this workgroup's chunk that the water level raises (count <= lambda < nb).
__device__ __forceinline__ bool slack_low(int t, int tiles, int nb, int64_t lam, const int32_t* counts) {
  return t < tiles && lam < nb && counts[t] <= lam;
}

// Sum over the workgroup (kQChunk threads = 4 waves) through `red`.
__device__ __forceinline__ int64_t chunk_sum(int64_t v, int64_t* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const int64_t all = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return all;
}

__global__ __launch_bounds__(kQChunk) void slack_low_kernel(const int32_t* __restrict__ counts, int tiles, int nb,
                                                            const int64_t* __restrict__ info,
                                                            int32_t* __restrict__ low_cnt) {
  __shared__ int64_t red[4];
  const int t = blockIdx.x * kQChunk + threadIdx.x;
  const int64_t all = chunk_sum(slack_low(t, tiles, nb, info[0], counts) ? 1 : 0, red);
  if (threadIdx.x == 0) low_cnt[blockIdx.x] = (int32_t)all;
}

__global__ __launch_bounds__(kQChunk) void slack_target_kernel(const int32_t* __restrict__ counts, int tiles,
                                                               int nb, const int64_t* __restrict__ info,
                                                               const int32_t* __restrict__ low_cnt,
                                                               int32_t* __restrict__ target) {
  __shared__ int64_t red[4];
  __shared__ int32_t wave_low[4];
  const int64_t lam = info[0], rest = info[1];
  // raised tiles in the chunks before this one
  int64_t before = 0;
  for (int ch = threadIdx.x; ch < (int)blockIdx.x; ch += kQChunk) before += low_cnt[ch];
  before = chunk_sum(before, red);
  const int t = blockIdx.x * kQChunk + threadIdx.x;
  const bool low = slack_low(t, tiles, nb, lam, counts);
  // rank among the chunk's raised tiles: earlier waves, then earlier lanes of this wave
  const uint64_t mask = __ballot(low);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wave_low[wave] = __popcll(mask);
  __syncthreads();
  int64_t rank = before + __popcll(mask & ((1ull << lane) - 1ull));
  for (int v = 0; v < wave; ++v) rank += wave_low[v];
  if (t < tiles) target[t] = lam >= nb ? nb : (low ? (int32_t)lam + (rank < rest ? 1 : 0) : counts[t]);
}

// ------------------------------------------------------------------ tile queue

// Longest first, ties by tile id: a counting sort over chunks of kQChunk tiles.
// Each chunk's histogram of counts goes to hist[(nb - c) * chunks + chunk], so an
// exclusive scan of the flat array gives, for each (count, chunk), the number of
// tiles that precede that chunk's tiles of that count in the queue.
__global__ __launch_bounds__(kQChunk) void queue_hist_kernel(const int32_t* __restrict__ counts, int tiles, int nb,
                                                             int chunks, int32_t* __restrict__ hist_flat,
                                                             int32_t* __restrict__ rank) {
  __shared__ int32_t c[kQChunk];
  __shared__ int32_t hist[kMaxBins];
  const int t = blockIdx.x * kQChunk + threadIdx.x;
  c[threadIdx.x] = t < tiles ? counts[t] : -1;
  for (int b = threadIdx.x; b <= nb; b += kQChunk) hist[b] = 0;
  __syncthreads();
  if (t < tiles) {
    const int mine = c[threadIdx.x];
    int r = 0;
    for (int u = 0; u < (int)threadIdx.x; ++u) r += c[u] == mine;
    rank[t] = r;
    atomicAdd(&hist[mine], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b <= nb; b += kQChunk) hist_flat[(size_t)(nb - b) * chunks + blockIdx.x] = hist[b];
}

// Exclusive scan of n ints in tiles of kScanTile: each workgroup scans its tile in
// place and writes the tile's total to sums[tile].
constexpr int kScanPer = 8;
constexpr int kScanTile = 256 * kScanPer;

__global__ __launch_bounds__(256) void scan_tile_kernel(int32_t* __restrict__ a, size_t n,
                                                        int32_t* __restrict__ sums) {
  __shared__ int32_t wave_tot[4];
  const size_t base = (size_t)blockIdx.x * kScanTile + (size_t)threadIdx.x * kScanPer;
  int32_t v[kScanPer];
  int32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    v[i] = base + i < n ? a[base + i] : 0;
    mine += v[i];
  }
  // inclusive scan of the threads' totals within the wave, then across the 4 waves
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t up = __shfl_up(incl, off);
    if (lane >= off) incl += up;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int32_t run = incl - mine;
  for (int w = 0; w < wave; ++w) run += wave_tot[w];
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    if (base + i < n) a[base + i] = run;
    run += v[i];
  }
  if (threadIdx.x == 255) sums[blockIdx.x] = run;
}

// Exclusive scan of the m tile totals in place (one workgroup, batches of 1024).
__global__ __launch_bounds__(1024) void scan_sums_kernel(int32_t* __restrict__ sums, int m) {
  __shared__ int64_t buf[1024];
  int64_t carry = 0;
  for (int b = 0; b < m; b += 1024) {
    const int i = b + threadIdx.x;
    const int64_t v = i < m ? sums[i] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan<int64_t>(v, buf, tot);
    if (i < m) sums[i] = (int32_t)(carry + ex);
    carry += tot;
  }
}

__global__ __launch_bounds__(256) void queue_scatter_kernel(const int32_t* __restrict__ counts, int tiles, int nb,
                                                            int chunks, const int32_t* __restrict__ hist_flat,
                                                            const int32_t* __restrict__ sums,
                                                            const int32_t* __restrict__ rank,
                                                            int32_t* __restrict__ queue) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= tiles) return;
  const size_t pos = (size_t)(nb - counts[t]) * chunks + t / kQChunk;
  queue[hist_flat[pos] + sums[pos / kScanTile] + rank[t]] = t;
}

__global__ __launch_bounds__(256) void queue_identity_kernel(int tiles, int32_t* __restrict__ queue) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < tiles) queue[t] = t;
}

// ------------------------------------------------------------------ query-block groups

// One wave per group unit u = (bh, q): the M neighbouring query blocks qM .. qM+M-1
// of head bh (those past nb are absent). Writes the ascending union of their
// retained lists, each entry j | (member m retains j) << (28 + m), and its length.
// Lane l owns block ids 32l .. 32l + 31 as M bitmaps in LDS. The list is staged in
// LDS and then written out by consecutive lanes (coalesced stores).
constexpr int kMaxUnion = 2048;  // the router's largest nb
template <int M>
__global__ __launch_bounds__(256) void group_merge_kernel(const int32_t* __restrict__ counts,
                                                          const int16_t* __restrict__ kv_idx, int nb, int per_head,
                                                          int units, uint32_t* __restrict__ unit_list,
                                                          int32_t* __restrict__ unit_cnt) {
  __shared__ uint32_t bits[4][M][64];
  __shared__ uint32_t stage[4][kMaxUnion];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int u = blockIdx.x * 4 + w;
  if (u >= units) return;
  const int bh = u / per_head;
  const int q = u - bh * per_head;
#pragma unroll
  for (int m = 0; m < M; ++m) bits[w][m][lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // eight list entries per lane in flight at a time (the loads do not wait on each other)
  constexpr int kInFlight = 8;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int qb = q * M + m;
    if (qb >= nb) continue;
    const int64_t t = (int64_t)bh * nb + qb;
    const int c = counts[t];
    const int16_t* row = kv_idx + t * nb;
    for (int i0 = lane; i0 < c; i0 += 64 * kInFlight) {
      int j[kInFlight];
#pragma unroll
      for (int a = 0; a < kInFlight; ++a) j[a] = i0 + 64 * a < c ? row[i0 + 64 * a] : -1;
#pragma unroll
      for (int a = 0; a < kInFlight; ++a)
        if (j[a] >= 0) atomicOr(&bits[w][m][j[a] >> 5], 1u << (j[a] & 31));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  uint32_t word[M];
  uint32_t any = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    word[m] = bits[w][m][lane];
    any |= word[m];
  }
  const int mine = __popc(any);
  int incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  int pos = incl - mine;
  for (int k = 0; k < 32; ++k) {
    if ((any >> k) & 1u) {
      uint32_t e = (uint32_t)(lane * 32 + k);
#pragma unroll
      for (int m = 0; m < M; ++m) e |= ((word[m] >> k) & 1u) << (28 + m);
      stage[w][pos++] = e;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int total = __shfl(incl, 63);
  uint32_t* out = unit_list + (size_t)u * nb;
  for (int i = lane; i < total; i += 64) out[i] = stage[w][i];
  if (lane == 63) unit_cnt[u] = incl;
}

// ------------------------------------------------------------------ queue segments (one per XCD)

constexpr int kSegments = 8;
constexpr int kUnitOverhead = 1;  // per-unit cost of the query loads and output writes, in key blocks

// sched[0..8]: bounds of the eight queue segments the attention kernel pulls
// from, one per XCD, over `units` work units with costs cost[u] (retained key
// blocks; NULL = all equal). balanced == 0: one segment holds every unit (plain
// list scheduling in queue order). balanced != 0: the units, in order, are cut
// where the running cost (cost + overhead) first reaches x/8 of the total, so
// each XCD gets a contiguous, equally heavy run of neighbouring query blocks:
// the one-GPU reading of the review's RLB with the XCDs (separate L2 caches) as
// the ranks. sched[9] = the unit kind for the attention kernel.
__global__ __launch_bounds__(1024) void segments_kernel(const int32_t* __restrict__ cost, int units, int balanced,
                                                        int kind, int32_t* __restrict__ sched) {
  __shared__ int64_t buf[1024];
  __shared__ int64_t target[kSegments + 1];
  __shared__ int32_t bound[kSegments + 1];
  if (threadIdx.x == 0) sched[kSegments + 1] = kind;
  if (!balanced) {
    if (threadIdx.x <= kSegments) sched[threadIdx.x] = threadIdx.x == 0 ? 0 : units;
    return;
  }
  int64_t mine = 0;
#pragma unroll 8
  for (int u = threadIdx.x; u < units; u += 1024) mine += (int64_t)cost[u] + kUnitOverhead;
  int64_t total;
  block_exclusive_scan<int64_t>(mine, buf, total);
  if (threadIdx.x <= kSegments) {
    target[threadIdx.x] = (total * threadIdx.x + kSegments - 1) / kSegments;
    bound[threadIdx.x] = units;
  }
  __syncthreads();
  // bound x = the smallest u whose preceding cost reaches target x: the unit v
  // with before(v) < target <= before(v) + cost(v) ends just before it
  int64_t seen = 0;
  // each chunk's costs are loaded while the previous chunk is scanned
  int64_t c_next = (int)threadIdx.x < units ? (int64_t)cost[threadIdx.x] + kUnitOverhead : 0;
  for (int u0 = 0; u0 < units; u0 += 1024) {
    const int u = u0 + threadIdx.x;
    const int64_t c = c_next;
    c_next = u + 1024 < units ? (int64_t)cost[u + 1024] + kUnitOverhead : 0;
    int64_t chunk;
    const int64_t before = seen + block_exclusive_scan<int64_t>(c, buf, chunk);
    if (u < units)
      for (int x = 1; x < kSegments; ++x)
        if (before < target[x] && target[x] <= before + c) bound[x] = u + 1;
    seen += chunk;
    __syncthreads();
  }
  if (threadIdx.x <= kSegments) sched[threadIdx.x] = threadIdx.x == 0 ? 0 : bound[threadIdx.x];
}

// The longest-first order of the group units inside each XCD run (the one-GPU
// reading of the review's RLB as a longest-processing-time-first queue, with the
// XCDs' contiguous runs as in the "xcd" schedule): run x = blockIdx.x holds the
// units sched[x] .. sched[x + 1] - 1, ordered by union length (cost) descending,
// ties by unit index. A stable counting sort over the run: the bins' starts from a
// histogram and its scan, then one wave walks the run 64 units at a time; a unit's
// place is its bin's running start plus the units of equal cost before it among
// the 64 (lanes of equal cost found by comparing the costs bit by bit across the
// wave), and the lowest lane of each such group advances the bin's start.
constexpr int kLptChunk = 4096;

__global__ __launch_bounds__(1024) void unit_lpt_kernel(const int32_t* __restrict__ cost, int units, int nb,
                                                        const int32_t* __restrict__ sched,
                                                        int32_t* __restrict__ unit_queue) {
  __shared__ int32_t start[kMaxBins];
  __shared__ int64_t buf[1024];
  __shared__ int32_t chunk[kLptChunk];
  const int lo = sched[blockIdx.x], hi = sched[blockIdx.x + 1];
  for (int b = threadIdx.x; b <= nb; b += 1024) start[b] = 0;
  __syncthreads();
  for (int u = lo + (int)threadIdx.x; u < hi; u += 1024) atomicAdd(&start[cost[u]], 1);
  __syncthreads();
  // bins in descending cost: the exclusive scan of the counts from cost nb down
  int64_t carry = 0;
  for (int b0 = 0; b0 <= nb; b0 += 1024) {
    const int b = nb - (b0 + (int)threadIdx.x);  // cost of this thread's bin
    const int64_t v = b >= 0 ? start[b] : 0;
    int64_t tot;
    const int64_t ex = block_exclusive_scan<int64_t>(v, buf, tot);
    __syncthreads();
    if (b >= 0) start[b] = (int32_t)(carry + ex);
    carry += tot;
    __syncthreads();
  }
  // the run's costs are staged in LDS a chunk at a time, so the walk issues no loads
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int bits = 32 - __clz(nb);  // costs lie in 0 .. nb
  for (int k0 = lo; k0 < hi; k0 += kLptChunk) {
    const int k1 = min(hi, k0 + kLptChunk);
    for (int u = k0 + (int)threadIdx.x; u < k1; u += 1024) chunk[u - k0] = cost[u];
    __syncthreads();
    if (threadIdx.x < 64) {
      for (int c0 = k0; c0 < k1; c0 += 64) {
        const int u = c0 + lane;
        const bool in = u < k1;
        const int mine = in ? chunk[u - k0] : 0;
        uint64_t eq = __ballot(in);
        for (int b = 0; b < bits; ++b) {
          const bool one = (mine >> b) & 1;
          const uint64_t m = __ballot(in && one);
          eq &= one ? m : ~m;
        }
        int pos = 0;
        if (in) pos = start[mine] + __popcll(eq & below);
        if (in) unit_queue[lo + pos] = u;
        __builtin_amdgcn_wave_barrier();
        if (in && (eq & below) == 0) start[mine] += __popcll(eq);
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ structured router

// The LVSA note's block-sparse pattern (a structured local window plus global
// anchor blocks that rotate with the diffusion step), in block ids: query block
// i keeps the key blocks j with |j - i| <= window, and every key block with
// j mod stride == offset (stride 0: none). The same for every head; one wave
// per tile row writes the ascending list by ballot and prefix count.
__global__ __launch_bounds__(256) void window_anchor_kernel(int nb, int tiles, int window, int stride, int offset,
                                                            int32_t* __restrict__ counts,
                                                            int16_t* __restrict__ kv_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= tiles) return;
  const int i = row % nb;
  const int lo = max(0, i - window), hi = min(nb - 1, i + window);
  int16_t* out = kv_idx + (size_t)row * nb;
  int n = 0;
  for (int j0 = 0; j0 < nb; j0 += 64) {
    const int j = j0 + lane;
    const bool in = j < nb && ((j >= lo && j <= hi) || (stride > 0 && j % stride == offset));
    const uint64_t mask = __ballot(in);
    if (in) out[n + __popcll(mask & ((1ull << lane) - 1))] = (int16_t)j;
    n += __popcll(mask);
  }
  if (lane == 0) counts[row] = n;
}

// ------------------------------------------------------------------ rank-level RLB and SASA

// The eight XCDs as the ranks of the xllm-io review's runtime stages (核心公式
// Eq. 1-2 and 5-10, 3.2 RLB, 3.3 SASA and its piecewise policy, parameters of
// 五). Rank r first holds the contiguous heads floor(r BH / 8) ..
// floor((r + 1) BH / 8) - 1 (the Ulysses head split). Loads are in retained
// blocks, W_r = sum of work_h over the rank's heads; L_r of Eq. 1 is W_r / nb,
// and every ratio below is the same in either unit.
//
// RLB searches the one-send-one-receive plans over the review's pair topologies
// (3.2): the eight ranks are matched in pairs (the 105 perfect matchings, in
// canonical order: the lowest unpaired rank with each higher unpaired rank,
// ascending, recursively), and a pair (a, b) either moves nothing, or a sends one
// of its heads to b, or b one of its heads to a, or they swap one head each (in
// that order; heads ascending, a's head varying slowest in a swap). The plan of
// least (max W^new, sum (W^new)^2) wins, ties to the first in the order matching,
// then the pairs' options with the first pair varying slowest. The pairs of a
// matching touch disjoint ranks, so each matching's best plan is exact pair by
// pair: its least maximum M is the largest over its pairs of the pair's least
// maximum, and each pair takes, among its options of maximum at most M, the first
// of least sum of squares. SASA gives rank r the budget E_r = floor(n1 dW_r) when
// dW_r = W_max - W_r exceeds n2 W_max (float64), spent by water-filling the
// rank's tiles along their importance order.
//
// info (float64, kRankInfo entries): [0] rho before, [1] after migration, [2]
// after augmentation; [3] policy taken (0 none, 1 SASA, 2 RLB + SASA, 3 RLB); [4]
// moves; [5..12] W before, [13..20] after migration, [21..28] after
// augmentation; [29..36] E_r; [37..60] the moves as (head, from, to), by sending
// rank; [61] candidate plans in the space (sum over matchings of the product of
// the pairs' option counts); [62] 0.
constexpr int kRanks = kSegments;
constexpr int kMatchings = 105;  // perfect matchings of eight ranks

__device__ double rank_rho(const int64_t* W) {
  int64_t mx = W[0], sum = 0;
  for (int r = 0; r < kRanks; ++r) {
    mx = W[r] > mx ? W[r] : mx;
    sum += W[r];
  }
  return (double)mx / ((double)sum / kRanks);
}

// matching t in canonical order: pairs (a[i], b[i]), i = 0..3, a ascending
__device__ void rank_matching(int t, int* pa, int* pb) {
  int free_[kRanks];
  for (int r = 0; r < kRanks; ++r) free_[r] = r;
  int n = kRanks;
  const int pick[3] = {t / 15 + 1, (t / 3) % 5 + 1, t % 3 + 1};
  for (int i = 0; i < 4; ++i) {
    const int j = i < 3 ? pick[i] : 1;
    pa[i] = free_[0];
    pb[i] = free_[j];
    for (int k = j; k + 1 < n; ++k) free_[k] = free_[k + 1];  // drop free_[j], then free_[0]
    for (int k = 0; k + 1 < n - 1; ++k) free_[k] = free_[k + 1];
    n -= 2;
  }
}

// The options of pair (a, b) in order; fn(index, moved head of a or -1, of b or -1, wa, wb)
// returns true to stop.
template <typename Fn>
__device__ void pair_options(const int32_t* work, const int* hlo, const int64_t* W, int a, int b, Fn fn) {
  const int na = hlo[a + 1] - hlo[a], nb_ = hlo[b + 1] - hlo[b];
  int idx = 0;
  if (fn(idx++, -1, -1, W[a], W[b])) return;
  for (int i = 0; i < na; ++i) {
    const int64_t d = work[hlo[a] + i];
    if (fn(idx++, hlo[a] + i, -1, W[a] - d, W[b] + d)) return;
  }
  for (int i = 0; i < nb_; ++i) {
    const int64_t d = work[hlo[b] + i];
    if (fn(idx++, -1, hlo[b] + i, W[a] + d, W[b] - d)) return;
  }
  for (int i = 0; i < na; ++i)
    for (int j = 0; j < nb_; ++j) {
      const int64_t x = work[hlo[a] + i], y = work[hlo[b] + j];
      if (fn(idx++, hlo[a] + i, hlo[b] + j, W[a] - x + y, W[b] - y + x)) return;
    }
}

__global__ __launch_bounds__(128) void rank_plan_kernel(const int32_t* __restrict__ work, int BH, int per_head,
                                                        int members, int policy, double k1, double k2, double n1,
                                                        double n2, int32_t* __restrict__ owner,
                                                        int32_t* __restrict__ head_order,
                                                        int64_t* __restrict__ budget, int32_t* __restrict__ sched,
                                                        double* __restrict__ info) {
  __shared__ int64_t W0[kRanks];
  __shared__ int hlo[kRanks + 1];
  __shared__ int mode;
  __shared__ int64_t red_max[128], red_sq[128];
  __shared__ int red_idx[128];
  const int tid = threadIdx.x;
  if (tid == 0) {
    for (int r = 0; r <= kRanks; ++r) hlo[r] = (int)((int64_t)r * BH / kRanks);
    for (int r = 0; r < kRanks; ++r) {
      int64_t w = 0;
      for (int h = hlo[r]; h < hlo[r + 1]; ++h) w += work[h];
      W0[r] = w;
    }
    const double rho = rank_rho(W0);
    mode = policy >= 0 ? policy : (rho < k1 ? 0 : rho < k2 ? 1 : 2);
    info[0] = rho;
    info[3] = (double)mode;
  }
  __syncthreads();
  const bool rlb = mode == 2 || mode == 3;
  // matching tid: its least maximum M and least sum of squares under M
  int64_t best_max = INT64_MAX, best_sq = INT64_MAX;
  int best_t = INT32_MAX;
  if (rlb && tid < kMatchings) {
    int pa[4], pb[4];
    rank_matching(tid, pa, pb);
    int64_t M = 0;
    for (int i = 0; i < 4; ++i) {
      int64_t bm = INT64_MAX;
      pair_options(work, hlo, W0, pa[i], pb[i], [&](int, int, int, int64_t wa, int64_t wb) {
        const int64_t m = wa > wb ? wa : wb;
        bm = m < bm ? m : bm;
        return false;
      });
      M = bm > M ? bm : M;
    }
    int64_t S = 0;
    for (int i = 0; i < 4; ++i) {
      int64_t least = INT64_MAX;
      pair_options(work, hlo, W0, pa[i], pb[i], [&](int, int, int, int64_t wa, int64_t wb) {
        if ((wa > wb ? wa : wb) <= M) {
          const int64_t q = wa * wa + wb * wb;
          least = q < least ? q : least;
        }
        return false;
      });
      S += least;
    }
    best_max = M;
    best_sq = S;
    best_t = tid;
  }
  red_max[tid] = best_max;
  red_sq[tid] = best_sq;
  red_idx[tid] = best_t;
  __syncthreads();
  for (int off = 64; off > 0; off >>= 1) {
    if (tid < off) {
      const int o = tid + off;
      if (red_max[o] < red_max[tid] ||
          (red_max[o] == red_max[tid] &&
           (red_sq[o] < red_sq[tid] || (red_sq[o] == red_sq[tid] && red_idx[o] < red_idx[tid])))) {
        red_max[tid] = red_max[o];
        red_sq[tid] = red_sq[o];
        red_idx[tid] = red_idx[o];
      }
    }
    __syncthreads();
  }
  if (tid != 0) return;
  for (int r = 0; r < kRanks; ++r)
    for (int h = hlo[r]; h < hlo[r + 1]; ++h) owner[h] = r;
  // candidate plans in the space
  double space = 0.0;
  for (int t = 0; t < kMatchings; ++t) {
    int pa[4], pb[4];
    rank_matching(t, pa, pb);
    double n = 1.0;
    for (int i = 0; i < 4; ++i) {
      const double na = hlo[pa[i] + 1] - hlo[pa[i]], nb_ = hlo[pb[i] + 1] - hlo[pb[i]];
      n *= 1.0 + na + nb_ + na * nb_;
    }
    space += n;
  }
  info[61] = rlb ? space : 0.0;
  info[62] = 0.0;
  int send_head[kRanks], send_to[kRanks];
  for (int r = 0; r < kRanks; ++r) send_head[r] = -1;
  if (rlb) {
    int pa[4], pb[4];
    rank_matching(red_idx[0], pa, pb);
    const int64_t M = red_max[0];
    for (int i = 0; i < 4; ++i) {
      int64_t least = INT64_MAX;
      pair_options(work, hlo, W0, pa[i], pb[i], [&](int, int, int, int64_t wa, int64_t wb) {
        if ((wa > wb ? wa : wb) <= M) {
          const int64_t q = wa * wa + wb * wb;
          least = q < least ? q : least;
        }
        return false;
      });
      const int a = pa[i], b = pb[i];
      pair_options(work, hlo, W0, a, b, [&](int, int ha, int hb, int64_t wa, int64_t wb) {
        if ((wa > wb ? wa : wb) > M || wa * wa + wb * wb != least) return false;
        if (ha >= 0) {
          send_head[a] = ha;
          send_to[a] = b;
        }
        if (hb >= 0) {
          send_head[b] = hb;
          send_to[b] = a;
        }
        return true;
      });
    }
  }
  int n_moves = 0;  // the moves by sending rank
  for (int r = 0; r < kRanks; ++r) {
    if (send_head[r] < 0) continue;
    owner[send_head[r]] = send_to[r];
    info[37 + 3 * n_moves] = send_head[r];
    info[38 + 3 * n_moves] = r;
    info[39 + 3 * n_moves] = send_to[r];
    ++n_moves;
  }
  int64_t W1[kRanks] = {};
  for (int h = 0; h < BH; ++h) W1[owner[h]] += work[h];
  int64_t wmax = 0;
  for (int r = 0; r < kRanks; ++r) wmax = W1[r] > wmax ? W1[r] : wmax;
  for (int r = 0; r < kRanks; ++r) {
    const int64_t dW = wmax - W1[r];
    int64_t e = 0;
    if ((mode == 1 || mode == 2) && (double)dW > n2 * (double)wmax) e = (int64_t)floor(n1 * (double)dW);
    budget[r] = e;
    info[5 + r] = (double)W0[r];
    info[13 + r] = (double)W1[r];
    info[29 + r] = (double)e;
  }
  info[1] = rank_rho(W1);
  info[4] = (double)n_moves;
  // queue segments: the ranks' heads in rank order, ascending within a rank
  int pos = 0;
  for (int r = 0; r < kRanks; ++r) {
    sched[r] = pos * per_head;
    for (int h = 0; h < BH; ++h)
      if (owner[h] == r) head_order[pos++] = h;
  }
  sched[kRanks] = pos * per_head;
  sched[kRanks + 1] = members;
}

// SASA step 2 on rank r = blockIdx.x: raise the lightest of the rank's tiles E_r
// times (ties: the lower position, positions running over the rank's heads in
// head_order and over query blocks within a head; full tiles skipped), in closed
// form as in slack_plan_kernel. target[t] = the new count of every tile.
__global__ __launch_bounds__(1024) void rank_fill_kernel(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ head_order,
                                                         const int32_t* __restrict__ sched, int per_head, int nb,
                                                         const int64_t* __restrict__ budget,
                                                         int32_t* __restrict__ target) {
  __shared__ int32_t hist[kMaxBins];
  __shared__ int64_t buf[1024];
  __shared__ int64_t cnt_lt_s[kMaxBins + 1];
  __shared__ int64_t sum_lt_s[kMaxBins + 1];
  __shared__ int64_t lam_s, rest_s;
  const int r = blockIdx.x;
  const int h0 = sched[r] / per_head, h1 = sched[r + 1] / per_head;
  const int n = (h1 - h0) * nb;  // the rank's tiles, by position
  auto tile = [&](int q) { return (size_t)head_order[h0 + q / nb] * nb + q % nb; };
  const int64_t E = budget[r];
  if (E == 0) {
    for (int q = threadIdx.x; q < n; q += 1024) target[tile(q)] = counts[tile(q)];
    return;
  }
  for (int b = threadIdx.x; b <= nb; b += 1024) hist[b] = 0;
  __syncthreads();
  for (int q = threadIdx.x; q < n; q += 1024) atomicAdd(&hist[counts[tile(q)]], 1);
  __syncthreads();
  const int bins = nb + 1;
  const int per = (bins + 1023) / 1024;
  const int b0 = threadIdx.x * per;
  int64_t my_cnt = 0, my_sum = 0;
  for (int b = b0; b < min(bins, b0 + per); ++b) {
    my_cnt += hist[b];
    my_sum += (int64_t)b * hist[b];
  }
  int64_t tot_cnt, tot_sum;
  int64_t run_cnt = block_exclusive_scan<int64_t>(my_cnt, buf, tot_cnt);
  int64_t run_sum = block_exclusive_scan<int64_t>(my_sum, buf, tot_sum);
  for (int b = b0; b < min(bins, b0 + per); ++b) {
    cnt_lt_s[b] = run_cnt;
    sum_lt_s[b] = run_sum;
    run_cnt += hist[b];
    run_sum += (int64_t)b * hist[b];
  }
  __syncthreads();
  int64_t ok = 0;
  for (int lam = threadIdx.x; lam <= nb; lam += 1024) ok += ((int64_t)lam * cnt_lt_s[lam] - sum_lt_s[lam]) <= E;
  int64_t n_ok;
  block_exclusive_scan<int64_t>(ok, buf, n_ok);
  if (threadIdx.x == 0) {
    const int64_t lam = n_ok - 1;
    lam_s = lam;
    rest_s = E - (lam * cnt_lt_s[lam] - sum_lt_s[lam]);
  }
  __syncthreads();
  const int lam = (int)lam_s;
  const int64_t rest = rest_s;
  int64_t seen = 0;
  for (int base = 0; base < n; base += 1024) {
    const int q = base + threadIdx.x;
    const int c = q < n ? counts[tile(q)] : nb;
    const int64_t low = (lam < nb && c <= lam) ? 1 : 0;
    int64_t chunk_total;
    const int64_t rank = seen + block_exclusive_scan<int64_t>(low, buf, chunk_total);
    if (q < n) target[tile(q)] = lam >= nb ? nb : (low ? lam + (rank < rest ? 1 : 0) : c);
    seen += chunk_total;
  }
}

// rho and the rank loads after augmentation (info[2], info[21..28]).
__global__ void rank_final_kernel(const int32_t* __restrict__ work, const int32_t* __restrict__ owner, int BH,
                                  double* __restrict__ info) {
  if (threadIdx.x != 0) return;
  int64_t W[kRanks] = {};
  for (int h = 0; h < BH; ++h) W[owner[h]] += work[h];
  for (int r = 0; r < kRanks; ++r) info[21 + r] = (double)W[r];
  info[2] = rank_rho(W);
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_pool(const absh_ctx* c, const void* xh, int xh_is_f32, float* xbar, int B, int H, int d,
                       hipStream_t s) {
  const unsigned grid = (unsigned)((uint64_t)B * H * c->nb);
  const bf16_t* x = reinterpret_cast<const bf16_t*>(xh);
  const float* xf = reinterpret_cast<const float*>(xh);
  if (d == 64 && !xh_is_f32)
    pool_kernel<64, bf16_t><<<grid, kPoolThreads, 0, s>>>(x, xbar, c->N, c->n_pad, c->nb, c->block);
  else if (d == 128 && !xh_is_f32)
    pool_kernel<128, bf16_t><<<grid, kPoolThreads, 0, s>>>(x, xbar, c->N, c->n_pad, c->nb, c->block);
  else if (d == 64)
    pool_kernel<64, float><<<grid, kPoolThreads, 0, s>>>(xf, xbar, c->N, c->n_pad, c->nb, c->block);
  else if (d == 128)
    pool_kernel<128, float><<<grid, kPoolThreads, 0, s>>>(xf, xbar, c->N, c->n_pad, c->nb, c->block);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_scores(const absh_ctx* c, const float* qbar, const float* kbar, float* S, int BH, int d,
                         hipStream_t s) {
  const int side = (c->nb + kTile - 1) / kTile;
  scores_kernel<<<(unsigned)((uint64_t)BH * side * side), 256, 0, s>>>(qbar, kbar, S, c->nb, d,
                                                                        sqrt((double)d), side);
  return hipGetLastError();
}

hipError_t launch_select(const absh_ctx* c, const RouteBuffers& rb, int tiles, double p, int k_floor,
                         int order_depth, int reselect, hipStream_t s, int unit_members) {
  const int nb = c->nb;
  const int groups = (nb + kSelRows - 1) / kSelRows;
  const unsigned grid = (unsigned)((uint64_t)(tiles / nb) * groups);
  const double sqrt_d = sqrt((double)rb.d);
  const size_t lds = (size_t)kSelRows * ((nb + 15) & ~15) * sizeof(float);
#define ABSH_SELECT_D(JJ, DD)                                                                          \
  do {                                                                                                 \
    if (reselect)                                                                                      \
      score_select_kernel<JJ, true, DD><<<grid, 256, lds, s>>>(rb.qbar, rb.kbar, nb, groups, sqrt_d, p, k_floor, \
                                                             order_depth, rb.target, rb.counts, rb.kv_idx,  \
                                                             rb.order);                                \
    else                                                                                               \
      score_select_kernel<JJ, false, DD><<<grid, 256, lds, s>>>(rb.qbar, rb.kbar, nb, groups, sqrt_d, p, k_floor, \
                                                              order_depth, rb.target, rb.counts, rb.kv_idx, \
                                                              rb.order);                               \
  } while (0)
#define ABSH_SELECT(JJ)                          \
  do {                                           \
    if (rb.d == 64)                              \
      ABSH_SELECT_D(JJ, 64);                     \
    else                                         \
      ABSH_SELECT_D(JJ, 128);                    \
  } while (0)
  if (rb.d != 64 && rb.d != 128) return hipErrorInvalidValue;
  const unsigned row_grid = (unsigned)((tiles + 3) / 4);
  if (rb.S) {  // scores in memory
    const bool units_too = !reselect && (unit_members == 2 || unit_members == 4);
    const int per_head = (nb + unit_members - 1) / (unit_members > 0 ? unit_members : 1);
    const int units = units_too ? (tiles / nb) * per_head : 0;
    const unsigned unit_grid = units_too ? (unsigned)((units + 4 / unit_members - 1) / (4 / unit_members)) : 0u;
#define ABSH_SELECT_S(JJ)                                                                                  \
  do {                                                                                                     \
    if (units_too)                                                                                         \
      select_units_kernel<JJ><<<unit_grid, 256, 0, s>>>(rb.S, nb, unit_members, per_head, units, p, k_floor,  \
                                                        order_depth, rb.counts, rb.kv_idx, rb.order,      \
                                                        rb.unit_list, rb.unit_cnt);                       \
    else if (reselect)                                                                                     \
      select_kernel<JJ, true><<<row_grid, 256, 0, s>>>(rb.S, nb, tiles, p, k_floor, order_depth, rb.target,  \
                                                       rb.counts, rb.kv_idx, rb.order);                   \
    else                                                                                                   \
      select_kernel<JJ, false><<<row_grid, 256, 0, s>>>(rb.S, nb, tiles, p, k_floor, order_depth, rb.target, \
                                                        rb.counts, rb.kv_idx, rb.order);                  \
  } while (0)
    if (nb <= 64) ABSH_SELECT_S(1);
    else if (nb <= 256) ABSH_SELECT_S(4);
    else if (nb <= 512) ABSH_SELECT_S(8);
    else if (nb <= 1024) ABSH_SELECT_S(16);
    else if (nb <= 1280) ABSH_SELECT_S(20);
    else if (nb <= 1536) ABSH_SELECT_S(24);
    else if (nb <= 2048) ABSH_SELECT_S(32);
    else return hipErrorInvalidValue;
#undef ABSH_SELECT_S
    return hipGetLastError();
  }
  if (nb <= 64) ABSH_SELECT(1);
  else if (nb <= 256) ABSH_SELECT(4);
  else if (nb <= 512) ABSH_SELECT(8);
  else if (nb <= 1024) ABSH_SELECT(16);
  else if (nb <= 1280) ABSH_SELECT(20);
  else if (nb <= 1536) ABSH_SELECT(24);
  else if (nb <= 2048) ABSH_SELECT(32);
  else return hipErrorInvalidValue;
#undef ABSH_SELECT
#undef ABSH_SELECT_D
  return hipGetLastError();
}

hipError_t launch_slack_plan(const absh_ctx* c, const RouteBuffers& rb, int tiles, double beta, hipStream_t s) {
  const int chunks = queue_chunks(tiles);
  int32_t* hist_g = rb.slack_aux;            // [nb + 1]
  int32_t* low_cnt = rb.slack_aux + kMaxBins;  // [chunks]
  zero_i32_kernel<<<(c->nb + 1 + 255) / 256, 256, 0, s>>>(hist_g, c->nb + 1);
  slack_hist_kernel<<<chunks, kQChunk, 0, s>>>(rb.counts, tiles, c->nb, hist_g);
  slack_plan_kernel<<<1, 1024, 0, s>>>(hist_g, c->nb, beta, rb.slack_info);
  slack_low_kernel<<<chunks, kQChunk, 0, s>>>(rb.counts, tiles, c->nb, rb.slack_info, low_cnt);
  slack_target_kernel<<<chunks, kQChunk, 0, s>>>(rb.counts, tiles, c->nb, rb.slack_info, low_cnt, rb.target);
  return hipGetLastError();
}

hipError_t launch_workload(const absh_ctx* c, const RouteBuffers& rb, int BH, hipStream_t s) {
  workload_kernel<<<BH, 256, 0, s>>>(rb.counts, c->nb, rb.work, rb.L);
  return hipGetLastError();
}

hipError_t launch_rank_stage(const absh_ctx* c, const RouteBuffers& rb, int BH, const RankOpts& o, hipStream_t s) {
  const int members = unit_members(c, ABSH_SCHED_RANKS);
  const int per_head = (c->nb + members - 1) / members;
  rank_plan_kernel<<<1, 128, 0, s>>>(rb.work, BH, per_head, members, o.policy, o.k1, o.k2, o.n1, o.n2, rb.owner,
                                      rb.head_order, rb.budget, rb.sched, rb.rank_info);
  return hipGetLastError();
}

hipError_t launch_rank_fill(const absh_ctx* c, const RouteBuffers& rb, hipStream_t s) {
  const int members = unit_members(c, ABSH_SCHED_RANKS);
  const int per_head = (c->nb + members - 1) / members;
  rank_fill_kernel<<<kRanks, 1024, 0, s>>>(rb.counts, rb.head_order, rb.sched, per_head, c->nb, rb.budget,
                                            rb.target);
  return hipGetLastError();
}

hipError_t launch_rank_final(const RouteBuffers& rb, int BH, hipStream_t s) {
  rank_final_kernel<<<1, 64, 0, s>>>(rb.work, rb.owner, BH, rb.rank_info);
  return hipGetLastError();
}

hipError_t launch_window_anchor(const absh_ctx* c, const RouteBuffers& rb, int tiles, int window, int stride,
                                int offset, hipStream_t s) {
  window_anchor_kernel<<<(unsigned)((tiles + 3) / 4), 256, 0, s>>>(c->nb, tiles, window, stride, offset, rb.counts,
                                                                    rb.kv_idx);
  return hipGetLastError();
}

int queue_chunks(int tiles) { return (tiles + kQChunk - 1) / kQChunk; }

int queue_scan_tiles(int tiles, int nb) {
  return (int)(((size_t)queue_chunks(tiles) * (nb + 1) + kScanTile - 1) / kScanTile);
}

int slack_aux_words(int tiles) { return kMaxBins + queue_chunks(tiles); }

int unit_members(const absh_ctx* c, int schedule) {
  // longest first: group units where the union kernel runs them (blocks of 64 and
  // 128), single tiles in the tile queue's order otherwise
  if (schedule == ABSH_SCHED_LPT && c->block < 64) return 1;
  return c->block >= 128 ? 2 : 4;
}

int unit_count(const absh_ctx* c, int BH, int members) { return BH * ((c->nb + members - 1) / members); }

hipError_t launch_groups(const absh_ctx* c, const RouteBuffers& rb, int BH, int members, hipStream_t s) {
  const int per_head = (c->nb + members - 1) / members;
  const int units = BH * per_head;
  const unsigned grid = (unsigned)((units + 3) / 4);
  if (members == 2)
    group_merge_kernel<2><<<grid, 256, 0, s>>>(rb.counts, rb.kv_idx, c->nb, per_head, units, rb.unit_list,
                                                rb.unit_cnt);
  else
    group_merge_kernel<4><<<grid, 256, 0, s>>>(rb.counts, rb.kv_idx, c->nb, per_head, units, rb.unit_list,
                                                rb.unit_cnt);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  zero_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_segments(const absh_ctx* c, const RouteBuffers& rb, int BH, int schedule, hipStream_t s) {
  const int members = unit_members(c, schedule);
  if (members == 1)
    segments_kernel<<<1, 1024, 0, s>>>(rb.counts, BH * c->nb, 0, 1, rb.sched);
  else
    segments_kernel<<<1, 1024, 0, s>>>(rb.unit_cnt, unit_count(c, BH, members),
                                       schedule == ABSH_SCHED_XCD || schedule == ABSH_SCHED_LPT, members, rb.sched);
  return hipGetLastError();
}

hipError_t launch_unit_lpt(const absh_ctx* c, const RouteBuffers& rb, int BH, hipStream_t s) {
  const int members = unit_members(c, ABSH_SCHED_LPT);
  unit_lpt_kernel<<<kSegments, 1024, 0, s>>>(rb.unit_cnt, unit_count(c, BH, members), c->nb, rb.sched,
                                             rb.unit_queue);
  return hipGetLastError();
}

hipError_t launch_queue(const absh_ctx* c, const RouteBuffers& rb, int tiles, int lpt, hipStream_t s) {
  const unsigned grid = (unsigned)((tiles + 255) / 256);
  if (!lpt) {
    queue_identity_kernel<<<grid, 256, 0, s>>>(tiles, rb.queue);
    return hipGetLastError();
  }
  const int chunks = queue_chunks(tiles);
  const size_t n = (size_t)chunks * (c->nb + 1);
  const int scan_tiles = queue_scan_tiles(tiles, c->nb);
  queue_hist_kernel<<<chunks, kQChunk, 0, s>>>(rb.counts, tiles, c->nb, chunks, rb.chunk_hist, rb.rank);
  scan_tile_kernel<<<scan_tiles, 256, 0, s>>>(rb.chunk_hist, n, rb.scan_sums);
  scan_sums_kernel<<<1, 1024, 0, s>>>(rb.scan_sums, scan_tiles);
  queue_scatter_kernel<<<grid, 256, 0, s>>>(rb.counts, tiles, c->nb, chunks, rb.chunk_hist, rb.scan_sums, rb.rank,
                                            rb.queue);
  return hipGetLastError();
}

}  // namespace absh
