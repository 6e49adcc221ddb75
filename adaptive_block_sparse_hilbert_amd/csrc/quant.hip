// V quantization to 8-bit floating point (the "V quantization" step of the
// xllm-io review of FVAttn, "Block-Sparse Attention Execution" and section 3.4).
//
// Format: OCP FP8 E4M3 (bias 7, largest magnitude 448, round to nearest even),
// one power-of-two scale 2^e per (batch, head, channel): e is the smallest
// integer with max_r |v[r, c]| * 2^-e <= 448. Scaling by a power of two is exact,
// so the encoding is the only rounding, and the scale can be applied to the
// attention output instead of to every value.
//
// Layout (ABSH_VT8): per (b, h), the keys in steps of 64 (n_pad / 64 steps), each
// step an image of 64 * d bytes that the attention kernel copies into LDS as is:
//   byte  eta * 32 d + 32 c + 16 (g ^ ((c >> 3) & 1)) + 8 a + i
//   holds channel c of key 32 eta + 16 a + 8 g + i   (eta, a, g in {0, 1}, i < 8).
// The 32 bytes a lane of the value product needs (channel c, keys of half g of
// the fp8 MFMA's k range) are then the 16 bytes at 32 c + 16 (g ^ ...) of both
// regions, and 16 lanes reading 16 channels hit 16 distinct bank groups.
#include "absh_internal.h"

namespace absh {
namespace {

constexpr int kThreads = 256;
constexpr int kAmaxSlices = 32;  // workgroups per head in the maximum pass

// Smallest e with amax * 2^-e <= 448 = 0.875 * 2^9, from amax = f 2^E with
// f in [0.5, 1): E - e <= 9 when f <= 0.875, else E - e <= 8. 0 for amax = 0.
__device__ __forceinline__ int scale_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);
  return f <= 0.875f ? E - 9 : E - 8;
}

__global__ __launch_bounds__(kThreads) void zero_words(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// amax_bits[bh * D + c] = max(amax_bits, bits of max |v[bh, r, c]| over this
// workgroup's rows): non-negative floats order like their bit patterns.
template <int D>
__global__ __launch_bounds__(kThreads) void channel_amax(const bf16_t* __restrict__ vh, uint32_t* __restrict__ amax_bits,
                                                         int n_pad) {
  constexpr int PIECES = D / 8;             // 16-byte pieces per row
  constexpr int ROWS = kThreads / PIECES;   // rows per pass of the workgroup
  __shared__ float red[ROWS][D + 1];
  const int bh = blockIdx.x;
  const int slice = blockIdx.y;
  const int piece = threadIdx.x % PIECES;
  const int r0 = threadIdx.x / PIECES;
  const int lo = (int)((int64_t)n_pad * slice / gridDim.y);
  const int hi = (int)((int64_t)n_pad * (slice + 1) / gridDim.y);
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bf16_t* base = vh + (size_t)bh * n_pad * D + piece * 8;
  for (int r = lo + r0; r < hi; r += ROWS) {
    const uint4 w = *reinterpret_cast<const uint4*>(base + (size_t)r * D);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m[2 * e] = fmaxf(m[2 * e], fabsf(bf16_to_f32((bf16_t)(u[e] & 0xFFFFu))));
      m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(bf16_to_f32((bf16_t)(u[e] >> 16))));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][piece * 8 + e] = m[e];
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += kThreads) {
    float x = 0.f;
    for (int r = 0; r < ROWS; ++r) x = fmaxf(x, red[r][c]);
    atomicMax(&amax_bits[(size_t)bh * D + c], __float_as_uint(x));
  }
}

// One workgroup per (b, h, 64-key step): encode the step's 64 x D values and
// write its image.
template <int D>
__global__ __launch_bounds__(kThreads) void quantize_step(const bf16_t* __restrict__ vh,
                                                          const uint32_t* __restrict__ amax_bits,
                                                          uint8_t* __restrict__ vt8, int n_pad) {
  constexpr int PIECES = D / 8;
  constexpr int IMG = 64 * D;
  __shared__ __attribute__((aligned(16))) uint8_t img[IMG];
  __shared__ int ex[D];
  const int steps = n_pad / 64;
  const int bh = blockIdx.x / steps;
  const int st = blockIdx.x % steps;
  for (int c = threadIdx.x; c < D; c += kThreads)
    ex[c] = scale_exponent(__uint_as_float(amax_bits[(size_t)bh * D + c]));
  __syncthreads();
  const bf16_t* src = vh + ((size_t)bh * n_pad + (size_t)st * 64) * D;
  for (int p = threadIdx.x; p < 64 * PIECES; p += kThreads) {
    const int key = p / PIECES;
    const int c0 = (p % PIECES) * 8;
    const uint4 w = *reinterpret_cast<const uint4*>(src + (size_t)key * D + c0);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    const int eta = key >> 5, a = (key >> 4) & 1, g = (key >> 3) & 1, i = key & 7;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      const float v = bf16_to_f32((bf16_t)(e & 1 ? u[e / 2] >> 16 : u[e / 2] & 0xFFFFu));
      const float x = ldexpf(v, -ex[c]);  // exact (|x| <= 448)
      const int code = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xFF;
      img[eta * 32 * D + 32 * c + 16 * (g ^ ((c >> 3) & 1)) + 8 * a + i] = (uint8_t)code;
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(vt8 + ((size_t)bh * steps + st) * IMG);
  for (int p = threadIdx.x; p < IMG / 16; p += kThreads) dst[p] = reinterpret_cast<const uint4*>(img)[p];
}

// vscale[i] = 2^e of the channel maximum held in the same word.
__global__ __launch_bounds__(kThreads) void finish_scales(float* __restrict__ vscale, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) vscale[i] = ldexpf(1.f, scale_exponent(vscale[i]));
}

template <int D>
void launch_d(const absh_ctx* c, const bf16_t* vh, uint8_t* vt8, float* vscale, int BH, hipStream_t s) {
  const int n = BH * D;
  uint32_t* amax = reinterpret_cast<uint32_t*>(vscale);  // the scales' words hold the maxima until the end
  const unsigned g1 = (unsigned)((n + kThreads - 1) / kThreads);
  zero_words<<<g1, kThreads, 0, s>>>(amax, n);
  channel_amax<D><<<dim3((unsigned)BH, kAmaxSlices), kThreads, 0, s>>>(vh, amax, c->n_pad);
  quantize_step<D><<<(unsigned)(BH * (c->n_pad / 64)), kThreads, 0, s>>>(vh, amax, vt8, c->n_pad);
  finish_scales<<<g1, kThreads, 0, s>>>(vscale, n);
}

}  // namespace

hipError_t launch_quantize_v(const absh_ctx* c, const void* vh, void* vt8, float* vscale, int BH, int d,
                             hipStream_t s) {
  const bf16_t* v = reinterpret_cast<const bf16_t*>(vh);
  uint8_t* out = reinterpret_cast<uint8_t*>(vt8);
  if (d == 64)
    launch_d<64>(c, v, out, vscale, BH, s);
  else if (d == 128)
    launch_d<128>(c, v, out, vscale, BH, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace absh
