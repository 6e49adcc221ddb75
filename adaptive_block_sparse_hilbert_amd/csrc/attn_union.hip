// Block-sparse attention for groups of neighbouring query blocks walking the
// union of their retained lists (xllm-io review of FVAttn, "Block-Sparse
// Attention Execution"; alanhou.org explainer, "Core Mechanism": each head
// attends only to its selected KV blocks), for gfx950.
//
// Work unit: MEMBERS neighbouring query blocks of one head (four of 64 rows or two
// of 128 rows, 256 query rows in all). The workgroup has eight waves and each
// wave owns 32 query rows of one member. Every entry of the unit's union list is a
// key block plus one flag per member; the workgroup stages the block's K and V^T
// into LDS once, and only the waves whose member retains the block compute on it.
// Waves that share a SIMD belong to different members, so when one skips a block
// the other has the matrix core to itself.
//
// Keys are processed in steps of 64 (a 128-key block is two steps). Per step a
// wave computes, with 32x32x16 bf16 MFMAs and fp32 accumulation:
//   S^T = K Q^T                  two 32x32 tiles, D/16 k-steps each
//   online softmax               fp32, base-2 exponent, lazy rescale of O
//   O^T += V^T P^T               D/32 tiles, four k-steps, P rounded to bf16
// The steps are software-pipelined inside each wave: while the exponentials of
// step k run on the vector ALU, the matrix core computes S^T of step k + 1, and the
// row maxima of step k + 1 are reduced while the value product of step k runs.
//
// With 8-bit values (the review's V quantization, ABSH_VT8 layout) the value
// product of a step is one 32x32x64 fp8 MFMA per O^T tile: P is rounded to E4M3
// (scaled so the row's reference maximum maps to at least 2^6 and nothing exceeds
// 2^8), V^T comes in E4M3 with one power-of-two scale per channel, applied to
// the output at the end. The row sum adds the same rounded probabilities. The
// fp8 MFMA takes byte b of lane (column c, half g) as k index 32 g + b in both
// operands, so byte 8 u + i of the P operand is element 8 (u % 2) + i of S^T tile
// u / 2, i.e. the lane's 32 probabilities in register order, and the V^T image
// stores the matching keys in the same byte positions.
//
// Operand layouts (lane l, column c = l % 32, half g = l / 32). For a 32x32x16
// MFMA the A operand of lane l is row c, k indices 8g..8g+7; the B operand is
// column c, the same k indices; accumulator element r of lane l is row
// 8(r/4) + 4g + r%4 of column c. In S^T the A rows of each 32-key tile are the
// keys with bits 2 and 3 of the row index exchanged, which makes accumulator
// element r hold key 16(r/8) + 8g + r%8: elements 8h..8h+7 of tile T are then
// exactly the eight consecutive keys the lane supplies as B operand of the value
// product for the 16-key step 2T + h. P never leaves registers.
//
// LDS: four slots for K (64 keys x D) and four for V^T (D x 64 keys), each slot
// its own LDS variable. Both are stored as 1 KB blocks of 8 rows x 128 bytes (a
// row's 128-byte chunk h, rows 8b .. 8b + 7): the 16-byte column c of row 8b + r
// sits at (c ^ (b & 1)) * 128 + 16 r. Each block is written by exactly one direct
// global-to-LDS load (16 bytes per lane, lane i at 16 i), whose lanes then cover
// eight whole 128-byte lines of K or V^T in memory. A quarter wave's 16-byte reads
// (16 consecutive rows of one column) fall on 16 distinct bank groups, and each
// lane's read addresses are one per-lane base plus immediates.
//
// Steps go in pairs with one workgroup barrier per pair. Step k reads V^T of step
// k and K of step k + 1, so a pair (k, k + 1) holds V^T of k, k + 1 and K of
// k + 1, k + 2. Its barrier releases the slots of the previous pair, and the pair
// fills them for the next one at four points spread over its two steps (V^T of
// k + 2 at the barrier, K of k + 3 inside step k, V^T of k + 3 after it, K of
// k + 4 inside step k + 1): spread out, the direct loads disturb the compute less
// than in one burst at the barrier.
#include <atomic>
#include <type_traits>

#include "absh_internal.h"

namespace absh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSegments = 8;    // XCDs of an MI355X: one queue segment each
constexpr int kFlagShift = 28;  // union entry: block id | (member m retains it) << (28 + m)
constexpr uint32_t kBlockMask = (1u << kFlagShift) - 1;
constexpr int kStepKeys = 64;

template <int D, int BLK, bool F8>
struct UCfg {
  // base-2 headroom before a row's reference max moves, and the base-2 offset of
  // the probabilities: P = 2^(s - m + OFF) <= 2^(LAZY + OFF), at most 2^8 for E4M3
  static constexpr float LAZY = F8 ? 2.0f : 8.0f;
  static constexpr float OFF = F8 ? 6.0f : 0.0f;
  static constexpr int MEMBERS = BLK >= 128 ? 2 : 4;
  static constexpr int WPM = BLK / 32;         // waves per member
  static constexpr int TW = MEMBERS * WPM;     // waves per workgroup
  static constexpr int THREADS = TW * 64;
  static constexpr int HPB = BLK / kStepKeys;  // steps per key block
  static constexpr int K_BYTES = kStepKeys * D * 2;
  static constexpr int V_BYTES = D * kStepKeys * (F8 ? 1 : 2);
  static constexpr int DS = D / 16;            // k-steps of S^T
  static constexpr int DT = D / 32;            // O^T tiles
  static constexpr int K_SLICES = K_BYTES / 1024;
  static constexpr int V_SLICES = V_BYTES / 1024;
  static constexpr int KPW = K_SLICES / TW;    // direct loads per wave per K slot
  static constexpr int VPW = (V_SLICES + TW - 1) / TW;  // direct loads per wave per V^T slot
  static constexpr int VT_ROW = BLK * 2;       // bytes per row of a bf16 V^T block in HBM
  static_assert(TW == 8, "eight waves per workgroup");
  static_assert(K_SLICES == 8 * KPW, "wave w loads the K blocks w + 8 i");
  static_assert(F8 ? V_SLICES <= 8 * VPW : V_SLICES == 8 * VPW, "wave w loads the V^T blocks w + 8 i");
};

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, uint32_t wave_off,
                                           char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void __attribute__((address_space(3)))*)lds_dst, 16, lane_off,
                                           wave_off, 0, 0);
}

constexpr int kRawBufferFlags = 0x00020000;  // raw buffer descriptor, 32-bit data format

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef const int32_t __attribute__((address_space(4)))* const_i32;
__device__ __forceinline__ const_i32 as_const(const int32_t* p) { return (const_i32)p; }

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

// Maximum (sum) of a lane's value and the value of lane l ^ 32.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D, int BLK, bool F8>
__global__ __launch_bounds__((UCfg<D, BLK, F8>::THREADS)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void union_attn_kernel(const bf16_t* __restrict__ qh, const bf16_t* __restrict__ kh, const char* __restrict__ vt,
                       const float* __restrict__ vscale, bf16_t* __restrict__ oh, AttnLists L,
                       int32_t* __restrict__ counters, int units, int nb, int n_pad, int N, float scale_log2,
                       const int32_t* __restrict__ operm, int H) {
  using C = UCfg<D, BLK, F8>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // One LDS variable per slot: distinct variables let the compiler see that the
  // reads of one slot do not alias the direct loads in flight into another.
  __shared__ __attribute__((aligned(1024))) char ks0[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char ks1[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char ks2[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char ks3[C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs0[C::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs1[C::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs2[C::V_BYTES];
  __shared__ __attribute__((aligned(1024))) char vs3[C::V_BYTES];
  auto kslot = [&](int i) __attribute__((always_inline)) -> char* {
    i &= 3;
    return i == 0 ? ks0 : i == 1 ? ks1 : i == 2 ? ks2 : ks3;
  };
  auto vslot = [&](int i) __attribute__((always_inline)) -> char* {
    i &= 3;
    return i == 0 ? vs0 : i == 1 ? vs1 : i == 2 ? vs2 : vs3;
  };
  __shared__ int s_next[2];
  // The output map is needed only after each unit's last step: parked in LDS, it
  // is not held in scalar registers across the step loop.
  __shared__ const int32_t* s_operm;
  __shared__ int s_heads;

  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();  // for the optional busy record
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets per-wave branches be scalar
  if (tid == 0) {
    s_operm = operm;
    s_heads = H;
  }
  const int col = lane & 31;
  const int g = lane >> 5;
  const int member = wave / C::WPM;
  const int rows0 = (wave % C::WPM) * 32;  // this wave's first row within its member's block
  const int xcd = blockIdx.x & (kSegments - 1);
  const bool dense = L.counts == nullptr;
  const int per_head = (nb + C::MEMBERS - 1) / C::MEMBERS;

  // Direct loads: wave w loads the blocks w, w + 8, ... of a slot, all with row
  // group b = w (K: blocks h * 8 + b; V^T: blocks b = w + 8 i, so b & 1 = w & 1).
  // Lane i fetches row 8 b + i % 8, 16-byte column (i / 8) ^ (b & 1) of the chunk.
  const uint32_t k_lane = (uint32_t)((lane % 8) * (2 * D) + ((lane / 8) ^ (wave & 1)) * 16);
  // (the 8-bit V^T image is stored as LDS wants it: lane i fetches bytes 16 i)
  const uint32_t v_lane = F8 ? (uint32_t)(16 * lane) : (uint32_t)((lane % 8) * C::VT_ROW + ((lane / 8) ^ (wave & 1)) * 16);
  // LDS reads: S^T row c of a tile is key kappa(c) (bits 2 and 3 exchanged); the
  // lane reads 16-byte column g (+ 2 per further k-step) of its row
  const int kappa = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
  auto rd_base = [&](int row) { return (uint32_t)((row / 8) * 1024 + (g ^ ((row / 8) & 1)) * 128 + (row % 8) * 16); };
  const uint32_t k_rd = rd_base(kappa);
  // 8-bit V^T: channel c's 16 bytes of half g sit at 32 c + 16 (g ^ ((c >> 3) & 1)) of
  // each of the two 32 D-byte regions
  const uint32_t v_rd = F8 ? (uint32_t)(32 * col + 16 * (g ^ ((col >> 3) & 1))) : rd_base(col);

  // The two waves of a SIMD (w and w + 4) run the same phases after each barrier.
  // The first wins issue arbitration, so it runs its step as if alone while the
  // second does its vector work under the first one's matrix phases.
  if (wave < 4) __builtin_amdgcn_s_setprio(1);

  const int32_t* bounds = dense ? nullptr : L.sched;
  unsigned dead = 0;
  if (tid == 0) s_next[0] = pull(counters, bounds, units, xcd, dead, L.strict);

  for (int parity = 0;; parity ^= 1) {
    __syncthreads();  // s_next[parity] is published; every wave is done with the previous unit
    const int pos = __builtin_amdgcn_readfirstlane(s_next[parity]);
    if (pos < 0) break;
    // segment position -> unit: through unit_queue (longest first within each run),
    // or head_order (segments following ranks), or in order
    int unit;
    if (L.unit_queue) {
      unit = __builtin_amdgcn_readfirstlane(as_const(L.unit_queue)[pos]);
    } else {
      const int slot = pos / per_head;
      const int bh_ = L.head_order ? __builtin_amdgcn_readfirstlane(as_const(L.head_order)[slot]) : slot;
      unit = bh_ * per_head + (pos - slot * per_head);
    }
    const int bh = unit / per_head;
    const int qb0 = (unit - bh * per_head) * C::MEMBERS;
    const int cnt = dense ? nb : as_const(L.unit_cnt)[unit];
    const_i32 list = dense ? nullptr : as_const(reinterpret_cast<const int32_t*>(L.unit_list) + (size_t)unit * nb);
    uint32_t present = 0;
#pragma unroll
    for (int m = 0; m < C::MEMBERS; ++m)
      if (qb0 + m < nb) present |= 1u << (kFlagShift + m);
    const int nsteps = cnt * C::HPB;
    // union entry of step k (0 past the end)
    auto entry = [&](int k) __attribute__((always_inline)) -> uint32_t {
      if (k >= nsteps) return 0u;
      const int e = C::HPB == 1 ? k : k / C::HPB;
      return list ? (uint32_t)list[e] : ((uint32_t)e | present);
    };
    // keys of step k that exist (the last block of a head can be short)
    auto valid_keys = [&](int k, uint32_t e) __attribute__((always_inline)) -> int {
      const int j = (int)(e & kBlockMask);
      const int half = C::HPB == 1 ? 0 : k % C::HPB;
      return min(kStepKeys, N - j * BLK - half * kStepKeys);
    };
    auto mine = [&](int k, uint32_t e) __attribute__((always_inline)) -> bool {
      return ((e >> (kFlagShift + member)) & 1u) && valid_keys(k, e) > 0;
    };

    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kh + (size_t)bh * n_pad * D), (short)0, n_pad * 2 * D, kRawBufferFlags);
    const size_t v_head = F8 ? (size_t)n_pad * D : (size_t)nb * D * C::VT_ROW;  // bytes per head
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vt + (size_t)bh * v_head), (short)0, (int)v_head, kRawBufferFlags);
    // K slot <- K of step k (union entry e); V^T slot <- V^T of step k
    auto issue_k = [&](int slot, int k, uint32_t e) __attribute__((always_inline)) {
      const uint32_t j = e & kBlockMask;
      const uint32_t half = C::HPB == 1 ? 0u : (uint32_t)(k % C::HPB);
      char* st = kslot(slot);
      const uint32_t row = j * BLK + half * kStepKeys + 8 * wave;
#pragma unroll
      for (int i = 0; i < C::KPW; ++i) load_lds16(krs, k_lane, row * (2 * D) + 128 * i, st + (wave + C::TW * i) * 1024);
    };
    auto issue_v = [&](int slot, int k, uint32_t e) __attribute__((always_inline)) {
      const uint32_t j = e & kBlockMask;
      const uint32_t half = C::HPB == 1 ? 0u : (uint32_t)(k % C::HPB);
      char* st = vslot(slot);
#pragma unroll
      for (int i = 0; i < C::VPW; ++i) {
        const int n = wave + C::TW * i;  // block: V^T rows 8 n .. 8 n + 7 (bf16), bytes 1024 n .. of the image (fp8)
        if (F8) {
          if (n < C::V_SLICES) load_lds16(vrs, v_lane, (j * C::HPB + half) * (uint32_t)C::V_BYTES + 1024 * n, st + n * 1024);
        } else {
          load_lds16(vrs, v_lane, j * (uint32_t)(D * C::VT_ROW) + (8 * n) * C::VT_ROW + half * 128, st + n * 1024);
        }
      }
    };

    // this wave's 32 query rows as the B operand of S^T = K Q^T
    const bool have = (present >> (kFlagShift + member)) & 1u;
    const int qrow = (qb0 + member) * BLK + rows0 + col;
    bf16x8 qf[C::DS];
    if (have) {
      const bf16_t* qsrc = qh + ((size_t)bh * n_pad + qrow) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qsrc + 16 * s);
    }

    // entries of steps k .. k + 4
    uint32_t e0 = entry(0), e1 = entry(1), e2 = entry(2), e3 = entry(3), e4 = entry(4);
    // prologue: K of steps 0, 1, 2 and V^T of steps 0, 1
    if (0 < nsteps) {
      issue_k(0, 0, e0);
      issue_v(0, 0, e0);
    }
    if (1 < nsteps) {
      issue_k(1, 1, e1);
      issue_v(1, 1, e1);
    }
    if (2 < nsteps) issue_k(2, 2, e2);
    if (tid == 0) s_next[parity ^ 1] = pull(counters, bounds, units, xcd, dead, L.strict);

    f32x16 o[C::DT];
#pragma unroll
    for (int t = 0; t < C::DT; ++t) o[t] = f32x16{};
    float l_run = 0.f;        // this lane's share of its row's sum of (rounded) probabilities
    float m_run = -INFINITY;  // the row's reference max, base-2 scaled
    f32x16 S[2];              // S^T of the step whose softmax comes next

    // The reference max moves only when a row's step max exceeds it by more than
    // LAZY (base 2): probabilities stay below 2^(LAZY + OFF) and O is rescaled
    // rarely. The result is the same softmax.
    auto rescale_to = [&](float m_blk) __attribute__((always_inline)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int t = 0; t < C::DT; ++t) o[t] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    };
    auto rescale = [&](float m_blk) __attribute__((always_inline)) {
      if (__any(m_blk > m_run + C::LAZY)) rescale_to(m_blk);
    };
    // probabilities of elements r0 .. r0 + n - 1 (n even) of S^T tile T, as bf16 into
    // the B operand of 16-key value step 2T + r0 / 8, and their row sum
    auto probs = [&](bf16x8 (&pf)[4], int T, int r0, int n) __attribute__((always_inline)) {
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int r = r0; r < r0 + n; r += 2) {
        const int u = 2 * T + r / 8, i = r % 8;
        pf[u][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[T][r], scale_log2, -m_run));
        pf[u][i + 1] = (__bf16)__builtin_amdgcn_exp2f(fmaf(S[T][r + 1], scale_log2, -m_run));
        // row sum of the same bf16 probabilities that enter the value product
        l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[u][i], pf[u][i + 1]}, one2, l_run, false);
      }
    };
    // masks element r of S^T tile T past `valid` keys: it is key 32 T + 16 (r / 8) + 8 g + r % 8
    auto mask = [&](int T, int r, int valid) __attribute__((always_inline)) {
      if (32 * T + 16 * (r / 8) + (r % 8) >= valid - 8 * g) S[T][r] = -INFINITY;
    };
    // 8-bit value product of one step: the 32 probabilities of both S^T tiles,
    // rounded to E4M3 four to a register (tile T elements 4 w' .. 4 w' + 3 in
    // register 4 T + w'), their row sum from the rounded values, then one fp8 MFMA
    // per O^T tile, its V^T operand the 16 bytes at vbase + 1024 t of each region.
    auto pv8 = [&](const char* vbase) __attribute__((always_inline)) {
      // V^T operands one tile ahead of their MFMA (tile 0 under the exponentials)
      auto frag = [&](int t) __attribute__((always_inline)) -> i32x8 {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(vbase + 1024 * t);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(vbase + 1024 * t + 32 * D);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      i32x8 va = frag(0);
      const float bias = C::OFF - m_run;
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
      i32x8 pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int T = w / 4, r = 4 * (w % 4);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S[T][r], scale_log2, bias));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S[T][r + 1], scale_log2, bias));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(S[T][r + 2], scale_log2, bias));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(S[T][r + 3], scale_log2, bias));
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, pk, true);
        pf[w] = pk;
        // E4M3 values are exact in bf16: the sum adds exactly what the MFMA multiplies
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pk, 1.0f, false), one2,
                                                l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pk, 1.0f, true), one2,
                                                l_run, false);
      }
#pragma unroll
      for (int t = 0; t < C::DT; ++t) {
        const i32x8 a = va;
        if (t + 1 < C::DT) va = frag(t + 1);
        o[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, o[t], 0, 0, 0, 0, 0, 0);
      }
    };

    // One step as a hand-ordered instruction stream. The matrix instructions go
    // in this order: value product of 16-key steps 0 and 1 (phase 0), S^T tile 0
    // of the next step (phase 1), value product of 16-key steps 2 and 3 (phase 2),
    // S^T tile 1 (phase 3). Each reads one 16-byte LDS fragment, fetched DIST
    // instructions ahead. The vector work rides along: the probabilities of tile 0
    // come first, those of tile 1 under phase 0, the row maxima of the new tile 0
    // under phase 3. Scheduling barriers keep each group of one LDS read, one
    // matrix instruction and its share of vector work in place.
    constexpr int NPV = 2 * C::DT;  // value-product instructions per phase
    constexpr int NQK = C::DS;      // S^T instructions per tile
    constexpr int DIST = 3;
    auto body = [&](auto pv_c, auto qk_c, auto masked_c, const char* kbase, const char* vbase, int valid)
                    __attribute__((always_inline)) -> float {
      constexpr bool DP = decltype(pv_c)::value;
      constexpr bool DQ = decltype(qk_c)::value;
      constexpr bool MK = decltype(masked_c)::value;
      constexpr int P0 = DP ? NPV : 0, P1 = DQ ? NQK : 0;
      constexpr int NOPS = 2 * (P0 + P1);
      // op i -> LDS fragment address
      auto frag = [&](int i) __attribute__((always_inline)) -> const bf16x8* {
        const int ph = i < P0 ? 0 : i < P0 + P1 ? 1 : i < 2 * P0 + P1 ? 2 : 3;
        const int j = ph == 0 ? i : ph == 1 ? i - P0 : ph == 2 ? i - P0 - P1 : i - 2 * P0 - P1;
        if (ph == 0 || ph == 2) {
          const int u = (ph == 0 ? 0 : 2) + j / C::DT, t = j % C::DT;
          return reinterpret_cast<const bf16x8*>(vbase + t * 4096 + u * 256);
        }
        // 32-key tile T, k-step j: chunk j / 4, row groups 4 T .. 4 T + 3
        const int T = ph == 1 ? 0 : 1;
        return reinterpret_cast<const bf16x8*>(kbase + ((j / 4) * 8 + 4 * T) * 1024 + (j % 4) * 256);
      };
      bf16x8 fr[DIST + 1];
      bf16x8 pf[4];
      float mx0 = -INFINITY;
#pragma unroll
      for (int i = 0; i < DIST; ++i)
        if (i < NOPS) fr[i] = *frag(i);
      if (DP) probs(pf, 0, 0, 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NOPS; ++i) {
        if (i + DIST < NOPS) fr[(i + DIST) % (DIST + 1)] = *frag(i + DIST);
        const bf16x8 a = fr[i % (DIST + 1)];
        const int ph = i < P0 ? 0 : i < P0 + P1 ? 1 : i < 2 * P0 + P1 ? 2 : 3;
        const int j = ph == 0 ? i : ph == 1 ? i - P0 : ph == 2 ? i - P0 - P1 : i - 2 * P0 - P1;
        if (ph == 0 || ph == 2) {
          const int u = (ph == 0 ? 0 : 2) + j / C::DT, t = j % C::DT;
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[u], o[t], 0, 0, 0);
        } else {
          const int T = ph == 1 ? 0 : 1;
          S[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[j], j == 0 ? f32x16{} : S[T], 0, 0, 0);
        }
        if (ph == 0) {
          // probabilities of tile 1, spread over phase 0
          constexpr int PER = P0 > 0 ? 16 / P0 : 16;
          probs(pf, 1, j * PER, PER);
        } else if (ph == 3) {
          // row maxima of the new tile 0, spread over phase 3
          constexpr int PER = P1 > 0 ? 16 / P1 : 16;
#pragma unroll
          for (int r = j * PER; r < j * PER + PER; ++r) {
            if (MK) mask(0, r, valid);
            mx0 = fmaxf(mx0, S[0][r]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!DQ) return -INFINITY;
      float mx = mx0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MK) mask(1, r, valid);
        mx = fmaxf(mx, S[1][r]);
      }
      return max_across_halves(mx) * scale_log2;
    };
    auto fused = [&](const char* kbase, const char* vbase, int valid, auto masked_c) __attribute__((always_inline))
        -> float {
      return body(T_(), T_(), masked_c, kbase, vbase, valid);
    };
    auto solo_pv = [&](const char* vbase) __attribute__((always_inline)) {
      if constexpr (F8)
        pv8(vbase);
      else
        body(T_(), F_(), F_(), nullptr, vbase, kStepKeys);
    };
    auto solo_qk = [&](const char* kbase, int valid, auto masked_c) __attribute__((always_inline)) -> float {
      return body(F_(), T_(), masked_c, kbase, nullptr, valid);
    };

    // step 0: S^T only
    wait_vm<0>();
    __syncthreads();
    {
      const int vk = valid_keys(0, e0);
      const float m = vk < kStepKeys ? solo_qk(ks0 + k_rd, vk, T_()) : solo_qk(ks0 + k_rd, vk, F_());
      if (mine(0, e0)) rescale(m);
    }
    // Pair start (k even): everything issued at the previous pair has landed, all
    // waves are done with steps k - 2 and k - 1, and their slots take V^T of
    // k + 2, k + 3 and K of k + 3, k + 4: the first here, the others at
    // load_k3 / load_v3 / load_k4 further into the pair.
    auto pair_start = [&](int k) __attribute__((always_inline)) {
      wait_vm<0>();
      __syncthreads();
      if (k + 2 < nsteps) issue_v(k + 2, k + 2, e2);
    };
    auto load_k3 = [&](int k) __attribute__((always_inline)) {
      if (k + 3 < nsteps) issue_k(k + 3, k + 3, e3);
    };
    auto load_v3 = [&](int k) __attribute__((always_inline)) {
      if (k + 3 < nsteps) issue_v(k + 3, k + 3, e3);
    };
    auto load_k4 = [&](int k) __attribute__((always_inline)) {
      if (k + 4 < nsteps) issue_k(k + 4, k + 4, e4);
    };
    auto pair_end = [&](int k) __attribute__((always_inline)) {
      e0 = e2;
      e1 = e3;
      e2 = e4;
      e3 = entry(k + 5);
      e4 = entry(k + 6);
    };
    // Steady state: step k (slots known at compile time through the unrolling
    // below, so the compiler need not wait for loads in flight into other slots)
    // with S^T of step k + 1 unmasked. The step is two straight-line parts that a
    // wave skips when its query block does not retain the block: softmax + value
    // product of step k, then S^T of step k + 1.
    auto step_fast = [&](int k, auto slot_c, uint32_t ek, uint32_t ek1, auto mid) __attribute__((always_inline)) {
      constexpr int SL = decltype(slot_c)::value;
      if (mine(k, ek)) solo_pv(vslot(SL) + v_rd);
      mid();
      if (mine(k + 1, ek1)) {
        const float m = body(F_(), T_(), F_(), kslot(SL + 1) + k_rd, nullptr, kStepKeys);
        if (__any(m > m_run + C::LAZY)) rescale_to(m);
      }
    };
    // Steps next to a head's short last block: run-time slots and masking.
    auto step_tail = [&](int k, uint32_t ek, uint32_t ek1) __attribute__((always_inline)) {
      const char* vbase = vslot(k) + v_rd;
      const char* kbase = kslot(k + 1) + k_rd;
      const bool now = mine(k, ek);
      const bool next = k + 1 < nsteps && mine(k + 1, ek1);
      const int vk1 = next ? valid_keys(k + 1, ek1) : kStepKeys;
      float m_blk = -INFINITY;
      if (now && next && F8) {
        solo_pv(vbase);
        m_blk = vk1 < kStepKeys ? solo_qk(kbase, vk1, T_()) : solo_qk(kbase, vk1, F_());
      } else if (now && next)
        m_blk = vk1 < kStepKeys ? fused(kbase, vbase, vk1, T_()) : fused(kbase, vbase, vk1, F_());
      else if (now)
        solo_pv(vbase);
      else if (next)
        m_blk = vk1 < kStepKeys ? solo_qk(kbase, vk1, T_()) : solo_qk(kbase, vk1, F_());
      if (next) rescale(m_blk);
    };
    // first step whose keys run short (the partial last block of a head), else nsteps
    int first_masked = nsteps;
    if (nsteps > 0) {
      const int nj = N - (nb - 1) * BLK;  // keys of the head's last block
      if (nj < BLK && (entry(nsteps - 1) & kBlockMask) == (uint32_t)(nb - 1))
        first_masked = nsteps - C::HPB + nj / kStepKeys;
    }
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // pairs whose steps both compute unmasked S^T for their next step: k + 2 < first_masked
    int k = 0;
    while (k + 2 < first_masked) {
      pair_start(k);
      step_fast(k, I0(), e0, e1, [&]() { load_k3(k); });
      load_v3(k);
      step_fast(k + 1, I1(), e1, e2, [&]() { load_k4(k); });
      pair_end(k);
      k += 2;
      if (k + 2 >= first_masked) break;
      pair_start(k);
      step_fast(k, I2(), e0, e1, [&]() { load_k3(k); });
      load_v3(k);
      step_fast(k + 1, I3(), e1, e2, [&]() { load_k4(k); });
      pair_end(k);
      k += 2;
    }
    for (; k < nsteps; k += 2) {
      pair_start(k);
      load_k3(k);
      step_tail(k, e0, e1);
      load_v3(k);
      load_k4(k);
      if (k + 1 < nsteps) step_tail(k + 1, e1, e2);
      pair_end(k);
    }

    if (have) {
      const float l = sum_across_halves(l_run);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      // Hilbert order (every padded row), or the caller's grid order: row r of
      // head (b, h) is token perm[r] of batch b, and pad rows are not written
      const int32_t* om = s_operm;
      const int nh = s_heads;
      const bool keep = om == nullptr || qrow < N;
      const size_t out_row = om == nullptr ? (size_t)bh * n_pad + qrow
                                           : ((size_t)(bh / nh) * N + (keep ? om[qrow] : 0)) * nh + bh % nh;
      bf16_t* orow = oh + out_row * D;
#pragma unroll
      for (int t = 0; t < C::DT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // elements 4 q .. 4 q + 3 of tile t: channels 32 t + 8 q + 4 g + 0 .. 3
          float sc[4] = {inv, inv, inv, inv};
          if constexpr (F8) {
            const float4 vs = *reinterpret_cast<const float4*>(vscale + (size_t)bh * D + 32 * t + 8 * q + 4 * g);
            sc[0] *= vs.x;
            sc[1] *= vs.y;
            sc[2] *= vs.z;
            sc[3] *= vs.w;
          }
          uint2 w;
          w.x = (uint32_t)f32_to_bf16(o[t][4 * q] * sc[0]) | ((uint32_t)f32_to_bf16(o[t][4 * q + 1] * sc[1]) << 16);
          w.y = (uint32_t)f32_to_bf16(o[t][4 * q + 2] * sc[2]) | ((uint32_t)f32_to_bf16(o[t][4 * q + 3] * sc[3]) << 16);
          if (keep) *reinterpret_cast<uint2*>(orow + 32 * t + 8 * q + 4 * g) = w;
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

template <int D, int BLK, bool F8>
hipError_t launch(const absh_ctx* c, const void* qh, const void* kh, const void* vt, const float* vscale, void* oh,
                  int B, int H, const AttnLists& L, bool dense, hipStream_t s, bool grid_out) {
  using C = UCfg<D, BLK, F8>;
  // resident workgroups per CU for this instantiation (one gfx950 value; computed once,
  // an atomic so that concurrent first calls from several threads are well defined)
  static std::atomic<int> occupancy{0};
  int per_cu = occupancy.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, union_attn_kernel<D, BLK, F8>, C::THREADS, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    occupancy.store(per_cu, std::memory_order_relaxed);
  }
  const int units = B * H * ((c->nb + C::MEMBERS - 1) / C::MEMBERS);
  const int grid = c->num_cus * per_cu;
  const float scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)D));
  AttnLists Lk = L;
  if (dense) Lk = AttnLists{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, C::MEMBERS};
  if (grid > c->num_cus * kMaxAttnWgPerCu) return hipErrorInvalidConfiguration;  // wg_busy's bound
  int32_t* counters = Lk.counters ? Lk.counters : c->counters;
  union_attn_kernel<D, BLK, F8><<<grid, C::THREADS, 0, s>>>(
      reinterpret_cast<const bf16_t*>(qh), reinterpret_cast<const bf16_t*>(kh), reinterpret_cast<const char*>(vt),
      vscale, reinterpret_cast<bf16_t*>(oh), Lk, counters, units, c->nb, c->n_pad, c->N, scale_log2,
      grid_out ? c->perm : nullptr, H);
  return hipGetLastError();
}

}  // namespace

bool union_attention_supported(int d, int block, int members) {
  return (d == 64 || d == 128) && ((block == 64 && members == 4) || (block == 128 && members == 2));
}

hipError_t launch_union_attention(const absh_ctx* c, const void* qh, const void* kh, const void* vt,
                                  const float* vscale, void* oh, int B, int H, int d, const AttnLists* lists,
                                  hipStream_t s, bool grid_out) {
  AttnLists L = lists ? *lists : AttnLists{};
  const bool dense = lists == nullptr;
#define ABSH_UNION(DD, BB)                                                                              \
  if (d == DD && c->block == BB)                                                                        \
    return vscale ? launch<DD, BB, true>(c, qh, kh, vt, vscale, oh, B, H, L, dense, s, grid_out)        \
                  : launch<DD, BB, false>(c, qh, kh, vt, nullptr, oh, B, H, L, dense, s, grid_out);
  ABSH_UNION(64, 64)
  ABSH_UNION(64, 128)
  ABSH_UNION(128, 64)
  ABSH_UNION(128, 128)
#undef ABSH_UNION
  return hipErrorInvalidValue;
}

}  // namespace absh
