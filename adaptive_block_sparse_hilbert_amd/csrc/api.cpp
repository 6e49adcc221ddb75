// C ABI of the library: argument validation (always before any HIP call),
// workspace layout, and the launch sequence of each entry point on the caller's
// stream. See include/absh.h for the contract of every function.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>

#include "absh_internal.h"

namespace {

thread_local std::string g_last_error;

absh_status fail(absh_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

absh_status hip_fail(hipError_t e, const char* where) {
  return fail(ABSH_EHIP, "%s: %s", where, hipGetErrorString(e));
}

#define ABSH_HIP(call, where)                     \
  do {                                            \
    hipError_t e_ = (call);                       \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxNb = 2048;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Route workspace of absh_route_static: one file-scope device array, of which each
// GPU the library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, so its device address on each GPU is looked
// up once (scratch_setup, with that GPU current) and only that address is used.
constexpr size_t kStaticScratchBytes = (size_t)ABSH_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `device`, which must be current.
hipError_t scratch_setup(int device) {
  if (device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

// Makes a GPU current for the rest of an entry point and gives the caller's
// current device back when the entry point returns (launches already queued on
// a stream are not affected by the switch back).
class DeviceScope {
 public:
  DeviceScope() = default;
  DeviceScope(const DeviceScope&) = delete;
  DeviceScope& operator=(const DeviceScope&) = delete;
  ~DeviceScope() {
    if (switched_) (void)hipSetDevice(prev_);
  }
  absh_status enter(int device) {
    ABSH_HIP(hipGetDevice(&prev_), "hipGetDevice");
    if (prev_ != device) {
      ABSH_HIP(hipSetDevice(device), "hipSetDevice");
      switched_ = true;
    }
    return ABSH_OK;
  }

 private:
  int prev_ = -1;
  bool switched_ = false;
};

absh_status check_ctx(const absh_ctx* c) {
  if (!c) return fail(ABSH_EINVAL, "ctx is NULL");
  return ABSH_OK;
}

absh_status check_shape(const absh_ctx* c, int B, int H, int d) {
  if (B < 1 || H < 1) return fail(ABSH_EINVAL, "B and H must be >= 1 (got B=%d H=%d)", B, H);
  if (d != 64 && d != 128) return fail(ABSH_EUNSUPPORTED, "head dim %d not built (64 or 128)", d);
  const double rows = (double)B * H * c->n_pad * d;
  if (rows >= 9.0e18) return fail(ABSH_EINVAL, "tensor too large");
  if ((double)B * H * c->nb >= 2147483647.0) return fail(ABSH_EINVAL, "B*H*nb must fit in int32");
  return ABSH_OK;
}

// Byte offsets of the route workspace regions.
struct WsLayout {
  size_t qbar, kbar, S, target, info, chunk_hist, scan_sums, slack_aux, rank, owner, budget, total;
};

// scores: room for the score matrix (absh_route); without it the selection computes
// the scores on chip (absh_route_static)
WsLayout ws_layout(const absh_ctx* c, int B, int H, int d, bool scores = true) {
  const size_t tiles = (size_t)B * H * c->nb;
  WsLayout w;
  size_t off = 0;
  w.qbar = off; off = align_up(off + tiles * d * sizeof(float));
  w.kbar = off; off = align_up(off + tiles * d * sizeof(float));
  w.S = (size_t)-1;
  if (scores) {
    w.S = off;
    off = align_up(off + tiles * c->nb * sizeof(float));
  }
  w.target = off; off = align_up(off + tiles * sizeof(int32_t));
  w.info = off; off = align_up(off + 4 * sizeof(int64_t));
  w.chunk_hist = off; off = align_up(off + (size_t)absh::queue_chunks((int)tiles) * (c->nb + 1) * sizeof(int32_t));
  w.scan_sums = off; off = align_up(off + (size_t)absh::queue_scan_tiles((int)tiles, c->nb) * sizeof(int32_t));
  w.slack_aux = off; off = align_up(off + (size_t)absh::slack_aux_words((int)tiles) * sizeof(int32_t));
  w.rank = off; off = align_up(off + tiles * sizeof(int32_t));
  w.owner = off; off = align_up(off + (size_t)B * H * sizeof(int32_t));
  w.budget = off; off = align_up(off + 8 * sizeof(int64_t));
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

int absh_version(void) { return 210; }

const char* absh_status_string(int status) {
  switch (status) {
    case ABSH_OK: return "ABSH_OK";
    case ABSH_EINVAL: return "ABSH_EINVAL";
    case ABSH_EUNSUPPORTED: return "ABSH_EUNSUPPORTED";
    case ABSH_EWORKSPACE: return "ABSH_EWORKSPACE";
    case ABSH_ENODEV: return "ABSH_ENODEV";
    case ABSH_EHIP: return "ABSH_EHIP";
    default: return "ABSH_UNKNOWN";
  }
}

const char* absh_last_error(void) { return g_last_error.c_str(); }

absh_status absh_create(absh_ctx** out, int T, int Y, int X, int block, int device, void* stream) {
  g_last_error.clear();
  if (!out) return fail(ABSH_EINVAL, "ctx output pointer is NULL");
  *out = nullptr;
  if (T < 1 || Y < 1 || X < 1) return fail(ABSH_EINVAL, "grid extents must be >= 1 (got %d x %d x %d)", T, Y, X);
  if (block != 16 && block != 64 && block != 128)
    return fail(ABSH_EUNSUPPORTED, "block size %d not built (16, 64 or 128)", block);
  const long long N = (long long)T * Y * X;
  if (N > (1LL << 30)) return fail(ABSH_EINVAL, "grid too large (%lld tokens)", N);
  int m = 1;
  while ((1 << m) < T || (1 << m) < Y || (1 << m) < X) ++m;
  if (m > 10) return fail(ABSH_EINVAL, "grid extent above 1024 along an axis");
  if (device < 0) return fail(ABSH_EINVAL, "device index %d < 0", device);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    (void)hipGetLastError();
    return fail(ABSH_ENODEV, "no HIP device available");
  }
  if (device >= ndev) return fail(ABSH_ENODEV, "device %d does not exist (%d present)", device, ndev);
  if (device >= kMaxDevices) return fail(ABSH_EUNSUPPORTED, "device index %d above %d", device, kMaxDevices - 1);
  DeviceScope dev;
  if (absh_status st = dev.enter(device)) return st;
  ABSH_HIP(scratch_setup(device), "absh_create: static scratch address");

  absh_ctx* c = new (std::nothrow) absh_ctx();
  if (!c) return fail(ABSH_EINVAL, "out of host memory");
  c->T = T; c->Y = Y; c->X = X; c->block = block;
  c->N = (int)N;
  c->nb = (int)((N + block - 1) / block);
  c->n_pad = c->nb * block;
  c->m = m;
  c->device = device;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int chunks = absh::hilbert_chunks(m);
  int32_t* chunk_counts = nullptr;
  hipError_t e = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipMalloc(&c->perm, sizeof(int32_t) * N);
  if (e == hipSuccess) e = hipMalloc(&c->inv, sizeof(int32_t) * N);
  if (e == hipSuccess) e = hipMalloc(&c->counters, sizeof(int32_t) * 16);
  if (e == hipSuccess) e = hipMemsetAsync(c->counters, 0, sizeof(int32_t) * 16, s);
  if (e == hipSuccess) e = hipMalloc(&chunk_counts, sizeof(int32_t) * chunks);
  if (e == hipSuccess) e = absh::launch_hilbert_perm(c, chunk_counts, chunks, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (chunk_counts) (void)hipFree(chunk_counts);
  if (e != hipSuccess) {
    absh_status st = hip_fail(e, "absh_create");
    if (c->perm) (void)hipFree(c->perm);
    if (c->inv) (void)hipFree(c->inv);
    if (c->counters) (void)hipFree(c->counters);
    delete c;
    return st;
  }
  *out = c;
  return ABSH_OK;
}

absh_status absh_destroy(absh_ctx* c) {
  g_last_error.clear();
  if (!c) return ABSH_OK;
  DeviceScope dev;
  absh_status st = dev.enter(c->device);
  if (st == ABSH_OK) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) st = hip_fail(e, "absh_destroy");
  }
  if (c->perm) (void)hipFree(c->perm);
  if (c->inv) (void)hipFree(c->inv);
  if (c->counters) (void)hipFree(c->counters);
  delete c;
  return st;
}

absh_status absh_dims(const absh_ctx* c, int* N, int* nb, int* n_pad) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (N) *N = c->N;
  if (nb) *nb = c->nb;
  if (n_pad) *n_pad = c->n_pad;
  return ABSH_OK;
}

absh_status absh_perm(const absh_ctx* c, const int32_t** perm, const int32_t** inv) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (perm) *perm = c->perm;
  if (inv) *inv = c->inv;
  return ABSH_OK;
}

absh_status absh_perm_copy(const absh_ctx* c, int32_t* perm_dst, int32_t* inv_dst, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t bytes = sizeof(int32_t) * c->N;
  if (perm_dst) ABSH_HIP(hipMemcpyAsync(perm_dst, c->perm, bytes, hipMemcpyDeviceToDevice, s), "absh_perm_copy");
  if (inv_dst) ABSH_HIP(hipMemcpyAsync(inv_dst, c->inv, bytes, hipMemcpyDeviceToDevice, s), "absh_perm_copy");
  return ABSH_OK;
}

absh_status absh_permute(absh_ctx* c, const void* x, absh_dtype xt, void* xh, int B, int H, int d,
                         absh_layout layout, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!x || !xh) return fail(ABSH_EINVAL, "x or xh is NULL");
  if (xt != ABSH_BF16 && xt != ABSH_F32) return fail(ABSH_EINVAL, "unknown dtype %d", (int)xt);
  if (layout != ABSH_ROWS && layout != ABSH_VT && layout != ABSH_ROWS_F32)
    return fail(ABSH_EINVAL, "unknown layout %d", (int)layout);
  if (!aligned16(x) || !aligned16(xh)) return fail(ABSH_EINVAL, "x and xh must be 16-byte aligned");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_permute(c, x, xt == ABSH_F32, xh, B, H, d, (int)layout, reinterpret_cast<hipStream_t>(stream)),
           "absh_permute");
  return ABSH_OK;
}

absh_status absh_permute_pool(absh_ctx* c, const void* x, absh_dtype xt, void* xh, float* xbar, int B, int H, int d,
                              absh_layout layout, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!x || !xh || !xbar) return fail(ABSH_EINVAL, "x, xh or xbar is NULL");
  if (xt != ABSH_BF16 && xt != ABSH_F32) return fail(ABSH_EINVAL, "unknown dtype %d", (int)xt);
  if (layout != ABSH_ROWS && layout != ABSH_ROWS_F32)
    return fail(ABSH_EINVAL, "absh_permute_pool writes rows: layout ABSH_ROWS or ABSH_ROWS_F32 (got %d)", (int)layout);
  if (!aligned16(x) || !aligned16(xh) || !aligned16(xbar))
    return fail(ABSH_EINVAL, "x, xh and xbar must be 16-byte aligned");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_permute_pool(c, x, xt == ABSH_F32, xh, xbar, B, H, d, (int)layout,
                                     reinterpret_cast<hipStream_t>(stream)),
           "absh_permute_pool");
  return ABSH_OK;
}

absh_status absh_unpermute(absh_ctx* c, const void* oh, void* o, int B, int H, int d, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!oh || !o) return fail(ABSH_EINVAL, "oh or o is NULL");
  if (!aligned16(oh) || !aligned16(o)) return fail(ABSH_EINVAL, "oh and o must be 16-byte aligned");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_unpermute(c, oh, o, B, H, d, reinterpret_cast<hipStream_t>(stream)), "absh_unpermute");
  return ABSH_OK;
}

absh_status absh_pool(absh_ctx* c, const void* xh, float* xbar, int B, int H, int d, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!xh || !xbar) return fail(ABSH_EINVAL, "xh or xbar is NULL");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_pool(c, xh, 0, xbar, B, H, d, reinterpret_cast<hipStream_t>(stream)), "absh_pool");
  return ABSH_OK;
}

absh_status absh_block_scores(absh_ctx* c, const float* qbar, const float* kbar, float* s, int B, int H, int d,
                              void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!qbar || !kbar || !s) return fail(ABSH_EINVAL, "qbar, kbar or s is NULL");
  if (!aligned16(qbar) || !aligned16(kbar)) return fail(ABSH_EINVAL, "qbar and kbar must be 16-byte aligned");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_scores(c, qbar, kbar, s, B * H, d, reinterpret_cast<hipStream_t>(stream)),
           "absh_block_scores");
  return ABSH_OK;
}

int absh_lists_units(const absh_ctx* c, int B, int H, int schedule) {
  if (!c || B < 1 || H < 1 || schedule < ABSH_SCHED_ORDER || schedule > ABSH_SCHED_RANKS) return 0;
  if ((double)B * H * c->nb >= 2147483647.0) return 0;
  return absh::unit_count(c, B * H, absh::unit_members(c, schedule));
}

}  // extern "C"

namespace {

// The buffers of absh_lists in field order, each 256-byte aligned inside one
// arena; units = the most any schedule makes. Offsets in bytes; -1 = absent.
struct ListsLayout {
  size_t counts, kv_idx, order, work, L, queue, sched, unit_list, unit_cnt, head_order, rank_info, unit_queue, pull,
      total;
};

bool lists_layout(const absh_ctx* c, int B, int H, int order_depth, ListsLayout* l) {
  if (!c || B < 1 || H < 1 || order_depth < 0 || order_depth > 64) return false;
  if ((double)B * H * c->nb >= 2147483647.0) return false;
  const size_t BH = (size_t)B * H, tiles = BH * c->nb, nb = (size_t)c->nb;
  size_t units = 0;
  for (int sch = ABSH_SCHED_ORDER; sch <= ABSH_SCHED_RANKS; ++sch)
    units = std::max(units, (size_t)absh::unit_count(c, B * H, absh::unit_members(c, sch)));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  l->counts = take(tiles * 4);
  l->kv_idx = take(tiles * nb * 2);
  l->order = order_depth > 0 ? take(tiles * (size_t)order_depth * 2) : (size_t)-1;
  l->work = take(BH * 4);
  l->L = take(BH * 4);
  l->queue = take(tiles * 4);
  l->sched = take(10 * 4);
  l->unit_list = take(units * nb * 4);
  l->unit_cnt = take(units * 4);
  l->head_order = take(BH * 4);
  l->rank_info = take(ABSH_RANK_INFO * 8);
  l->unit_queue = take(units * 4);
  l->pull = take(ABSH_PULL_WORDS * 4);
  l->total = off;
  return true;
}

}  // namespace

extern "C" {

size_t absh_lists_bytes(const absh_ctx* c, int B, int H, int order_depth) {
  ListsLayout l;
  return lists_layout(c, B, H, order_depth, &l) ? l.total : 0;
}

absh_status absh_lists_carve(const absh_ctx* c, int B, int H, int order_depth, void* arena, size_t arena_bytes,
                             absh_lists* out) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (!arena || !out) return fail(ABSH_EINVAL, "arena or out is NULL");
  ListsLayout l;
  if (!lists_layout(c, B, H, order_depth, &l)) return fail(ABSH_EINVAL, "bad shape or order_depth");
  if (arena_bytes < l.total) return fail(ABSH_EWORKSPACE, "arena has %zu bytes, %zu needed", arena_bytes, l.total);
  if ((reinterpret_cast<uintptr_t>(arena) & (kAlign - 1)) != 0)
    return fail(ABSH_EINVAL, "arena must be %zu-byte aligned", kAlign);
  char* base = reinterpret_cast<char*>(arena);
  *out = absh_lists{};
  out->counts = reinterpret_cast<int32_t*>(base + l.counts);
  out->kv_idx = reinterpret_cast<int16_t*>(base + l.kv_idx);
  out->order = l.order == (size_t)-1 ? nullptr : reinterpret_cast<int16_t*>(base + l.order);
  out->work = reinterpret_cast<int32_t*>(base + l.work);
  out->L = reinterpret_cast<float*>(base + l.L);
  out->queue = reinterpret_cast<int32_t*>(base + l.queue);
  out->sched = reinterpret_cast<int32_t*>(base + l.sched);
  out->unit_list = reinterpret_cast<uint32_t*>(base + l.unit_list);
  out->unit_cnt = reinterpret_cast<int32_t*>(base + l.unit_cnt);
  out->head_order = reinterpret_cast<int32_t*>(base + l.head_order);
  out->rank_info = reinterpret_cast<double*>(base + l.rank_info);
  out->unit_queue = reinterpret_cast<int32_t*>(base + l.unit_queue);
  out->pull = reinterpret_cast<int32_t*>(base + l.pull);
  out->schedule = -1;
  return ABSH_OK;
}

int absh_attn_workgroups(const absh_ctx* c) { return c ? c->num_cus * absh::kMaxAttnWgPerCu : 0; }

size_t absh_route_workspace_bytes(const absh_ctx* c, int B, int H, int d) {
  if (!c || B < 1 || H < 1 || d < 1) return 0;
  return ws_layout(c, B, H, d).total;
}

size_t absh_workspace_bytes(const absh_ctx* c, int B, int H, int d) { return absh_route_workspace_bytes(c, B, H, d); }

}  // extern "C"

namespace {

// The routing of absh_route; `scores`: the score matrix goes through the workspace
// (score and select kernels), else the selection computes the scores on chip.
// means_q / means_k: block means the caller already has (absh_route_means); then
// qh and kh are not read and the pooling is skipped. check_only: validate the
// arguments and return before any HIP call.
absh_status route_impl(absh_ctx* c, const void* qh, const void* kh, absh_dtype qk_type, int B, int H, int d,
                       const absh_route_opts* opts, absh_lists* out, void* ws, size_t ws_bytes, void* stream,
                       bool scores, const float* means_q = nullptr, const float* means_k = nullptr,
                       bool check_only = false) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!opts || !out) return fail(ABSH_EINVAL, "opts or out is NULL");
  if (opts->router != ABSH_ROUTER_TOPP && opts->router != ABSH_ROUTER_WINDOW_ANCHOR)
    return fail(ABSH_EINVAL, "unknown router %d", opts->router);
  const bool structured = opts->router == ABSH_ROUTER_WINDOW_ANCHOR;
  const bool given = means_q != nullptr;
  if (given && structured) return fail(ABSH_EINVAL, "routing from block means takes the Top-p router");
  if (structured) {
    if (opts->window < 0 || opts->anchor_stride < 0 || opts->anchor_shift < 0 || opts->step < 0)
      return fail(ABSH_EINVAL, "window, anchor_stride, anchor_shift and step must be >= 0");
    if (opts->slack_frac != 0.0 || opts->order_depth != 0)
      return fail(ABSH_EINVAL, "the window/anchor router takes no slack_frac and no order_depth");
    if (opts->schedule == ABSH_SCHED_RANKS)
      return fail(ABSH_EUNSUPPORTED, "the window/anchor router has no importance order for ABSH_SCHED_RANKS");
  } else {
    if (given) {
      if (!means_k) return fail(ABSH_EINVAL, "kbar is NULL");
      if (!aligned16(means_q) || !aligned16(means_k)) return fail(ABSH_EINVAL, "qbar and kbar must be 16-byte aligned");
    } else {
      if (!qh || !kh) return fail(ABSH_EINVAL, "qh or kh is NULL");
      if (qk_type != ABSH_BF16 && qk_type != ABSH_F32) return fail(ABSH_EINVAL, "unknown dtype %d", (int)qk_type);
      if (!aligned16(qh) || !aligned16(kh)) return fail(ABSH_EINVAL, "qh and kh must be 16-byte aligned");
    }
    if (!(opts->p > 0.0 && opts->p <= 1.0)) return fail(ABSH_EINVAL, "p must lie in (0, 1] (got %g)", opts->p);
    if (opts->k_floor < 0) return fail(ABSH_EINVAL, "k_floor must be >= 0 (got %d)", opts->k_floor);
  }
  if (!(opts->slack_frac >= 0.0 && opts->slack_frac < 1.0))
    return fail(ABSH_EINVAL, "slack_frac must lie in [0, 1) (got %g)", opts->slack_frac);
  if (opts->order_depth < 0 || opts->order_depth > 64)
    return fail(ABSH_EINVAL, "order_depth must lie in [0, 64] (got %d)", opts->order_depth);
  if (opts->schedule < ABSH_SCHED_ORDER || opts->schedule > ABSH_SCHED_RANKS)
    return fail(ABSH_EINVAL, "unknown schedule %d", opts->schedule);
  const bool ranks = opts->schedule == ABSH_SCHED_RANKS;
  if (ranks) {
    if (opts->rank_policy < -1 || opts->rank_policy > 3)
      return fail(ABSH_EINVAL, "rank_policy must lie in -1 .. 3 (got %d)", opts->rank_policy);
    if (opts->strict_ranks != 0 && opts->strict_ranks != 1)
      return fail(ABSH_EINVAL, "strict_ranks must be 0 or 1 (got %d)", opts->strict_ranks);
    if (!(opts->k1 > 0.0 && opts->k1 <= opts->k2))
      return fail(ABSH_EINVAL, "need 0 < k1 <= k2 (got %g, %g)", opts->k1, opts->k2);
    if (!(opts->n1 >= 0.0 && opts->n1 < 1.0) || !(opts->n2 >= 0.0))
      return fail(ABSH_EINVAL, "need 0 <= n1 < 1 and n2 >= 0 (got %g, %g)", opts->n1, opts->n2);
    if (!out->head_order || !out->rank_info)
      return fail(ABSH_EINVAL, "head_order and rank_info must be non-NULL for ABSH_SCHED_RANKS");
    if ((int64_t)B * H > 1024)
      return fail(ABSH_EUNSUPPORTED, "ABSH_SCHED_RANKS takes at most 1024 heads (B*H = %lld)", (long long)B * H);
    if ((double)B * H * c->nb * c->nb >= 2147483648.0)
      return fail(ABSH_EUNSUPPORTED, "ABSH_SCHED_RANKS needs B*H*nb*nb < 2^31 (rank loads squared in int64)");
  }
  if (!out->counts || !out->kv_idx || !out->work || !out->L || !out->queue || !out->sched)
    return fail(ABSH_EINVAL, "counts, kv_idx, work, L, queue and sched must be non-NULL");
  if (opts->order_depth > 0 && !out->order) return fail(ABSH_EINVAL, "order is NULL but order_depth > 0");
  const int members = absh::unit_members(c, opts->schedule);
  if (members > 1 && (!out->unit_list || !out->unit_cnt))
    return fail(ABSH_EINVAL, "unit_list and unit_cnt must be non-NULL for this schedule");
  if (opts->schedule == ABSH_SCHED_LPT && members > 1 && !out->unit_queue)
    return fail(ABSH_EINVAL, "unit_queue must be non-NULL for ABSH_SCHED_LPT with blocks of 64 or 128");
  if (c->nb > kMaxNb) return fail(ABSH_EUNSUPPORTED, "nb = %d above the router's %d", c->nb, kMaxNb);
  const WsLayout w = ws_layout(c, B, H, d, scores);
  if (!ws) return fail(ABSH_EWORKSPACE, "workspace is NULL (%zu bytes needed)", w.total);
  if (ws_bytes < w.total) return fail(ABSH_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, w.total);
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(ABSH_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  if (check_only) return ABSH_OK;
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  float* qbar = given ? const_cast<float*>(means_q) : reinterpret_cast<float*>(base + w.qbar);
  float* kbar = given ? const_cast<float*>(means_k) : reinterpret_cast<float*>(base + w.kbar);
  absh::RouteBuffers rb;
  rb.S = scores ? reinterpret_cast<float*>(base + w.S) : nullptr;
  rb.qbar = qbar;
  rb.kbar = kbar;
  rb.d = d;
  rb.counts = out->counts;
  rb.kv_idx = out->kv_idx;
  rb.order = out->order;
  rb.work = out->work;
  rb.L = out->L;
  rb.queue = out->queue;
  rb.target = reinterpret_cast<int32_t*>(base + w.target);
  rb.slack_info = reinterpret_cast<int64_t*>(base + w.info);
  rb.chunk_hist = reinterpret_cast<int32_t*>(base + w.chunk_hist);
  rb.scan_sums = reinterpret_cast<int32_t*>(base + w.scan_sums);
  rb.slack_aux = reinterpret_cast<int32_t*>(base + w.slack_aux);
  rb.rank = reinterpret_cast<int32_t*>(base + w.rank);
  rb.sched = out->sched;
  rb.unit_list = out->unit_list;
  rb.unit_cnt = out->unit_cnt;
  rb.unit_queue = out->unit_queue;
  rb.owner = reinterpret_cast<int32_t*>(base + w.owner);
  rb.budget = reinterpret_cast<int64_t*>(base + w.budget);
  rb.head_order = ranks ? out->head_order : nullptr;
  rb.rank_info = ranks ? out->rank_info : nullptr;
  const int tiles = B * H * c->nb;
  bool units_in_select = false;

  if (structured) {
    const int offset = opts->anchor_stride > 0
                           ? (int)(((int64_t)opts->step * opts->anchor_shift) % opts->anchor_stride)
                           : 0;
    // a window of nb - 1 already reaches every block: larger ones are the same pattern
    const int window = std::min(opts->window, c->nb - 1);
    ABSH_HIP(absh::launch_window_anchor(c, rb, tiles, window, opts->anchor_stride, offset, s),
             "absh_route: window/anchor lists");
  } else {
    if (!given) {
      ABSH_HIP(absh::launch_pool(c, qh, qk_type == ABSH_F32, qbar, B, H, d, s), "absh_route: pool q");
      ABSH_HIP(absh::launch_pool(c, kh, qk_type == ABSH_F32, kbar, B, H, d, s), "absh_route: pool k");
    }
    if (rb.S) ABSH_HIP(absh::launch_scores(c, qbar, kbar, const_cast<float*>(rb.S), B * H, d, s), "absh_route: scores");
    // when no later stage changes the counts, the selection also writes the units' union lists
    units_in_select = rb.S && members > 1 && opts->slack_frac <= 0.0 && !ranks;
    ABSH_HIP(absh::launch_select(c, rb, tiles, opts->p, opts->k_floor, opts->order_depth, 0, s,
                                 units_in_select ? members : 0),
             "absh_route: select");
  }
  if (opts->slack_frac > 0.0) {
    ABSH_HIP(absh::launch_slack_plan(c, rb, tiles, opts->slack_frac, s), "absh_route: slack plan");
    ABSH_HIP(absh::launch_select(c, rb, tiles, opts->p, opts->k_floor, 0, 1, s), "absh_route: slack fill");
  }
  ABSH_HIP(absh::launch_workload(c, rb, B * H, s), "absh_route: workload");
  if (ranks) {
    // rank loads, policy, RLB plan, SASA budgets and the rank segments; then each
    // rank's tiles are extended along their importance order, and loads redone
    const absh::RankOpts ro{opts->rank_policy, opts->k1, opts->k2, opts->n1, opts->n2};
    ABSH_HIP(absh::launch_rank_stage(c, rb, B * H, ro, s), "absh_route: rank plan");
    ABSH_HIP(absh::launch_rank_fill(c, rb, s), "absh_route: rank fill");
    ABSH_HIP(absh::launch_select(c, rb, tiles, opts->p, opts->k_floor, 0, 1, s), "absh_route: rank fill select");
    ABSH_HIP(absh::launch_workload(c, rb, B * H, s), "absh_route: workload after fill");
    ABSH_HIP(absh::launch_rank_final(rb, B * H, s), "absh_route: rank report");
  }
  ABSH_HIP(absh::launch_queue(c, rb, tiles, opts->schedule == ABSH_SCHED_LPT, s), "absh_route: queue");
  if (members > 1 && !units_in_select) ABSH_HIP(absh::launch_groups(c, rb, B * H, members, s), "absh_route: groups");
  if (!ranks) ABSH_HIP(absh::launch_segments(c, rb, B * H, opts->schedule, s), "absh_route: segments");
  if (opts->schedule == ABSH_SCHED_LPT && members > 1)
    ABSH_HIP(absh::launch_unit_lpt(c, rb, B * H, s), "absh_route: unit queue");
  if (out->pull) ABSH_HIP(absh::launch_zero_i32(out->pull, ABSH_PULL_WORDS, s), "absh_route: pull counters");
  out->schedule = opts->schedule;
  out->strict_ranks = ranks ? opts->strict_ranks : 0;
  return ABSH_OK;
}

}  // namespace

extern "C" {

absh_status absh_route(absh_ctx* c, const void* qh, const void* kh, absh_dtype qk_type, int B, int H, int d,
                       const absh_route_opts* opts, absh_lists* out, void* ws, size_t ws_bytes, void* stream) {
  return route_impl(c, qh, kh, qk_type, B, H, d, opts, out, ws, ws_bytes, stream, true);
}

absh_status absh_route_means(absh_ctx* c, const float* qbar, const float* kbar, int B, int H, int d,
                             const absh_route_opts* opts, absh_lists* out, void* ws, size_t ws_bytes, void* stream) {
  if (!qbar) {
    g_last_error.clear();
    return fail(ABSH_EINVAL, "qbar is NULL");
  }
  return route_impl(c, nullptr, nullptr, ABSH_F32, B, H, d, opts, out, ws, ws_bytes, stream, true, qbar, kbar);
}

absh_status absh_route_static(absh_ctx* c, const void* qh, const void* kh, absh_dtype qk_type, int B, int H, int d,
                              const absh_route_opts* opts, absh_lists* out, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  const size_t need = ws_layout(c, B, H, d, false).total;
  if (need > kStaticScratchBytes)
    return fail(ABSH_EWORKSPACE, "absh_route_static: this shape needs %zu bytes of scratch, above its %zu-byte maximum",
                need, kStaticScratchBytes);
  void* ptr = scratch_ptr(c->device);
  if (!ptr) return fail(ABSH_EINVAL, "absh_route_static: no static scratch on device %d", c->device);
  return route_impl(c, qh, kh, qk_type, B, H, d, opts, out, ptr, kStaticScratchBytes, stream, false);
}

}  // extern "C"

namespace {

// Validation and kernel view of the lists of absh_sparse_attn / _v8.
absh_status attn_lists(const absh_ctx* c, const absh_lists* lists, absh::AttnLists* L) {
  *L = absh::AttnLists{};
  if (!lists) return ABSH_OK;
  if (!lists->counts || !lists->kv_idx || !lists->queue || !lists->sched)
    return fail(ABSH_EINVAL, "lists needs counts, kv_idx, queue and sched");
  if (lists->schedule < ABSH_SCHED_ORDER || lists->schedule > ABSH_SCHED_RANKS)
    return fail(ABSH_EINVAL, "lists->schedule %d is not a schedule (was absh_route run?)", lists->schedule);
  if (lists->schedule == ABSH_SCHED_RANKS && !lists->head_order)
    return fail(ABSH_EINVAL, "lists needs head_order for ABSH_SCHED_RANKS");
  const int members = absh::unit_members(c, lists->schedule);
  if (members > 1 && (!lists->unit_list || !lists->unit_cnt))
    return fail(ABSH_EINVAL, "lists needs unit_list and unit_cnt for this schedule");
  if (lists->schedule == ABSH_SCHED_LPT && members > 1 && !lists->unit_queue)
    return fail(ABSH_EINVAL, "lists needs unit_queue for ABSH_SCHED_LPT");
  L->queue = lists->queue;
  L->counts = lists->counts;
  L->kv_idx = lists->kv_idx;
  L->unit_list = lists->unit_list;
  L->unit_cnt = lists->unit_cnt;
  L->sched = lists->sched;
  L->members = members;
  if (lists->schedule == ABSH_SCHED_LPT && members > 1) L->unit_queue = lists->unit_queue;
  L->counters = lists->pull;
  L->wg_busy = lists->wg_busy;
  if (lists->schedule == ABSH_SCHED_RANKS) {
    L->head_order = lists->head_order;
    L->strict = lists->strict_ranks ? 1 : 0;
  }
  return ABSH_OK;
}

}  // namespace

extern "C" {

absh_status absh_sparse_attn(absh_ctx* c, const void* qh, const void* kh, const void* vt, int B, int H, int d,
                             const absh_lists* lists, void* oh, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!qh || !kh || !vt || !oh) return fail(ABSH_EINVAL, "qh, kh, vt or oh is NULL");
  if (!aligned16(qh) || !aligned16(kh) || !aligned16(vt) || !aligned16(oh))
    return fail(ABSH_EINVAL, "qh, kh, vt and oh must be 16-byte aligned");
  absh::AttnLists L;
  if (absh_status st = attn_lists(c, lists, &L)) return st;
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_attention(c, qh, kh, vt, oh, B, H, d, lists ? &L : nullptr,
                                  reinterpret_cast<hipStream_t>(stream)),
           "absh_sparse_attn");
  return ABSH_OK;
}

absh_status absh_quantize_v(absh_ctx* c, const void* vh, int B, int H, int d, void* vt8, float* vscale,
                            void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (c->block != 64 && c->block != 128)
    return fail(ABSH_EUNSUPPORTED, "8-bit values need block 64 or 128 (context has %d)", c->block);
  if (!vh || !vt8 || !vscale) return fail(ABSH_EINVAL, "vh, vt8 or vscale is NULL");
  if (!aligned16(vh) || !aligned16(vt8) || !aligned16(vscale))
    return fail(ABSH_EINVAL, "vh, vt8 and vscale must be 16-byte aligned");
  if ((double)B * H * (c->n_pad / 64) >= 2147483647.0) return fail(ABSH_EINVAL, "B*H*n_pad/64 must fit in int32");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_quantize_v(c, vh, vt8, vscale, B * H, d, reinterpret_cast<hipStream_t>(stream)),
           "absh_quantize_v");
  return ABSH_OK;
}

absh_status absh_sparse_attn_v8(absh_ctx* c, const void* qh, const void* kh, const void* vt8, const float* vscale,
                                int B, int H, int d, const absh_lists* lists, void* oh, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!qh || !kh || !vt8 || !vscale || !oh) return fail(ABSH_EINVAL, "qh, kh, vt8, vscale or oh is NULL");
  if (!aligned16(qh) || !aligned16(kh) || !aligned16(vt8) || !aligned16(vscale) || !aligned16(oh))
    return fail(ABSH_EINVAL, "qh, kh, vt8, vscale and oh must be 16-byte aligned");
  absh::AttnLists L;
  if (absh_status st = attn_lists(c, lists, &L)) return st;
  const int members = lists ? L.members : (c->block >= 128 ? 2 : 4);
  if (!absh::union_attention_supported(d, c->block, members))
    return fail(ABSH_EUNSUPPORTED, "8-bit values need block 64 or 128");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  ABSH_HIP(absh::launch_union_attention(c, qh, kh, vt8, vscale, oh, B, H, d, lists ? &L : nullptr,
                                        reinterpret_cast<hipStream_t>(stream)),
           "absh_sparse_attn_v8");
  return ABSH_OK;
}

absh_status absh_sparse_attn_grid(absh_ctx* c, const void* qh, const void* kh, const void* vt, const float* vscale,
                                  int B, int H, int d, const absh_lists* lists, void* o, void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!qh || !kh || !vt || !o) return fail(ABSH_EINVAL, "qh, kh, vt or o is NULL");
  if (!aligned16(qh) || !aligned16(kh) || !aligned16(vt) || !aligned16(o) || (vscale && !aligned16(vscale)))
    return fail(ABSH_EINVAL, "qh, kh, vt, vscale and o must be 16-byte aligned");
  absh::AttnLists L;
  if (absh_status st = attn_lists(c, lists, &L)) return st;
  const int members = lists ? L.members : (c->block >= 128 ? 2 : 4);
  if (vscale && !absh::union_attention_supported(d, c->block, members))
    return fail(ABSH_EUNSUPPORTED, "8-bit values need block 64 or 128");
  DeviceScope dev;
  if (absh_status st = dev.enter(c->device)) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (vscale)
    ABSH_HIP(absh::launch_union_attention(c, qh, kh, vt, vscale, o, B, H, d, lists ? &L : nullptr, s, true),
             "absh_sparse_attn_grid");
  else
    ABSH_HIP(absh::launch_attention(c, qh, kh, vt, o, B, H, d, lists ? &L : nullptr, s, true),
             "absh_sparse_attn_grid");
  return ABSH_OK;
}

}  // extern "C"

namespace {

// absh_forward's workspace: the Hilbert-order rows of q and k, V^T, then
// absh_route's workspace (whose block-mean slots take the means of q and k). The
// attention writes o in grid order itself, so no Hilbert-order output is kept.
struct FwdLayout {
  size_t qh, kh, vt, route, total;
};

FwdLayout fwd_layout(const absh_ctx* c, int B, int H, int d) {
  FwdLayout f{};
  const size_t rows = (size_t)B * H * c->n_pad * d * 2;
  const size_t vt = (size_t)B * H * c->nb * d * absh::vt_keys(c->block) * 2;
  size_t off = 0;
  f.qh = off; off = align_up(off + rows);
  f.kh = off; off = align_up(off + rows);
  f.vt = off; off = align_up(off + vt);
  f.route = off; off = align_up(off + ws_layout(c, B, H, d).total);
  f.total = off;
  return f;
}

}  // namespace

extern "C" {

size_t absh_forward_workspace_bytes(const absh_ctx* c, int B, int H, int d) {
  if (!c || B < 1 || H < 1 || d < 1) return 0;
  return fwd_layout(c, B, H, d).total;
}

absh_status absh_forward(absh_ctx* c, const void* q, const void* k, const void* v, absh_dtype xt, void* o, int B,
                         int H, int d, const absh_route_opts* opts, absh_lists* lists, void* ws, size_t ws_bytes,
                         void* stream) {
  g_last_error.clear();
  if (absh_status st = check_ctx(c)) return st;
  if (absh_status st = check_shape(c, B, H, d)) return st;
  if (!q || !k || !v || !o) return fail(ABSH_EINVAL, "q, k, v or o is NULL");
  if (!opts || !lists) return fail(ABSH_EINVAL, "opts or lists is NULL");
  if (opts->router != ABSH_ROUTER_TOPP) return fail(ABSH_EINVAL, "absh_forward takes the Top-p router");
  const FwdLayout f = fwd_layout(c, B, H, d);
  if (!ws) return fail(ABSH_EWORKSPACE, "workspace is NULL (%zu bytes needed)", f.total);
  if (ws_bytes < f.total) return fail(ABSH_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, f.total);
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return fail(ABSH_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  char* base = reinterpret_cast<char*>(ws);
  void* qh = base + f.qh;
  void* kh = base + f.kh;
  void* vt = base + f.vt;
  char* rws = base + f.route;
  const WsLayout w = ws_layout(c, B, H, d);
  float* qbar = reinterpret_cast<float*>(rws + w.qbar);
  float* kbar = reinterpret_cast<float*>(rws + w.kbar);
  // every argument is checked before the first launch
  if (xt != ABSH_BF16 && xt != ABSH_F32) return fail(ABSH_EINVAL, "unknown dtype %d", (int)xt);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ABSH_EINVAL, "q, k, v and o must be 16-byte aligned");
  if (absh_status st = route_impl(c, nullptr, nullptr, ABSH_BF16, B, H, d, opts, lists, rws, ws_bytes - f.route,
                                  stream, true, qbar, kbar, true))
    return st;  // (the lists' buffers the attention reads are the ones the routing checks)
  if (absh_status st = absh_permute_pool(c, q, xt, qh, qbar, B, H, d, ABSH_ROWS, stream)) return st;
  if (absh_status st = absh_permute_pool(c, k, xt, kh, kbar, B, H, d, ABSH_ROWS, stream)) return st;
  if (absh_status st = absh_permute(c, v, xt, vt, B, H, d, ABSH_VT, stream)) return st;
  if (absh_status st = route_impl(c, nullptr, nullptr, ABSH_BF16, B, H, d, opts, lists, rws, ws_bytes - f.route,
                                  stream, true, qbar, kbar))
    return st;
  return absh_sparse_attn_grid(c, qh, kh, vt, nullptr, B, H, d, lists, o, stream);
}

}  // extern "C"
