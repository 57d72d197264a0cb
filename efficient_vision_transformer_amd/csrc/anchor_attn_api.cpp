// anchor_attn_api.cpp -- the C ABI declared in include/anchor_attn.h.
//
// Validation, plan selection, the grow-only workspace and kernel launches.  Nothing here
// computes any part of the method on the host: every step runs in the HIP kernels.
#include "anchor_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"
#include "split_plan.h"

struct anchor_attn_ctx {
  int device = 0;
  int num_cus = 256;
  void* workspace = nullptr;        // split plan and backward partials
  size_t workspace_bytes = 0;
  anchor_attn_plan_t plan = ANCHOR_ATTN_PLAN_AUTO;
  aa::GemmCache* gemm = nullptr;    // block projections (created on first use)
  void* block_ws = nullptr;         // block: projected Q|V, H and the GEMM workspace
  size_t block_ws_bytes = 0;
  // Workspaces replaced by larger ones.  They stay allocated until anchor_attn_destroy:
  // a HIP graph captured before the growth still holds their addresses.
  std::vector<void*> retired;
  // Test hook (environment variable ANCHOR_ATTN_FAIL_ALLOC_ABOVE, read at create): device
  // allocations of more than this many bytes fail as if the device were out of memory.
  size_t fail_alloc_above = SIZE_MAX;
};

namespace {

using aa::FusedPlan;
using aa::Geometry;
using aa::SplitPlan;

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Element strides (batch, head, token) from the caller: null keeps *w (the contiguous
// layout); otherwise each stride must be non-negative and a multiple of 16 bytes.
bool take_view(const long long* s3, size_t es, aa::View* w) {
  if (!s3) return true;
  for (int i = 0; i < 3; ++i)
    if (s3[i] < 0 || ((unsigned long long)s3[i] * es) % 16 != 0) return false;
  *w = aa::View{s3[0], s3[1], s3[2]};
  return true;
}

// Bytes from a view's first element to one past its last (B, h, n >= 1).
size_t view_extent(const aa::View& w, int B, int h, int n, int d, size_t es) {
  const long long last = (long long)(B - 1) * w.sb + (long long)(h - 1) * w.sh +
                         (long long)(n - 1) * w.st;
  return ((size_t)last + (size_t)d) * es;
}

// True when distinct (batch, head, token) rows of a view never share an element: taken
// in increasing stride, every stride of a dimension with more than one index is at least
// the span of the rows below it.
bool view_injective(const aa::View& w, int B, int h, int n, int d) {
  struct Dim {
    long long stride, count;
  } dims[3] = {{w.sb, B}, {w.sh, h}, {w.st, n}};
  std::sort(dims, dims + 3, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
  long long span = d;
  for (const Dim& dm : dims) {
    if (dm.count <= 1) continue;
    if (dm.stride < span) return false;
    span += dm.stride * (dm.count - 1);
  }
  return true;
}

// The int a caller passed for an enum parameter, read without loading it as the enum type
// (a C caller may pass any int; in C++ a value outside the enumerators' range must not be
// loaded as the enum).
template <typename E>
int raw(const E* p) {
  static_assert(sizeof(E) == sizeof(int), "int-sized enum");
  int v;
  std::memcpy(&v, p, sizeof v);
  return v;
}

// Argument checks shared by forward and describe.  Returns SUCCESS and fills *g, or the
// error.  *empty is set when there is no work (B*h*n == 0).
anchor_attn_status_t check_shape(int B, int h, int n, int m, int d, int dtype_raw,
                                 Geometry* g, bool* empty) {
  if (B < 0 || h < 0 || n < 0 || m < 0 || d < 0) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  if (m == 0 || d == 0) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  if (dtype_raw != ANCHOR_ATTN_FP32 && dtype_raw != ANCHOR_ATTN_BF16) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  const anchor_attn_dtype_t dtype = (anchor_attn_dtype_t)dtype_raw;
  if (d != 32 && d != 64 && d != 128) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  // d = 128 in fp32: the split plan's forward up to 128 anchors
  if (d == 128 && dtype != ANCHOR_ATTN_BF16 && m > 128) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  if (m > 512) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  // more than 256 anchors: the bf16 split plan at d <= 64 only
  if (m > 256 && (dtype != ANCHOR_ATTN_BF16 || d > 64)) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  const long long slices = (long long)B * (long long)h;
  *empty = (slices == 0 || n == 0);
  // Index limits: per-slice offsets are 64-bit, but grids and token indices are 32-bit.
  if (slices > (1LL << 24) || (long long)n > (1LL << 28)) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  g->B = B; g->h = h; g->n = n; g->m = m; g->d = d;
  // anchors padded to a multiple of 32, of 64 above 128 anchors and of 128 above 256 (the
  // split plan's anchor-split pass 1 divides the tiles among four or eight waves)
  g->m_pad = (m <= 128) ? (m + 31) / 32 * 32 : (m <= 256) ? (m + 63) / 64 * 64 : (m + 127) / 128 * 128;
  g->at = g->m_pad / 16;
  g->slices = slices;
  g->c2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  const aa::View contiguous{(long long)h * n * d, (long long)n * d, (long long)d};
  g->vw = aa::Views{contiguous, contiguous, contiguous};
  return ANCHOR_ATTN_SUCCESS;
}

SplitPlan make_split_plan(const Geometry& g, anchor_attn_dtype_t dtype, int num_cus) {
  return aa::split_plan(g, dtype == ANCHOR_ATTN_BF16, num_cus);
}

enum class Chosen { Fused, Split, Unsupported };

// Linear attention split plan: chunks of whole 128-token blocks (four waves x one
// 32-token pair), about one pass-1 workgroup per CU (half the partials of two: dense
// 41.7 -> 39.5 us, long 71.9 -> 69.0 us) and sixteen pass-2 workgroups per CU (against
// four: dense 39.4 -> 36.9 us, long 69.4 -> 63.8 us; eight gave 37.0 and 68.1).
aa::LinearSplitPlan make_linear_plan(const Geometry& g, int num_cus) {
  aa::LinearSplitPlan p{};
  const int n = g.n, blk = 128;
  auto chunking = [&](long long want, int* chunks, int* len) {
    const int maxc = (n + blk - 1) / blk;
    const int c = (int)std::min<long long>(maxc, std::max<long long>(1, (want + g.slices - 1) / g.slices));
    int l = (n + c - 1) / c;
    l = (l + blk - 1) / blk * blk;
    *len = l;
    *chunks = (n + l - 1) / l;
  };
  chunking(1LL * num_cus, &p.chunks1, &p.chunk_len1);
  chunking(16LL * num_cus, &p.chunks2, &p.chunk_len2);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  p.part_bytes = al((size_t)g.slices * p.chunks1 * g.d * g.d * sizeof(float));
  p.zpart_bytes = al((size_t)g.slices * p.chunks1 * g.d * sizeof(float));
  p.sop_bytes = al((size_t)g.slices * g.d * g.d * 2);
  p.z_bytes = al((size_t)g.slices * g.d * sizeof(float));
  return p;
}

Chosen choose(const anchor_attn_ctx* ctx, const Geometry& g, anchor_attn_dtype_t dtype,
              FusedPlan* fp) {
  const bool fused_ok = (dtype == ANCHOR_ATTN_BF16) && aa::fused_supported(g, ctx->num_cus, fp);
  switch (ctx->plan) {
    case ANCHOR_ATTN_PLAN_FUSED: return fused_ok ? Chosen::Fused : Chosen::Unsupported;
    case ANCHOR_ATTN_PLAN_SPLIT: return Chosen::Split;
    default:
      // one workgroup per slice pays off once the slices alone fill half of the CUs
      return (fused_ok && g.slices * 2 >= ctx->num_cus) ? Chosen::Fused : Chosen::Split;
  }
}

// The backward (bf16; m <= 256 at d <= 64, m <= 128 at d = 128): one workgroup per slice
// when that plan applies, else the split passes; the context's plan setting is honoured as
// for the forward.
Chosen choose_backward(const anchor_attn_ctx* ctx, const Geometry& g, anchor_attn_dtype_t dtype) {
  if (dtype == ANCHOR_ATTN_FP32) {
    // fp32: the split passes only (m <= 256, d = 32 or 64)
    if (!aa::bwd_fp32_supported(g) || ctx->plan == ANCHOR_ATTN_PLAN_FUSED) return Chosen::Unsupported;
    return Chosen::Split;
  }
  if (dtype != ANCHOR_ATTN_BF16 || !aa::bwd_split_supported(g)) return Chosen::Unsupported;
  const bool fused_ok = aa::bwd_fused_supported(g);
  switch (ctx->plan) {
    case ANCHOR_ATTN_PLAN_FUSED: return fused_ok ? Chosen::Fused : Chosen::Unsupported;
    case ANCHOR_ATTN_PLAN_SPLIT: return Chosen::Split;
    default: return (fused_ok && g.slices * 2 >= ctx->num_cus) ? Chosen::Fused : Chosen::Split;
  }
}

const char* chosen_name(Chosen c) {
  return c == Chosen::Fused ? "fused" : (c == Chosen::Split ? "split" : "unsupported");
}

// Allocates `bytes` of device memory for the context (honouring the test hook).
anchor_attn_status_t device_alloc(anchor_attn_ctx* ctx, size_t bytes, void** out) {
  *out = nullptr;
  if (bytes > ctx->fail_alloc_above) return ANCHOR_ATTN_ERROR_OUT_OF_MEMORY;
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();  // clear this thread's error state
    return ANCHOR_ATTN_ERROR_OUT_OF_MEMORY;
  }
  *out = p;
  return ANCHOR_ATTN_SUCCESS;
}

// Grows a grow-only buffer to at least `bytes`.  The old buffer is retired, not freed (a
// captured graph may still use it); on failure the buffer is left as it was.
anchor_attn_status_t grow(anchor_attn_ctx* ctx, void** buf, size_t* have, size_t bytes) {
  if (bytes <= *have) return ANCHOR_ATTN_SUCCESS;
  try {
    ctx->retired.reserve(ctx->retired.size() + 1);
  } catch (...) {
    return ANCHOR_ATTN_ERROR_OUT_OF_MEMORY;
  }
  void* p = nullptr;
  const anchor_attn_status_t st = device_alloc(ctx, bytes, &p);
  if (st != ANCHOR_ATTN_SUCCESS) return st;
  if (*buf) ctx->retired.push_back(*buf);
  *buf = p;
  *have = bytes;
  return ANCHOR_ATTN_SUCCESS;
}

anchor_attn_status_t ensure_workspace(anchor_attn_ctx* ctx, size_t bytes) {
  return grow(ctx, &ctx->workspace, &ctx->workspace_bytes, bytes);
}

// Everything a forward of geometry g needs before it can be enqueued without failing: a
// plan, and the split plan's workspace.  Call with the device current.
anchor_attn_status_t prepare_forward(anchor_attn_ctx* ctx, const Geometry& g,
                                     anchor_attn_dtype_t dtype) {
  FusedPlan fp{};
  const Chosen c = choose(ctx, g, dtype, &fp);
  if (c == Chosen::Unsupported) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  if (c == Chosen::Split) return ensure_workspace(ctx, make_split_plan(g, dtype, ctx->num_cus).workspace_bytes());
  return ANCHOR_ATTN_SUCCESS;
}

// Enqueues the forward with the split plan's partials in `ws` (at least `ws_bytes`; unused
// by the fused plan).
anchor_attn_status_t run_forward_ws(anchor_attn_ctx* ctx, const Geometry& g,
                                    anchor_attn_dtype_t dtype, const void* Q, const void* U,
                                    const void* V, void* H, void* ws, size_t ws_bytes,
                                    hipStream_t s) {
  FusedPlan fp{};
  const Chosen c = choose(ctx, g, dtype, &fp);
  hipError_t e;
  if (c == Chosen::Fused) {
    e = aa::launch_fused_bf16(g, fp, Q, U, V, H, s);
  } else if (c == Chosen::Split) {
    const SplitPlan p = make_split_plan(g, dtype, ctx->num_cus);
    if (ws_bytes < p.workspace_bytes()) return ANCHOR_ATTN_ERROR_OUT_OF_MEMORY;
    e = (dtype == ANCHOR_ATTN_BF16) ? aa::launch_split_bf16(g, p, Q, U, V, H, ws, s)
                                    : aa::launch_split_fp32(g, p, Q, U, V, H, ws, s);
  } else {
    return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return ANCHOR_ATTN_ERROR_HIP;
  }
  return ANCHOR_ATTN_SUCCESS;
}

// Enqueues the forward (after prepare_forward succeeded for g).
anchor_attn_status_t run_forward(anchor_attn_ctx* ctx, const Geometry& g, anchor_attn_dtype_t dtype,
                                 const void* Q, const void* U, const void* V, void* H,
                                 hipStream_t s) {
  return run_forward_ws(ctx, g, dtype, Q, U, V, H, ctx->workspace, ctx->workspace_bytes, s);
}

// ---- scratch of anchor_attn_forward_noalloc --------------------------------------------
// The split plan's partials for callers that cannot allocate: a fixed array in device
// memory, one copy per GPU the library runs on (held until the process ends).  In host
// code `scratch` is only a handle for hipGetSymbolAddress; kernels receive the device
// address that call returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, looked up once per device with that
// device current.
anchor_attn_status_t scratch_on_device(int dev, void** out) {
  *out = nullptr;
  if (dev < 0 || dev >= kMaxDevices) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return ANCHOR_ATTN_ERROR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ANCHOR_ATTN_SUCCESS;
}

}  // namespace

extern "C" {

const char* anchor_attn_status_string(anchor_attn_status_t s) {
  switch (raw(&s)) {
    case ANCHOR_ATTN_SUCCESS: return "ANCHOR_ATTN_SUCCESS";
    case ANCHOR_ATTN_ERROR_INVALID_VALUE: return "ANCHOR_ATTN_ERROR_INVALID_VALUE";
    case ANCHOR_ATTN_ERROR_NOT_SUPPORTED: return "ANCHOR_ATTN_ERROR_NOT_SUPPORTED";
    case ANCHOR_ATTN_ERROR_OUT_OF_MEMORY: return "ANCHOR_ATTN_ERROR_OUT_OF_MEMORY";
    case ANCHOR_ATTN_ERROR_HIP: return "ANCHOR_ATTN_ERROR_HIP";
  }
  return "ANCHOR_ATTN_ERROR_UNKNOWN_STATUS";
}

anchor_attn_status_t anchor_attn_create(anchor_attn_ctx** out) {
  if (!out) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  *out = nullptr;
  try {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
      (void)hipGetLastError();
      return ANCHOR_ATTN_ERROR_HIP;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ANCHOR_ATTN_ERROR_HIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return ANCHOR_ATTN_ERROR_HIP;
    anchor_attn_ctx* ctx = new (std::nothrow) anchor_attn_ctx;
    if (!ctx) return ANCHOR_ATTN_ERROR_OUT_OF_MEMORY;
    ctx->device = dev;
    ctx->num_cus = cus > 0 ? cus : 256;
    if (const char* lim = std::getenv("ANCHOR_ATTN_FAIL_ALLOC_ABOVE")) {
      char* end = nullptr;
      const unsigned long long v = std::strtoull(lim, &end, 10);
      if (end && end != lim && *end == '\0') ctx->fail_alloc_above = (size_t)v;
    }
    *out = ctx;
    return ANCHOR_ATTN_SUCCESS;
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

anchor_attn_status_t anchor_attn_destroy(anchor_attn_ctx* ctx) {
  if (!ctx) return ANCHOR_ATTN_SUCCESS;
  anchor_attn_status_t st = ANCHOR_ATTN_SUCCESS;
  if (ctx->workspace || ctx->block_ws || ctx->gemm || !ctx->retired.empty()) {
    DeviceGuard guard(ctx->device);
    if (ctx->workspace && hipFree(ctx->workspace) != hipSuccess) st = ANCHOR_ATTN_ERROR_HIP;
    if (ctx->block_ws && hipFree(ctx->block_ws) != hipSuccess) st = ANCHOR_ATTN_ERROR_HIP;
    for (void* p : ctx->retired)
      if (hipFree(p) != hipSuccess) st = ANCHOR_ATTN_ERROR_HIP;
    aa::gemm_cache_destroy(ctx->gemm);
  }
  delete ctx;
  return st;
}

anchor_attn_status_t anchor_attn_set_plan(anchor_attn_ctx* ctx, anchor_attn_plan_t plan) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  const int pr = raw(&plan);
  if (pr != ANCHOR_ATTN_PLAN_AUTO && pr != ANCHOR_ATTN_PLAN_FUSED && pr != ANCHOR_ATTN_PLAN_SPLIT)
    return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  ctx->plan = plan;
  return ANCHOR_ATTN_SUCCESS;
}

anchor_attn_status_t anchor_attn_describe_plan(anchor_attn_ctx* ctx, int B, int h, int n, int m,
                                               int d, anchor_attn_dtype_t dtype, char* buf,
                                               int len) {
  if (!ctx || !buf || len <= 0) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, m, d, raw(&dtype), &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    if (empty) {
      std::snprintf(buf, (size_t)len, "empty: no work");
      return ANCHOR_ATTN_SUCCESS;
    }
    FusedPlan fp{};
    const Chosen c = choose(ctx, g, dtype, &fp);
    if (c == Chosen::Unsupported) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    if (c == Chosen::Fused) {
      std::snprintf(buf, (size_t)len,
                    "fused: grid=%lld (%lld whole slices + %lld shared by two) wg=%d waves "
                    "pairs_per_wave=%d %s m_pad=%d workspace=0; backward: %s",
                    (long long)(g.slices + fp.shared), (long long)(g.slices - fp.shared),
                    (long long)fp.shared, fp.waves, fp.pairs_per_wave,
                    fp.keep_a ? "A kept" : "A recomputed", g.m_pad,
                    chosen_name(choose_backward(ctx, g, dtype)));
    } else {
      const SplitPlan p = make_split_plan(g, dtype, ctx->num_cus);
      std::snprintf(buf, (size_t)len,
                    "split: pass1 grid=%lld chunk=%d x%d | finalize grid=%lld | pass2 grid=%lld "
                    "chunk=%d x%d | m_pad=%d workspace=%zu; backward: %s",
                    (long long)(g.slices * p.chunks1), p.chunk_len1, p.chunks1,
                    (long long)(g.slices * g.at), (long long)(g.slices * p.chunks2), p.chunk_len2,
                    p.chunks2, g.m_pad, p.workspace_bytes(),
                    chosen_name(choose_backward(ctx, g, dtype)));
    }
    return ANCHOR_ATTN_SUCCESS;
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

static anchor_attn_status_t forward_strided_impl(anchor_attn_ctx* ctx, const void* Q,
                                                 const long long* q_strides, const void* U,
                                                 const void* V, const long long* v_strides,
                                                 void* H, const long long* h_strides, int B,
                                                 int h, int n, int m, int d,
                                                 int dtype_raw, void* stream) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, m, d, dtype_raw, &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    const anchor_attn_dtype_t dtype = (anchor_attn_dtype_t)dtype_raw;
    const size_t es = (dtype == ANCHOR_ATTN_BF16) ? 2 : 4;
    if (!take_view(q_strides, es, &g.vw.q) || !take_view(v_strides, es, &g.vw.v) ||
        !take_view(h_strides, es, &g.vw.o))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (empty) return ANCHOR_ATTN_SUCCESS;
    if (!Q || !U || !V || !H) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const uintptr_t mis = ((uintptr_t)Q | (uintptr_t)U | (uintptr_t)V | (uintptr_t)H) & 15u;
    if (mis) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (!view_injective(g.vw.o, B, h, n, d)) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const size_t qx = view_extent(g.vw.q, B, h, n, d, es), vx = view_extent(g.vw.v, B, h, n, d, es);
    const size_t hx = view_extent(g.vw.o, B, h, n, d, es);
    const size_t ub = (size_t)h * (size_t)m * (size_t)d * es;
    if (overlaps(H, hx, Q, qx) || overlaps(H, hx, V, vx) || overlaps(H, hx, U, ub))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;

    DeviceGuard guard(ctx->device);
    if (!guard.ok) return ANCHOR_ATTN_ERROR_HIP;
    st = prepare_forward(ctx, g, dtype);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    return run_forward(ctx, g, dtype, Q, U, V, H, (hipStream_t)stream);
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

anchor_attn_status_t anchor_attn_forward_strided(anchor_attn_ctx* ctx, const void* Q,
                                                 const long long* q_strides, const void* U,
                                                 const void* V, const long long* v_strides,
                                                 void* H, const long long* h_strides, int B,
                                                 int h, int n, int m, int d,
                                                 anchor_attn_dtype_t dtype, void* stream) {
  return forward_strided_impl(ctx, Q, q_strides, U, V, v_strides, H, h_strides, B, h, n, m, d,
                              raw(&dtype), stream);
}

anchor_attn_status_t anchor_attn_forward_noalloc(anchor_attn_ctx* ctx, const void* Q,
                                                 const void* U, const void* V, void* H, int B,
                                                 int h, int n, int m, int d,
                                                 anchor_attn_dtype_t dtype, void* stream) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, m, d, raw(&dtype), &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    if (empty) return ANCHOR_ATTN_SUCCESS;
    if (!Q || !U || !V || !H) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (((uintptr_t)Q | (uintptr_t)U | (uintptr_t)V | (uintptr_t)H) & 15u)
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const size_t es = (dtype == ANCHOR_ATTN_BF16) ? 2 : 4;
    const size_t tb = (size_t)B * h * n * d * es, ub = (size_t)h * (size_t)m * (size_t)d * es;
    if (overlaps(H, tb, Q, tb) || overlaps(H, tb, V, tb) || overlaps(H, tb, U, ub))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    FusedPlan fp{};
    const Chosen c = choose(ctx, g, dtype, &fp);
    if (c == Chosen::Unsupported) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    // the split plan's partials must fit the fixed scratch
    if (c == Chosen::Split && make_split_plan(g, dtype, ctx->num_cus).workspace_bytes() > kScratchBytes)
      return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    DeviceGuard guard(ctx->device);
    if (!guard.ok) return ANCHOR_ATTN_ERROR_HIP;
    void* ws = nullptr;
    if (c == Chosen::Split) {
      st = scratch_on_device(ctx->device, &ws);
      if (st != ANCHOR_ATTN_SUCCESS) return st;
    }
    return run_forward_ws(ctx, g, dtype, Q, U, V, H, ws, ws ? kScratchBytes : 0,
                          (hipStream_t)stream);
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

anchor_attn_status_t anchor_attn_forward(anchor_attn_ctx* ctx, const void* Q, const void* U,
                                         const void* V, void* H, int B, int h, int n, int m,
                                         int d, anchor_attn_dtype_t dtype, void* stream) {
  return forward_strided_impl(ctx, Q, nullptr, U, V, nullptr, H, nullptr, B, h, n, m, d,
                              raw(&dtype), stream);
}

anchor_attn_status_t anchor_attn_block_forward(anchor_attn_ctx* ctx, const void* X, const void* Wqv,
                                               const void* bqv, const void* U, const void* Wo,
                                               const void* bo, void* Y, int B, int n, int h,
                                               int m, int d, anchor_attn_dtype_t dtype,
                                               void* stream) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, m, d, raw(&dtype), &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    if (dtype != ANCHOR_ATTN_BF16) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    const long long C = (long long)h * d, T = (long long)B * n;
    if (2 * C > (1LL << 30) || T > (1LL << 31)) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    if (empty) return ANCHOR_ATTN_SUCCESS;   // no tokens, or C = 0: Y is empty
    if (!X || !Wqv || !U || !Wo || !Y) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const uintptr_t mis = ((uintptr_t)X | (uintptr_t)Wqv | (uintptr_t)bqv | (uintptr_t)U |
                           (uintptr_t)Wo | (uintptr_t)bo | (uintptr_t)Y) & 15u;
    if (mis) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const size_t es = 2;
    const size_t yb = (size_t)T * C * es;
    const void* ins[6] = {X, Wqv, bqv, U, Wo, bo};
    const size_t insz[6] = {(size_t)T * C * es, (size_t)C * 2 * C * es, (size_t)2 * C * es,
                            (size_t)h * m * d * es, (size_t)C * C * es, (size_t)C * es};
    for (int i = 0; i < 6; ++i)
      if (ins[i] && overlaps(Y, yb, ins[i], insz[i])) return ANCHOR_ATTN_ERROR_INVALID_VALUE;

    // The attention reads Q and V from the projection [T, 2C] (head j's dims at columns
    // j*d .. and C + j*d ..) and writes H as [T, C] with the same head-major columns.
    g.vw.q = aa::View{(long long)n * 2 * C, d, 2 * C};
    g.vw.v = g.vw.q;
    g.vw.o = aa::View{(long long)n * C, d, C};

    // The Q|V projection fused in front of the layer (one kernel writes H) unless the split
    // plan is forced or the shape is outside that kernel's limits; otherwise the projection
    // runs through hipBLASLt and the layer reads it in place.
    const bool fuse = ctx->plan != ANCHOR_ATTN_PLAN_SPLIT && aa::block_fused_supported(g);
    DeviceGuard guard(ctx->device);
    if (!guard.ok) return ANCHOR_ATTN_ERROR_HIP;
    if (!ctx->gemm && !(ctx->gemm = aa::gemm_cache_create())) return ANCHOR_ATTN_ERROR_HIP;
    if ((!fuse && !aa::gemm_prepare(ctx->gemm, T, (int)C, (int)(2 * C), bqv != nullptr)) ||
        !aa::gemm_prepare(ctx->gemm, T, (int)C, (int)C, bo != nullptr))
      return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    if (!fuse) {
      st = prepare_forward(ctx, g, dtype);
      if (st != ANCHOR_ATTN_SUCCESS) return st;
    }
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t qvb = fuse ? 0 : al((size_t)T * 2 * C * es), hb = al((size_t)T * C * es);
    const size_t need = qvb + hb + aa::kGemmWorkspaceBytes;
    st = grow(ctx, &ctx->block_ws, &ctx->block_ws_bytes, need);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    char* w = (char*)ctx->block_ws;
    void* QV = w;
    void* Hb = w + qvb;
    void* gws = w + qvb + hb;
    hipStream_t s = (hipStream_t)stream;
    if (fuse) {
      if (aa::launch_block_fused_bf16(g, X, Wqv, bqv, U, Hb, s) != hipSuccess) {
        (void)hipGetLastError();
        return ANCHOR_ATTN_ERROR_HIP;
      }
    } else {
      if (aa::gemm_run(ctx->gemm, X, Wqv, bqv, QV, T, (int)C, (int)(2 * C), gws, s) != hipSuccess) {
        (void)hipGetLastError();
        return ANCHOR_ATTN_ERROR_HIP;
      }
      st = run_forward(ctx, g, dtype, QV, U, (const char*)QV + C * es, Hb, s);
      if (st != ANCHOR_ATTN_SUCCESS) return st;
    }
    if (aa::gemm_run(ctx->gemm, Hb, Wo, bo, Y, T, (int)C, (int)C, gws, s) != hipSuccess) {
      (void)hipGetLastError();
      return ANCHOR_ATTN_ERROR_HIP;
    }
    return ANCHOR_ATTN_SUCCESS;
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

anchor_attn_status_t anchor_attn_relu_linear_forward(
    anchor_attn_ctx* ctx, const void* Q, const long long* q_strides, const void* K,
    const long long* k_strides, const void* V, const long long* v_strides, void* O,
    const long long* o_strides, int B, int h, int n, int d, float cmin, float qscale,
    anchor_attn_dtype_t dtype, void* stream) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, 1, d, raw(&dtype), &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    if (!(cmin > 0.f) || !std::isfinite(cmin) || !(qscale > 0.f) || !std::isfinite(qscale))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (dtype != ANCHOR_ATTN_BF16) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    const size_t es = 2;
    aa::View qw = g.vw.q, kw = g.vw.q, vw = g.vw.q, ow = g.vw.q;
    if (!take_view(q_strides, es, &qw) || !take_view(k_strides, es, &kw) ||
        !take_view(v_strides, es, &vw) || !take_view(o_strides, es, &ow))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (empty) return ANCHOR_ATTN_SUCCESS;
    if (!Q || !K || !V || !O) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) & 15u)
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (!view_injective(ow, B, h, n, d)) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const size_t ox = view_extent(ow, B, h, n, d, es);
    if (overlaps(O, ox, Q, view_extent(qw, B, h, n, d, es)) ||
        overlaps(O, ox, K, view_extent(kw, B, h, n, d, es)) ||
        overlaps(O, ox, V, view_extent(vw, B, h, n, d, es)))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    DeviceGuard guard(ctx->device);
    if (!guard.ok) return ANCHOR_ATTN_ERROR_HIP;
    // One workgroup per slice once the slices fill half of the CUs (or when forced);
    // otherwise the split plan.
    const bool split = ctx->plan == ANCHOR_ATTN_PLAN_SPLIT ||
                       (ctx->plan == ANCHOR_ATTN_PLAN_AUTO && g.slices * 2 < ctx->num_cus);
    hipError_t e;
    if (split) {
      const aa::LinearSplitPlan p = make_linear_plan(g, ctx->num_cus);
      st = ensure_workspace(ctx, p.workspace_bytes());
      if (st != ANCHOR_ATTN_SUCCESS) return st;
      e = aa::launch_relu_linear_split_bf16(g, p, Q, qw, K, kw, V, vw, O, ow, cmin / qscale,
                                            ctx->workspace, (hipStream_t)stream);
    } else {
      e = aa::launch_relu_linear_bf16(g, Q, qw, K, kw, V, vw, O, ow, cmin / qscale, ctx->num_cus,
                                      (hipStream_t)stream);
    }
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return ANCHOR_ATTN_ERROR_HIP;
    }
    return ANCHOR_ATTN_SUCCESS;
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

anchor_attn_status_t anchor_attn_nystrom_forward(anchor_attn_ctx* ctx, const void* Q,
                                                 const void* K, const void* V, const int* idx,
                                                 void* H, int B, int h, int n, int s, int d,
                                                 anchor_attn_dtype_t dtype, void* stream) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    if (B < 0 || h < 0 || n < 0) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if ((long long)B * h * n == 0) return ANCHOR_ATTN_SUCCESS;
    if (s < 1 || s > n) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, s, d, raw(&dtype), &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    if (dtype != ANCHOR_ATTN_BF16 || s > 128 || (d == 128 && s > 96))
      return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    if (!Q || !K || !V || !idx || !H) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)H) & 15u) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if ((uintptr_t)idx & 3u) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const size_t bytes = (size_t)B * h * n * d * 2;
    if (overlaps(H, bytes, Q, bytes) || overlaps(H, bytes, K, bytes) ||
        overlaps(H, bytes, V, bytes) || overlaps(H, bytes, idx, (size_t)B * s * sizeof(int)))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    DeviceGuard guard(ctx->device);
    if (!guard.ok) return ANCHOR_ATTN_ERROR_HIP;
    const SplitPlan p = make_split_plan(g, dtype, ctx->num_cus);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t rows = al((size_t)g.slices * s * d * 2);
    const size_t cmax = al((size_t)g.slices * p.chunks1 * g.m_pad * sizeof(float));
    st = ensure_workspace(ctx, p.workspace_bytes() + rows + cmax);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    char* ws = (char*)ctx->workspace;
    aa::NystromBuffers nb{};
    nb.part = (float*)ws;
    nb.dpart = (float*)(ws + p.part_bytes);
    nb.wop = (__bf16*)(ws + p.part_bytes + p.dpart_bytes);
    nb.kt = (__bf16*)(ws + p.workspace_bytes());
    nb.cmax = (float*)(ws + p.workspace_bytes() + rows);
    const hipError_t e = aa::launch_nystrom_bf16(g, p, Q, K, V, idx, H, nb, (hipStream_t)stream);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return ANCHOR_ATTN_ERROR_HIP;
    }
    return ANCHOR_ATTN_SUCCESS;
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

static anchor_attn_status_t backward_strided_impl(
    anchor_attn_ctx* ctx, const void* Q, const long long* q_strides, const void* U, const void* V,
    const long long* v_strides, const void* dH, const long long* dh_strides, void* dQ,
    const long long* dq_strides, void* dU, void* dV, const long long* dv_strides, int B, int h,
    int n, int m, int d, int dtype_raw, void* stream) {
  if (!ctx) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
  try {
    Geometry g{};
    bool empty = false;
    anchor_attn_status_t st = check_shape(B, h, n, m, d, dtype_raw, &g, &empty);
    if (st != ANCHOR_ATTN_SUCCESS) return st;
    const anchor_attn_dtype_t dtype = (anchor_attn_dtype_t)dtype_raw;
    const Chosen plan = choose_backward(ctx, g, dtype);
    if (plan == Chosen::Unsupported) return ANCHOR_ATTN_ERROR_NOT_SUPPORTED;
    const size_t es = (dtype == ANCHOR_ATTN_FP32) ? 4 : 2;
    aa::BwdViews bv{g.vw.q, g.vw.q, g.vw.q, g.vw.q, g.vw.q};
    if (!take_view(q_strides, es, &bv.q) || !take_view(v_strides, es, &bv.v) ||
        !take_view(dh_strides, es, &bv.g) || !take_view(dq_strides, es, &bv.dq) ||
        !take_view(dv_strides, es, &bv.dv))
      return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const size_t ub = (size_t)h * (size_t)m * (size_t)d * es;
    if (ub > 0 && !dU) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (!empty && (!Q || !U || !V || !dH || !dQ || !dV)) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    const uintptr_t mis = ((uintptr_t)Q | (uintptr_t)U | (uintptr_t)V | (uintptr_t)dH |
                           (uintptr_t)dQ | (uintptr_t)dU | (uintptr_t)dV) & 15u;
    if (mis) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
    if (!empty) {
      if (!view_injective(bv.dq, B, h, n, d) || !view_injective(bv.dv, B, h, n, d))
        return ANCHOR_ATTN_ERROR_INVALID_VALUE;
      const void* ins[4] = {Q, V, dH, U};
      const size_t insz[4] = {view_extent(bv.q, B, h, n, d, es), view_extent(bv.v, B, h, n, d, es),
                              view_extent(bv.g, B, h, n, d, es), ub};
      void* outs[3] = {dQ, dV, dU};
      const size_t outsz[3] = {view_extent(bv.dq, B, h, n, d, es),
                               view_extent(bv.dv, B, h, n, d, es), ub};
      for (int o = 0; o < 3; ++o) {
        if (!outsz[o]) continue;
        for (int i = 0; i < 4; ++i)
          if (insz[i] && overlaps(outs[o], outsz[o], ins[i], insz[i])) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
        for (int o2 = o + 1; o2 < 3; ++o2)
          if (outsz[o2] && overlaps(outs[o], outsz[o], outs[o2], outsz[o2])) return ANCHOR_ATTN_ERROR_INVALID_VALUE;
      }
    }

    DeviceGuard guard(ctx->device);
    if (!guard.ok) return ANCHOR_ATTN_ERROR_HIP;
    hipStream_t s = (hipStream_t)stream;
    if (empty) {
      // no tokens: dU = 0 (dQ and dV are empty); a fill kernel, not a memset node
      if (ub > 0 && aa::launch_zero(dU, ub, s) != hipSuccess) {
        (void)hipGetLastError();
        return ANCHOR_ATTN_ERROR_HIP;
      }
      return ANCHOR_ATTN_SUCCESS;
    }
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    hipError_t e;
    if (plan == Chosen::Fused) {
      st = ensure_workspace(ctx, al((size_t)g.slices * g.m_pad * g.d * sizeof(float)));
      if (st != ANCHOR_ATTN_SUCCESS) return st;
      e = aa::launch_backward_fused_bf16(g, bv, Q, U, V, dH, dQ, dU, dV, (float*)ctx->workspace, s);
    } else if (dtype == ANCHOR_ATTN_FP32) {
      const SplitPlan p = make_split_plan(g, dtype, ctx->num_cus);
      const size_t part = al((size_t)g.slices * p.chunks1 * g.m_pad * g.d * sizeof(float));
      const size_t dpart = al((size_t)g.slices * p.chunks1 * g.m_pad * sizeof(float));
      const size_t rows = al((size_t)g.slices * g.m_pad * g.d * sizeof(float));
      const size_t ddb = al((size_t)g.slices * g.m_pad * sizeof(float));
      const size_t dsb = al((size_t)g.slices * (size_t)g.n * g.m_pad * sizeof(float));
      st = ensure_workspace(ctx, 3 * part + dpart + 2 * rows + ddb + dsb);
      if (st != ANCHOR_ATTN_SUCCESS) return st;
      char* w = (char*)ctx->workspace;
      aa::BackwardBuffersF32 wb{};
      wb.partP = (float*)w; w += part;
      wb.partG = (float*)w; w += part;
      wb.partU = (float*)w; w += part;
      wb.dpart = (float*)w; w += dpart;
      wb.wrm = (float*)w; w += rows;
      wb.dprm = (float*)w; w += rows;
      wb.dd = (float*)w; w += ddb;
      wb.ds = (float*)w;
      e = aa::launch_backward_fp32(g, p, wb, bv, Q, U, V, dH, dQ, dU, dV, s);
    } else {
      const SplitPlan p = aa::split_plan(g, true, ctx->num_cus, /*dual=*/g.d <= 64 || g.at <= 6);
      const size_t part = al((size_t)g.slices * p.chunks1 * g.m_pad * g.d * sizeof(float));
      const size_t dpart = al((size_t)g.slices * p.chunks1 * g.m_pad * sizeof(float));
      const size_t ops = al((size_t)g.slices * g.m_pad * g.d * es);
      const size_t ddb = al((size_t)g.slices * g.m_pad * sizeof(float));
      // per-token log-sum-exp from pass 1 to the token pass above 128 anchors
      const size_t lseb = g.at > 8 ? al((size_t)g.slices * g.n * sizeof(float)) : 0;
      st = ensure_workspace(ctx, 3 * part + dpart + 2 * ops + ddb + lseb);
      if (st != ANCHOR_ATTN_SUCCESS) return st;
      char* w = (char*)ctx->workspace;
      aa::BackwardBuffers wb{};
      wb.partP = (float*)w; w += part;
      wb.partG = (float*)w; w += part;
      wb.partU = (float*)w; w += part;
      wb.dpart = (float*)w; w += dpart;
      wb.wu = w; w += ops;
      wb.dprm = w; w += ops;
      wb.dd = (float*)w; w += ddb;
      wb.lse = lseb ? (float*)w : nullptr;
      aa::token_pass_chunks(g, p, ctx->num_cus, &wb.chunks_t, &wb.chunk_len_t);
      e = aa::launch_backward_bf16(g, p, wb, bv, Q, U, V, dH, dQ, dU, dV, s);
    }
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return ANCHOR_ATTN_ERROR_HIP;
    }
    return ANCHOR_ATTN_SUCCESS;
  } catch (...) {
    return ANCHOR_ATTN_ERROR_HIP;
  }
}

anchor_attn_status_t anchor_attn_backward_strided(
    anchor_attn_ctx* ctx, const void* Q, const long long* q_strides, const void* U, const void* V,
    const long long* v_strides, const void* dH, const long long* dh_strides, void* dQ,
    const long long* dq_strides, void* dU, void* dV, const long long* dv_strides, int B, int h,
    int n, int m, int d, anchor_attn_dtype_t dtype, void* stream) {
  return backward_strided_impl(ctx, Q, q_strides, U, V, v_strides, dH, dh_strides, dQ,
                               dq_strides, dU, dV, dv_strides, B, h, n, m, d, raw(&dtype), stream);
}

anchor_attn_status_t anchor_attn_backward(anchor_attn_ctx* ctx, const void* Q, const void* U,
                                          const void* V, const void* dH, void* dQ, void* dU,
                                          void* dV, int B, int h, int n, int m, int d,
                                          anchor_attn_dtype_t dtype, void* stream) {
  return backward_strided_impl(ctx, Q, nullptr, U, V, nullptr, dH, nullptr, dQ, nullptr, dU, dV,
                               nullptr, B, h, n, m, d, raw(&dtype), stream);
}

}  // extern "C"
