// Host side of the C ABI declared in include/moe_layer.h: argument checks,
// workspace layout and kernel sequencing.  Nothing here touches the device
// before every argument has been checked.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "moe_internal.h"

namespace {

thread_local std::string g_error;

// Caller-supplied timing events for the next forward call on this thread.
struct LaunchMarks {
  hipEvent_t ev[64];
  int32_t cap = 0;
  int32_t used = 0;
  int32_t* n_out = nullptr;
};
thread_local LaunchMarks g_marks;

// Scope of one API call that may consume the timing events: the destructor
// publishes the count and clears the setting when the call ends, whichever
// way it ends.
struct MarkScope {
  ~MarkScope() {
    if (g_marks.cap > 0 && g_marks.n_out) *g_marks.n_out = g_marks.used;
    g_marks.cap = 0;
    g_marks.used = 0;
    g_marks.n_out = nullptr;
  }
};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return MOE_OK;
}

bool pow2_in(int32_t v, int32_t lo, int32_t hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// True if the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

int64_t blob_bytes_raw(const moe_desc& d, int32_t inter) {
  const int64_t q = static_cast<int64_t>(d.hidden) * inter * d.bits / 8;
  const int64_t s = static_cast<int64_t>(d.hidden) * (inter / 64) * (d.sb_dtype == MOE_F32 ? 4 : 2);
  return 3 * q + 6 * s;
}

// Checks the descriptor; returns MOE_OK or MOE_EINVAL with the reason set.
int check_desc(const moe_desc* d) {
  if (!d) return fail(MOE_EINVAL, "descriptor is NULL");
  if (!pow2_in(d->hidden, 64, 2048)) return fail(MOE_EINVAL, "hidden=%d must be a power of two in [64, 2048]", d->hidden);
  if (!pow2_in(d->inter, 64, 2048)) return fail(MOE_EINVAL, "inter=%d must be a power of two in [64, 2048]", d->inter);
  if (!pow2_in(d->shared_inter, 64, 2048))
    return fail(MOE_EINVAL, "shared_inter=%d must be a power of two in [64, 2048]", d->shared_inter);
  if (d->n_experts < 1 || d->n_experts > 1024) return fail(MOE_EINVAL, "n_experts=%d must be in [1, 1024]", d->n_experts);
  if (d->top_k < 1 || d->top_k > d->n_experts || d->top_k > 64)
    return fail(MOE_EINVAL, "top_k=%d must be in [1, min(n_experts, 64)]", d->top_k);
  if (d->bits != 4 && d->bits != 8) return fail(MOE_EINVAL, "bits=%d must be 4 or 8", d->bits);
  if (d->group_size != 64) return fail(MOE_EINVAL, "group_size=%d must be 64", d->group_size);
  for (int32_t dt : {d->act_dtype, d->sb_dtype, d->out_dtype})
    if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_EINVAL, "dtype code %d is neither MOE_F32 nor MOE_BF16", dt);
  const int64_t rb = blob_bytes_raw(*d, d->inter), sb = blob_bytes_raw(*d, d->shared_inter);
  if (d->blob_stride < rb || d->blob_stride % 256)
    return fail(MOE_EINVAL, "blob_stride=%lld must be >= %lld and a multiple of 256", (long long)d->blob_stride,
                (long long)rb);
  if (d->shared_stride < sb || d->shared_stride % 256)
    return fail(MOE_EINVAL, "shared_stride=%lld must be >= %lld and a multiple of 256", (long long)d->shared_stride,
                (long long)sb);
  if (d->pool_bytes < rb) return fail(MOE_EINVAL, "pool_bytes=%lld smaller than one blob", (long long)d->pool_bytes);
  return MOE_OK;
}

int check_T(int32_t T) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d is negative", T);
  if (T > 65536) return fail(MOE_EINVAL, "T=%d exceeds 65536", T);
  return MOE_OK;
}

int check_ws(const moe_desc& d, int32_t T, const void* ws, size_t ws_bytes, moe::WsLayout* L) {
  if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
  *L = moe::ws_layout(d, T);
  if (ws_bytes < L->total)
    return fail(MOE_ENOMEM, "workspace has %zu bytes, %zu needed for T=%d", ws_bytes, L->total, T);
  return MOE_OK;
}

// Fused-kernel plans, cached per (device, shape, T): the occupancy query is
// host work that should not repeat on every call.
int cached_plan(const moe_desc& d, int T, moe::FusedPlan* plan) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int, int, int, int, int, int, int>, moe::FusedPlan> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  const auto key = std::make_tuple(dev, d.hidden, d.n_experts, d.top_k, d.inter, d.shared_inter, d.bits,
                                   d.act_dtype, d.sb_dtype, d.out_dtype, T);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) { *plan = it->second; return MOE_OK; }
  const int rc = moe::fused_plan(d, T, plan);
  if (rc == MOE_OK) cache[key] = *plan;
  return rc;
}

// Stack-kernel plans, cached per (device, E, k, output dtype).
int cached_stack_plan(const moe_desc& d, moe::StackPlan* plan) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int>, std::pair<int, moe::StackPlan>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  const auto key = std::make_tuple(dev, d.n_experts, d.top_k, d.out_dtype);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it == cache.end()) {
    moe::StackPlan p{};
    const int rc = moe::stack_plan(d, &p);
    it = cache.emplace(key, std::make_pair(rc, p)).first;
  }
  *plan = it->second.second;
  return it->second.first;
}

// Plans of the stack kernel for 2..8 tokens, cached per (device, E, k, output dtype).
int cached_stack_t_plan(const moe_desc& d, moe::StackPlan* plan) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int>, std::pair<int, moe::StackPlan>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  const auto key = std::make_tuple(dev, d.n_experts, d.top_k, d.out_dtype);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it == cache.end()) {
    moe::StackPlan p{};
    const int rc = moe::stack_t_plan(d, &p);
    it = cache.emplace(key, std::make_pair(rc, p)).first;
  }
  *plan = it->second.second;
  return it->second.first;
}

int finish(int rc) {
  if (rc != MOE_OK) {
    hipError_t e = hipGetLastError();
    return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point: one file-scope device array per
// GPU (each GPU the library runs on holds its own copy until the process
// ends), used as the workspace.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a host-side stand-in, not a device
// address): set-up looks up each device's address once with
// hipGetSymbolAddress, with that device current, and keeps it.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  void* ptr = nullptr;   // device address of this GPU's copy
  bool ready = false;    // cleared once (the first call on the device)
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's scratch address, cleared on `stream` at its first use; the
// clear is a fill kernel (no memset), so it may be captured in a graph.
int scratch_for_current_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ENODEV, "no current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ENODEV, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (!sl.ptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    sl.ptr = p;
  }
  if (!sl.ready) {
    if (moe::launch_ws_init(static_cast<uint8_t*>(sl.ptr), kScratchBytes, stream) != MOE_OK)
      return fail(MOE_EHIP, "clearing the scratch failed: %s", hipGetErrorString(hipGetLastError()));
    sl.ready = true;
  }
  *out = static_cast<uint8_t*>(sl.ptr);
  return MOE_OK;
}

}  // namespace

namespace moe {
// The thread's error text for entry points defined in other files.
int api_fail(int code, const char* msg) { return fail(code, "%s", msg); }
int api_ok() { return ok(); }
}  // namespace moe

namespace moe {
bool next_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (g_marks.used + 2 > g_marks.cap) return false;
  *start = g_marks.ev[g_marks.used];
  *stop = g_marks.ev[g_marks.used + 1];
  g_marks.used += 2;
  return true;
}
}  // namespace moe

extern "C" {

int64_t moe_blob_bytes(const moe_desc* d, int32_t shared) {
  if (check_desc(d) != MOE_OK) return -1;
  return blob_bytes_raw(*d, shared ? d->shared_inter : d->inter);
}

size_t moe_workspace_bytes(const moe_desc* d, int32_t T_max) {
  if (check_desc(d) != MOE_OK || check_T(T_max) != MOE_OK) return 0;
  return moe::ws_layout(*d, T_max).total;
}

int moe_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return fail(MOE_EINVAL, "workspace is NULL or not 256-byte aligned");
  if (ws_bytes < 256) return fail(MOE_ENOMEM, "workspace smaller than its control block");
  return finish(moe::launch_ws_init(static_cast<uint8_t*>(workspace), ws_bytes, static_cast<hipStream_t>(stream)));
}

int moe_router_topk(const moe_desc* d, int32_t T, const void* x, const void* router_w, int32_t* topk_ids,
                    float* topk_w, void* workspace, size_t ws_bytes, void* stream) {
  MarkScope marks;
  int rc;
  if ((rc = check_desc(d)) || (rc = check_T(T))) return rc;
  if (!x || !router_w || !topk_ids || !topk_w) return fail(MOE_EINVAL, "NULL x, router_w, topk_ids or topk_w");
  if (!aligned(x, 16) || !aligned(router_w, 16)) return fail(MOE_EINVAL, "x and router_w must be 16-byte aligned");
  moe::WsLayout L;
  if ((rc = check_ws(*d, T, workspace, ws_bytes, &L))) return rc;
  if (T == 0) return ok();
  moe::Call c{};
  c.d = *d;
  c.T = T;
  c.x = x;
  c.router_w = router_w;
  c.ws = static_cast<uint8_t*>(workspace);
  c.L = L;
  c.stream = static_cast<hipStream_t>(stream);
  if (moe::prefill_supported(*d, T)) return finish(moe::launch_prefill_router(c, topk_ids, topk_w));
  return finish(moe::launch_router_topk(c, topk_ids, topk_w));
}

int moe_experts_forward(const moe_desc* d, int32_t T, const void* x, const int32_t* topk_ids, const float* topk_w,
                        const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                        void* workspace, size_t ws_bytes, void* stream) {
  MarkScope marks;
  int rc;
  if ((rc = check_desc(d)) || (rc = check_T(T))) return rc;
  if (!x || !topk_ids || !topk_w || !slot_table || !pool_base || !shared_w || !out)
    return fail(MOE_EINVAL, "NULL input or output pointer");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(slot_table, 8) || !aligned(pool_base, 256) ||
      !aligned(shared_w, 256) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(MOE_EINVAL, "misaligned pointer (x/out 16, slot_table 8, pool_base/shared_w 256)");
  moe::WsLayout L;
  if ((rc = check_ws(*d, T, workspace, ws_bytes, &L))) return rc;
  if (T == 0) return ok();
  moe::Call c{};
  c.d = *d;
  c.T = T;
  c.x = x;
  c.slot_table = slot_table;
  c.pool = static_cast<const uint8_t*>(pool_base);
  c.shared = static_cast<const uint8_t*>(shared_w);
  c.out = out;
  c.ws = static_cast<uint8_t*>(workspace);
  c.L = L;
  c.ids = topk_ids;
  c.wts = topk_w;
  c.stream = static_cast<hipStream_t>(stream);
  if (moe::prefill_supported(*d, T)) return finish(moe::launch_prefill_experts(c));
  return finish(moe::launch_experts(c));
}

static int layer_forward(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                         const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                         void* workspace, size_t ws_bytes, int32_t* topk_ids, float* topk_w, void* stream,
                         bool allow_fused, void* x_next = nullptr) {
  MarkScope marks;
  int rc;
  if ((rc = check_desc(d)) || (rc = check_T(T))) return rc;
  if (!x || !router_w || !slot_table || !pool_base || !shared_w || !out)
    return fail(MOE_EINVAL, "NULL input or output pointer");
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(out, 16) || !aligned(slot_table, 8) ||
      !aligned(pool_base, 256) || !aligned(shared_w, 256))
    return fail(MOE_EINVAL, "misaligned pointer (x/router_w/out 16, slot_table 8, pool_base/shared_w 256)");
  if (x_next) {
    if (d->out_dtype != MOE_F32 || !aligned(x_next, 16))
      return fail(MOE_EINVAL, "x_next needs fp32 output and 16-byte alignment");
    // the fused combine writes out and x_next element by element while other
    // blocks still read x: x_next must share no byte with x or with out
    const size_t act = d->act_dtype == MOE_F32 ? 4 : 2, n = static_cast<size_t>(T) * d->hidden;
    if (overlaps(x_next, n * act, x, n * act) || overlaps(x_next, n * act, out, n * 4))
      return fail(MOE_EINVAL, "x_next overlaps x or out");
  }
  moe::WsLayout L;
  if ((rc = check_ws(*d, T, workspace, ws_bytes, &L))) return rc;
  if (T == 0) return ok();
  moe::Call c{};
  c.d = *d;
  c.T = T;
  c.x = x;
  c.x_next = x_next;
  c.router_w = router_w;
  c.slot_table = slot_table;
  c.pool = static_cast<const uint8_t*>(pool_base);
  c.shared = static_cast<const uint8_t*>(shared_w);
  c.out = out;
  c.ws = static_cast<uint8_t*>(workspace);
  c.L = L;
  c.ids = reinterpret_cast<const int32_t*>(c.ws + L.ids);
  c.wts = reinterpret_cast<const float*>(c.ws + L.wts);
  c.ids_out = topk_ids;
  c.wts_out = topk_w;
  c.stream = static_cast<hipStream_t>(stream);
  if (allow_fused && T == 1 && moe::stack_supported(*d)) {
    moe::StackPlan sp;
    if (cached_stack_plan(*d, &sp) == MOE_OK) {
      moe::StackCall sc{};
      sc.d = *d;
      sc.n_layers = 1;
      sc.T = 1;
      sc.x = x;
      sc.router_w = router_w;
      sc.slot_table = slot_table;
      sc.pool = c.pool;
      sc.shared = c.shared;
      sc.out = out;
      sc.x_chain = x_next;
      sc.ids_out = topk_ids;
      sc.wts_out = topk_w;
      sc.ws = c.ws;
      sc.L = L;
      sc.stream = c.stream;
      return finish(moe::launch_decode_stack(sc, sp));
    }
  }
  if (allow_fused && moe::fused_supported(*d, T)) {
    moe::FusedPlan plan;
    if (cached_plan(*d, T, &plan) == MOE_OK) return finish(moe::launch_decode_fused(c, plan));
  }
  // the other paths take the stack step as a kernel of its own
  const auto step = [&](int r) {
    if (r != MOE_OK || !x_next) return r;
    return moe::launch_residual(d->act_dtype, x, static_cast<const float*>(out), x_next,
                                static_cast<int64_t>(T) * d->hidden, c.stream);
  };
  if (allow_fused && moe::prefill_supported(*d, T)) {
    if ((rc = moe::launch_prefill_router(c, topk_ids, topk_w))) return finish(rc);
    return finish(step(moe::launch_prefill_experts(c)));
  }
  if ((rc = moe::launch_router_topk(c, topk_ids, topk_w))) return finish(rc);
  return finish(step(moe::launch_experts(c)));
}

int moe_stack_forward(const moe_desc* d, int32_t n_layers, int32_t T, const void* x, int64_t x_stride,
                      const void* router_w, int64_t router_stride, const int64_t* slot_table, int64_t slot_stride,
                      const void* pool_base, const void* shared_w, int64_t shared_stride, void* out,
                      int64_t out_stride, void* x_chain, int64_t chain_stride, int32_t* topk_ids, float* topk_w,
                      void* workspace, size_t ws_bytes, void* stream) {
  MarkScope marks;
  int rc;
  if ((rc = check_desc(d)) || (rc = check_T(T))) return rc;
  if (n_layers < 0 || n_layers > 4096) return fail(MOE_EINVAL, "n_layers=%d must be in [0, 4096]", n_layers);
  if (!x || !router_w || !slot_table || !pool_base || !shared_w || !out)
    return fail(MOE_EINVAL, "NULL input or output pointer");
  const size_t act = d->act_dtype == MOE_F32 ? 4 : 2, outsz = d->out_dtype == MOE_F32 ? 4 : 2;
  const int64_t xb = static_cast<int64_t>(T) * d->hidden * act, ob = static_cast<int64_t>(T) * d->hidden * outsz;
  const int64_t rbytes = static_cast<int64_t>(d->n_experts) * d->hidden * act;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(out, 16) || !aligned(slot_table, 8) ||
      !aligned(pool_base, 256) || !aligned(shared_w, 256) || (x_chain && !aligned(x_chain, 16)))
    return fail(MOE_EINVAL, "misaligned pointer (x/router_w/out/x_chain 16, slot_table 8, pool_base/shared_w 256)");
  if (n_layers > 1 &&
      ((!x_chain && (x_stride < xb || x_stride % 16)) || router_stride < rbytes || router_stride % 16 ||
       slot_stride < static_cast<int64_t>(d->n_experts) * 8 || slot_stride % 8 || shared_stride < d->shared_stride ||
       shared_stride % 256 || out_stride < ob || out_stride % 16 || (x_chain && (chain_stride < xb || chain_stride % 16))))
    return fail(MOE_EINVAL, "a per-layer stride is smaller than one layer's data or misaligned");
  if (x_chain) {
    if (d->out_dtype != MOE_F32) return fail(MOE_EINVAL, "x_chain needs fp32 output");
    const int64_t span = (n_layers - 1) * chain_stride + xb;
    if (overlaps(x_chain, span, x, xb) || overlaps(x_chain, span, out, (n_layers - 1) * out_stride + ob))
      return fail(MOE_EINVAL, "x_chain overlaps x or out");
  }
  moe::WsLayout L;
  if ((rc = check_ws(*d, T, workspace, ws_bytes, &L))) return rc;
  if (T == 0 || n_layers == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 1 && moe::stack_supported(*d)) {
    moe::StackPlan sp;
    if (cached_stack_plan(*d, &sp) == MOE_OK) {
      moe::StackCall sc{};
      sc.d = *d;
      sc.n_layers = n_layers;
      sc.T = 1;
      sc.x = x;
      sc.x_stride = x_stride;
      sc.router_w = router_w;
      sc.router_stride = router_stride;
      sc.slot_table = slot_table;
      sc.slot_stride = slot_stride;
      sc.pool = static_cast<const uint8_t*>(pool_base);
      sc.shared = static_cast<const uint8_t*>(shared_w);
      sc.shared_stride = shared_stride;
      sc.out = out;
      sc.out_stride = out_stride;
      sc.x_chain = x_chain;
      sc.chain_stride = chain_stride;
      sc.ids_out = topk_ids;
      sc.wts_out = topk_w;
      sc.ws = static_cast<uint8_t*>(workspace);
      sc.L = L;
      sc.stream = st;
      return finish(moe::launch_decode_stack(sc, sp));
    }
  }
  if (!x_chain && moe::stack_t_supported(*d, T)) {
    moe::StackPlan sp;
    if (cached_stack_t_plan(*d, &sp) == MOE_OK) {
      moe::StackCall sc{};
      sc.d = *d;
      sc.n_layers = n_layers;
      sc.T = T;
      sc.x = x;
      sc.x_stride = x_stride;
      sc.router_w = router_w;
      sc.router_stride = router_stride;
      sc.slot_table = slot_table;
      sc.slot_stride = slot_stride;
      sc.pool = static_cast<const uint8_t*>(pool_base);
      sc.shared = static_cast<const uint8_t*>(shared_w);
      sc.shared_stride = shared_stride;
      sc.out = out;
      sc.out_stride = out_stride;
      sc.ids_out = topk_ids;
      sc.wts_out = topk_w;
      sc.ws = static_cast<uint8_t*>(workspace);
      sc.L = L;
      sc.stream = st;
      return finish(moe::launch_decode_stack_t(sc, sp));
    }
  }
  // any other shape or T: the layers one call after another
  const size_t k = static_cast<size_t>(T) * d->top_k;
  for (int32_t l = 0; l < n_layers; ++l) {
    const uint8_t* xl = (x_chain && l > 0) ? static_cast<const uint8_t*>(x_chain) + (l - 1) * chain_stride
                                           : static_cast<const uint8_t*>(x) + l * x_stride;
    const uint8_t* rl = static_cast<const uint8_t*>(router_w) + l * router_stride;
    const int64_t* sl = reinterpret_cast<const int64_t*>(reinterpret_cast<const uint8_t*>(slot_table) + l * slot_stride);
    const uint8_t* shl = static_cast<const uint8_t*>(shared_w) + l * shared_stride;
    uint8_t* ol = static_cast<uint8_t*>(out) + l * out_stride;
    int32_t* il = topk_ids ? topk_ids + l * k : nullptr;
    float* wl = topk_w ? topk_w + l * k : nullptr;
    if (x_chain)
      rc = moe_layer_forward_chain(d, T, xl, rl, sl, pool_base, shl, ol,
                                   static_cast<uint8_t*>(x_chain) + l * chain_stride, workspace, ws_bytes, il, wl,
                                   stream);
    else
      rc = moe_layer_forward(d, T, xl, rl, sl, pool_base, shl, ol, workspace, ws_bytes, il, wl, stream);
    if (rc != MOE_OK) return rc;
  }
  return ok();
}

int moe_layer_forward_chain(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                            const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                            void* x_next, void* workspace, size_t ws_bytes, int32_t* topk_ids, float* topk_w,
                            void* stream) {
  if (!x_next) return fail(MOE_EINVAL, "NULL x_next");
  return layer_forward(d, T, x, router_w, slot_table, pool_base, shared_w, out, workspace, ws_bytes, topk_ids,
                       topk_w, stream, true, x_next);
}

int moe_layer_forward(const moe_desc* d, int32_t T, const void* x, const void* router_w, const int64_t* slot_table,
                      const void* pool_base, const void* shared_w, void* out, void* workspace, size_t ws_bytes,
                      int32_t* topk_ids, float* topk_w, void* stream) {
  return layer_forward(d, T, x, router_w, slot_table, pool_base, shared_w, out, workspace, ws_bytes, topk_ids,
                       topk_w, stream, true);
}

int moe_layer_forward_staged(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                             const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                             void* workspace, size_t ws_bytes, int32_t* topk_ids, float* topk_w, void* stream) {
  return layer_forward(d, T, x, router_w, slot_table, pool_base, shared_w, out, workspace, ws_bytes, topk_ids,
                       topk_w, stream, false);
}

int moe_layer_forward_noalloc(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                              const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                              int32_t* topk_ids, float* topk_w, uint32_t* status, void* stream) {
  int rc;
  if ((rc = check_desc(d)) || (rc = check_T(T))) return rc;
  const size_t need = moe::ws_layout(*d, T).total;
  if (need > kScratchBytes)
    return fail(MOE_ENOMEM, "T=%d needs %zu bytes of workspace; the no-allocation entry point has %zu", T, need,
                kScratchBytes);
  if (status && !aligned(status, 4)) return fail(MOE_EINVAL, "status must be 4-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  if (T > 0 && (rc = scratch_for_current_device(st, &ws))) return rc;
  if (T == 0) {
    // the argument checks of moe_layer_forward, nothing enqueued: any
    // 256-aligned workspace address passes them, and none is touched
    static __align__(256) uint8_t no_ws[256];
    return layer_forward(d, T, x, router_w, slot_table, pool_base, shared_w, out, no_ws, need, topk_ids, topk_w,
                         stream, true);
  }
  if ((rc = layer_forward(d, T, x, router_w, slot_table, pool_base, shared_w, out, ws, kScratchBytes, topk_ids,
                          topk_w, stream, true)))
    return rc;
  if (status) return finish(moe::launch_take_flags(reinterpret_cast<uint32_t*>(ws + moe::ws_layout(*d, T).ctrl),
                                                   status, st));
  return MOE_OK;
}

int moe_layer_forward_scalar(const moe_desc* d, int32_t T, const void* x, const void* router_w,
                             const int64_t* slot_table, const void* pool_base, const void* shared_w, void* out,
                             void* workspace, size_t ws_bytes, int32_t* topk_ids, float* topk_w, void* stream) {
  MarkScope marks;
  int rc;
  if ((rc = check_desc(d)) || (rc = check_T(T))) return rc;
  if (!x || !router_w || !slot_table || !pool_base || !shared_w || !out)
    return fail(MOE_EINVAL, "NULL input or output pointer");
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(out, 16) || !aligned(slot_table, 8) ||
      !aligned(pool_base, 256) || !aligned(shared_w, 256))
    return fail(MOE_EINVAL, "misaligned pointer (x/router_w/out 16, slot_table 8, pool_base/shared_w 256)");
  moe::WsLayout L;
  if ((rc = check_ws(*d, T, workspace, ws_bytes, &L))) return rc;
  if (T == 0) return ok();
  moe::Call c{};
  c.d = *d;
  c.T = T;
  c.x = x;
  c.router_w = router_w;
  c.slot_table = slot_table;
  c.pool = static_cast<const uint8_t*>(pool_base);
  c.shared = static_cast<const uint8_t*>(shared_w);
  c.out = out;
  c.ws = static_cast<uint8_t*>(workspace);
  c.L = L;
  c.ids_out = topk_ids;
  c.wts_out = topk_w;
  c.stream = static_cast<hipStream_t>(stream);
  return finish(moe::launch_scalar(c));
}

int moe_residual_add(int32_t T, int32_t H, int32_t act_dtype, const void* x, const float* y, void* x_next,
                     void* stream) {
  if (T < 0 || H < 1 || static_cast<int64_t>(T) * H >= (int64_t(1) << 31))
    return fail(MOE_EINVAL, "T must be >= 0 and H >= 1, with T * H < 2^31");
  if (act_dtype != MOE_F32 && act_dtype != MOE_BF16) return fail(MOE_EINVAL, "act_dtype must be MOE_F32 or MOE_BF16");
  if (!x || !y || !x_next) return fail(MOE_EINVAL, "NULL x, y or x_next");
  {
    // each element is read and then written by one thread: x_next may be x
    // exactly, but no other overlap with x or y is race-free
    const size_t n = static_cast<size_t>(T) * H, act = act_dtype == MOE_F32 ? 4 : 2;
    if ((x_next != x && overlaps(x_next, n * act, x, n * act)) || overlaps(x_next, n * act, y, n * 4))
      return fail(MOE_EINVAL, "x_next overlaps y, or overlaps x other than exactly in place");
  }
  if (T == 0) return ok();
  return finish(moe::launch_residual(act_dtype, x, y, x_next,
                                     static_cast<int64_t>(T) * H, static_cast<hipStream_t>(stream)));
}

int moe_status_check(void* workspace, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return fail(MOE_EINVAL, "workspace is NULL or not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t flags = 0, zero = 0;
  if (hipMemcpyAsync(&flags, workspace, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(MOE_EHIP, "status read failed: %s", hipGetErrorString(hipGetLastError()));
  if (flags) {
    if (hipMemcpyAsync(workspace, &zero, 4, hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return fail(MOE_EHIP, "status clear failed: %s", hipGetErrorString(hipGetLastError()));
    if (flags & 2u)
      return fail(MOE_ETIMEOUT, "a bounded in-kernel wait of the fused decode kernel expired; its output is invalid");
    if (flags & 1u)
      return fail(MOE_ERANGE, "a kernel skipped a pair: slot offset outside the pool or expert id outside [0, E)");
    return fail(MOE_EOVERFLOW, "the prefill path rounded a value outside the float16 range; the output holds inf or NaN");
  }
  return ok();
}

int moe_set_launch_events(void* const* events, int32_t capacity, int32_t* n_recorded) {
  g_marks.cap = 0;
  g_marks.used = 0;
  g_marks.n_out = nullptr;
  if (!events) return ok();
  if (capacity < 1 || !n_recorded) return fail(MOE_EINVAL, "capacity must be >= 1 and n_recorded non-NULL");
  const int32_t n = capacity < 64 ? capacity : 64;
  for (int32_t i = 0; i < n; ++i) g_marks.ev[i] = static_cast<hipEvent_t>(events[i]);
  *n_recorded = 0;
  g_marks.cap = n;
  g_marks.n_out = n_recorded;
  return ok();
}

const char* moe_last_error(void) { return g_error.c_str(); }

}  // extern "C"
