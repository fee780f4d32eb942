// Partial residency: a fixed set of HBM slots caching expert blobs that live
// in pinned host memory (host code only; the C ABI is in include/moe_layer.h).
//
// The pages stream experts that do not fit in fast memory from a larger,
// slower store, keep the frequently used ones resident in a bounded pool with
// a frequency plus recency policy, and order the GPU work with explicit hazard
// management (linlog.top article, core design 3, the expert cache pool;
// Swiftlet README translation, "How it works" and "Relation to
// TurboFieldfare"; kerneldigest.dev article, inference flow, the cache step).
// Here the store is pinned host memory, the fast memory is a slot pool in
// HBM, copies run on a caller-given side stream, and every ordering is
// expressed with HIP events, never with host waits:
//   - a slot is overwritten only after the compute_done event of the last
//     call that read it (write-after-read);
//   - compute waits on `ready`, recorded after all copies issued so far, and
//     copies of one cache are kept in issue order even across copy streams
//     (read-after-write, also for hits on blobs still in flight).
// Policy (a reading of "LFU + recency"): evict the resident blob, not needed
// by the current call and not held by a call not yet released, with the
// fewest uses; ties go to the oldest last use, then the lower (layer, id).
// Uses count once per call that needs the blob and restart at eviction.
// Empty slots are taken first, lowest slot first.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <set>
#include <tuple>
#include <vector>

#include "moe_layer.h"

namespace {

struct Slot {
  int32_t layer = -1, id = -1;   // resident blob, or -1 when empty
  int64_t uses = 0;
  int64_t last = -1;             // tick of the last call that needed it
  int32_t held = 0;              // acquires not yet released
  hipEvent_t reader = nullptr;   // compute_done of the last released reader
};

// Eviction order key: (occupied, uses, last use, layer, id, slot); empty slots
// sort first.
using Key = std::tuple<int, int64_t, int64_t, int32_t, int32_t, int32_t>;

}  // namespace

struct moe_cache {
  int32_t n_slots = 0, n_layers = 0, n_experts = 0;
  int64_t stride = 0;
  uint8_t* pool = nullptr;
  const uint8_t* host = nullptr;
  bool planning = false;               // no pool: policy only, no device work
  std::vector<Slot> slots;
  std::vector<int32_t> where;          // [layer * E + id] -> slot or -1
  std::set<Key> evictable;             // slots with held == 0
  std::vector<std::vector<std::vector<int32_t>>> pending;   // per layer: slot lists of unreleased acquires
  int64_t tick = 0, hits = 0, misses = 0, evictions = 0;
  hipEvent_t last_copies = nullptr;    // recorded after the latest acquire's copies
  hipStream_t last_stream = nullptr;
  bool any_copies = false;

  Key key(int32_t s) const {
    const Slot& x = slots[s];
    return Key(x.layer < 0 ? 0 : 1, x.uses, x.last, x.layer, x.id, s);
  }
  void hold(int32_t s) {
    if (slots[s].held++ == 0) evictable.erase(key(s));
  }
  void unhold(int32_t s) {
    if (--slots[s].held == 0) evictable.insert(key(s));
  }
};

namespace {

thread_local char g_cache_err[256];

int cache_fail(int code, const char* msg) {
  std::strncpy(g_cache_err, msg, sizeof(g_cache_err) - 1);
  return code;
}

}  // namespace

extern "C" {

moe_cache* moe_cache_create(int32_t n_slots, int64_t stride, void* pool_base, const void* host_pinned,
                            int32_t n_layers, int32_t n_experts) {
  if (n_slots < 1 || stride < 256 || stride % 256 || n_layers < 1 || n_experts < 1 || n_experts > 1024 ||
      static_cast<int64_t>(n_layers) * n_experts > (1 << 26))
    return nullptr;
  if ((pool_base == nullptr) != (host_pinned == nullptr)) return nullptr;
  if (pool_base && (reinterpret_cast<uintptr_t>(pool_base) & 255)) return nullptr;
  moe_cache* c = new moe_cache;
  c->n_slots = n_slots;
  c->n_layers = n_layers;
  c->n_experts = n_experts;
  c->stride = stride;
  c->pool = static_cast<uint8_t*>(pool_base);
  c->host = static_cast<const uint8_t*>(host_pinned);
  c->planning = pool_base == nullptr;
  c->slots.resize(n_slots);
  c->where.assign(static_cast<size_t>(n_layers) * n_experts, -1);
  c->pending.resize(n_layers);
  for (int32_t s = 0; s < n_slots; ++s) c->evictable.insert(c->key(s));
  if (!c->planning && hipEventCreateWithFlags(&c->last_copies, hipEventDisableTiming) != hipSuccess) {
    delete c;
    return nullptr;
  }
  return c;
}

int moe_cache_acquire(moe_cache* c, int32_t layer, const int32_t* ids_host, int32_t n, int64_t* slot_table_host,
                      void* copy_stream, void* ready) {
  if (!c || !ids_host || !slot_table_host || n < 0 || layer < 0 || layer >= c->n_layers)
    return cache_fail(MOE_EINVAL, "bad cache, layer, ids or slot table");
  if (!c->planning && !ready) return cache_fail(MOE_EINVAL, "ready event is NULL");
  const int32_t E = c->n_experts;
  // distinct experts of this call, in ascending id
  std::vector<char> need(E, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t e = ids_host[i];
    if (e < 0 || e >= E) return cache_fail(MOE_EINVAL, "expert id outside [0, n_experts)");
    need[e] = 1;
  }
  int32_t distinct = 0;
  for (int32_t e = 0; e < E; ++e) distinct += need[e];
  if (distinct > c->n_slots) return cache_fail(MOE_ENOSPC, "more distinct experts than slots");
  // Slots held by unreleased calls cannot be victims: check that enough remain.
  int32_t misses_needed = 0;
  for (int32_t e = 0; e < E; ++e)
    if (need[e] && c->where[static_cast<size_t>(layer) * E + e] < 0) ++misses_needed;
  int32_t free_victims = 0;
  for (const Key& k : c->evictable) {
    const int32_t s = std::get<5>(k);
    const Slot& x = c->slots[s];
    if (x.layer == layer && x.id >= 0 && need[x.id]) continue;
    if (++free_victims >= misses_needed) break;
  }
  if (free_victims < misses_needed)
    return cache_fail(MOE_ENOSPC, "not enough slots free of unreleased calls for this call's misses");

  const int64_t now = c->tick++;
  hipStream_t cs = static_cast<hipStream_t>(copy_stream);
  if (!c->planning && c->any_copies && cs != c->last_stream &&
      hipStreamWaitEvent(cs, c->last_copies, 0) != hipSuccess)
    return cache_fail(MOE_EHIP, "hipStreamWaitEvent failed");
  std::vector<int32_t> held;
  held.reserve(distinct);
  // hits first: they are held, so no miss of this call can evict them
  for (int32_t e = 0; e < E; ++e) {
    if (!need[e]) continue;
    const int32_t s = c->where[static_cast<size_t>(layer) * E + e];
    if (s < 0) continue;
    c->hold(s);
    Slot& x = c->slots[s];
    x.uses += 1;
    x.last = now;
    held.push_back(s);
    slot_table_host[e] = static_cast<int64_t>(s) * c->stride;
    ++c->hits;
  }
  hipEvent_t waited = nullptr;
  for (int32_t e = 0; e < E; ++e) {
    if (!need[e] || c->where[static_cast<size_t>(layer) * E + e] >= 0) continue;
    const int32_t s = std::get<5>(*c->evictable.begin());
    c->hold(s);
    Slot& x = c->slots[s];
    if (x.layer >= 0) {
      c->where[static_cast<size_t>(x.layer) * E + x.id] = -1;
      ++c->evictions;
    }
    if (!c->planning) {
      if (x.reader && x.reader != waited) {
        if (hipStreamWaitEvent(cs, x.reader, 0) != hipSuccess) return cache_fail(MOE_EHIP, "hipStreamWaitEvent failed");
        waited = x.reader;
      }
      const uint8_t* src = c->host + (static_cast<size_t>(layer) * E + e) * c->stride;
      if (hipMemcpyAsync(c->pool + static_cast<size_t>(s) * c->stride, src, c->stride, hipMemcpyHostToDevice, cs) !=
          hipSuccess)
        return cache_fail(MOE_EHIP, "hipMemcpyAsync failed");
      c->any_copies = true;
    }
    x.layer = layer;
    x.id = e;
    x.uses = 1;
    x.last = now;
    x.reader = nullptr;
    c->where[static_cast<size_t>(layer) * E + e] = s;
    held.push_back(s);
    slot_table_host[e] = static_cast<int64_t>(s) * c->stride;
    ++c->misses;
  }
  c->pending[layer].push_back(std::move(held));
  if (!c->planning) {
    if (hipEventRecord(static_cast<hipEvent_t>(ready), cs) != hipSuccess ||
        hipEventRecord(c->last_copies, cs) != hipSuccess)
      return cache_fail(MOE_EHIP, "hipEventRecord failed");
    c->last_stream = cs;
  }
  return MOE_OK;
}

int moe_cache_release(moe_cache* c, int32_t layer, void* compute_done) {
  if (!c || layer < 0 || layer >= c->n_layers) return cache_fail(MOE_EINVAL, "bad cache or layer");
  if (c->pending[layer].empty()) return cache_fail(MOE_EINVAL, "no unreleased acquire for this layer");
  if (!c->planning && !compute_done) return cache_fail(MOE_EINVAL, "compute_done event is NULL");
  std::vector<int32_t> held = std::move(c->pending[layer].front());
  c->pending[layer].erase(c->pending[layer].begin());
  for (int32_t s : held) {
    // the key does not involve the reader event, so it can change while held or not
    c->slots[s].reader = static_cast<hipEvent_t>(compute_done);
    c->unhold(s);
  }
  return MOE_OK;
}

void moe_cache_stats(const moe_cache* c, int64_t* hits, int64_t* misses, int64_t* evictions) {
  if (!c) return;
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (evictions) *evictions = c->evictions;
}

int moe_cache_slot_of(const moe_cache* c, int32_t layer, int32_t id) {
  if (!c || layer < 0 || layer >= c->n_layers || id < 0 || id >= c->n_experts) return -1;
  return c->where[static_cast<size_t>(layer) * c->n_experts + id];
}

void moe_cache_destroy(moe_cache* c) {
  if (!c) return;
  if (c->last_copies) hipEventDestroy(c->last_copies);
  delete c;
}

const char* moe_cache_last_error(void) { return g_cache_err; }

}  // extern "C"
