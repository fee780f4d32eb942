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
//
// The expert store (moe_store_*) is the slow tier on disk: one container file
// of fixed-stride blobs, so that an expert is fetched with one positioned read
// at an offset computed from (layer, id), with no mapping of the file into the
// address space (linlog.top article, core design 2, fixed-stride reads;
// Swiftlet README translation, "How it works").  A cache built on a store
// reads each miss into one of a few pinned staging buffers and copies it from
// there into its slot on the copy stream; a staging buffer is read into again
// only after its previous copy has finished (a host wait on its event).
#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cerrno>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <set>
#include <thread>
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

struct moe_store {
  int fd = -1;
  int32_t n_layers = 0, n_experts = 0;
  int64_t stride = 0, blob_bytes = 0;
  bool direct = false, writable = false;
  uint8_t* bounce = nullptr;   // O_DIRECT: page-aligned pageable buffer the reads land in
};

struct moe_cache {
  int32_t n_slots = 0, n_layers = 0, n_experts = 0;
  int64_t stride = 0;
  uint8_t* pool = nullptr;
  const uint8_t* host = nullptr;
  moe_store* store = nullptr;          // misses read from this file instead of `host`
  uint8_t* staging = nullptr;          // [n_staging][stride] pinned
  int32_t n_staging = 0, next_stage = 0;
  std::vector<hipEvent_t> stage_ev;    // recorded after the copy out of each staging buffer
  std::vector<char> stage_busy;
  uint8_t* bounce = nullptr;           // O_DIRECT store: [n_staging][stride] page-aligned, pageable
  bool planning = false;               // no pool: policy only, no device work
  std::vector<Slot> slots;
  std::vector<int32_t> where;          // [layer * E + id] -> slot or -1
  std::set<Key> evictable;             // slots with held == 0
  std::vector<std::vector<std::vector<int32_t>>> pending;   // per layer: slot lists of unreleased acquires
  int64_t tick = 0, hits = 0, misses = 0, evictions = 0;
  hipEvent_t last_copies = nullptr;    // recorded after the latest acquire's copies
  hipStream_t last_stream = nullptr;
  bool any_copies = false;
  bool keep_counts = true;             // MOE_CACHE_KEEP_COUNTS (the default): uses survive eviction
  std::vector<int64_t> count;          // [layer * E + id] uses so far (kept across evictions)
  int64_t fault_at = -1;               // copies until an injected failure (-1: none)

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

int io_fail(const char* what, int err) {
  std::snprintf(g_cache_err, sizeof(g_cache_err), "%s: %s", what, err ? std::strerror(err) : "file ends early");
  return MOE_EIO;
}

constexpr int64_t kStoreHeader = 4096;
constexpr char kStoreMagic[8] = {'M', 'O', 'E', 'B', 'L', 'O', 'B', '1'};

struct StoreHeader {
  char magic[8];
  int32_t n_layers, n_experts;
  int64_t stride, blob_bytes;
};

bool store_shape_ok(int32_t n_layers, int32_t n_experts, int64_t stride, int64_t blob_bytes) {
  if (n_layers < 1 || n_experts < 1 || stride < 4096 || stride % 4096 || blob_bytes < 1 || blob_bytes > stride)
    return false;
  // total size fits a signed 64-bit file offset with room to spare
  return static_cast<double>(n_layers) * n_experts * static_cast<double>(stride) < 4.0e18;
}

int64_t blob_offset(const moe_store* s, int32_t layer, int32_t id) {
  return kStoreHeader + (static_cast<int64_t>(layer) * s->n_experts + id) * s->stride;
}

// Positioned transfer of exactly n bytes, resuming after short counts.
template <typename F>
int full_io(F op, int64_t n, const char* what) {
  int64_t done = 0;
  while (done < n) {
    const ssize_t r = op(done, n - done);
    if (r < 0) {
      if (errno == EINTR) continue;
      return io_fail(what, errno);
    }
    if (r == 0) return io_fail(what, 0);
    done += r;
  }
  return MOE_OK;
}

// With O_DIRECT the read lands in a page-aligned pageable buffer (the store's
// own, or one per staging buffer of a cache) and is copied out: the kernel
// cannot pin pages of a HIP pinned allocation for a direct transfer (the read
// fails with EFAULT), and a caller's buffer need not be aligned.  Reads of
// one store may run concurrently (pread has no file position).
int store_read(moe_store* s, int32_t layer, int32_t id, void* dst, uint8_t* bounce) {
  uint8_t* p = s->direct ? bounce : static_cast<uint8_t*>(dst);
  const int64_t off = blob_offset(s, layer, id);
  const int rc =
      full_io([&](int64_t done, int64_t left) { return pread(s->fd, p + done, static_cast<size_t>(left), off + done); },
              s->stride, "pread of an expert blob");
  if (rc == MOE_OK && s->direct) std::memcpy(dst, p, static_cast<size_t>(s->stride));
  return rc;
}

}  // namespace

namespace {

// True if the copy about to be issued is the one an injected fault targets
// (moe_cache_inject_fault); the fault then disarms.
bool take_fault(moe_cache* c) {
  if (c->fault_at < 0) return false;
  if (c->fault_at-- == 0) {
    c->fault_at = -1;
    return true;
  }
  return false;
}

struct MissJob {
  int32_t e, s;
  hipEvent_t reader;   // compute_done of the slot's last reader, or null
};

// The copy into a victim slot waits for the last reader of that slot.
int wait_reader(hipStream_t cs, const MissJob& j, hipEvent_t* waited) {
  if (j.reader && j.reader != *waited) {
    if (hipStreamWaitEvent(cs, j.reader, 0) != hipSuccess) return cache_fail(MOE_EHIP, "hipStreamWaitEvent failed");
    *waited = j.reader;
  }
  return MOE_OK;
}

int copy_from_host(moe_cache* c, int32_t layer, const std::vector<MissJob>& jobs, hipStream_t cs) {
  hipEvent_t waited = nullptr;
  for (const MissJob& j : jobs) {
    if (wait_reader(cs, j, &waited) != MOE_OK) return MOE_EHIP;
    const uint8_t* src = c->host + (static_cast<size_t>(layer) * c->n_experts + j.e) * c->stride;
    if (take_fault(c)) return cache_fail(MOE_EHIP, "injected copy failure");
    if (hipMemcpyAsync(c->pool + static_cast<size_t>(j.s) * c->stride, src, c->stride, hipMemcpyHostToDevice, cs) !=
        hipSuccess)
      return cache_fail(MOE_EHIP, "hipMemcpyAsync failed");
  }
  return MOE_OK;
}

// Misses in batches of up to n_staging: each batch waits for the copies out of
// its staging buffers issued earlier, reads its blobs with one positioned read
// each, concurrently (one thread per blob: a single synchronous read stream
// leaves the device mostly idle), then issues the copies in order.
int copy_from_store(moe_cache* c, int32_t layer, const std::vector<MissJob>& jobs, hipStream_t cs) {
  hipEvent_t waited = nullptr;
  const size_t n = jobs.size();
  std::vector<int32_t> stage(c->n_staging);
  std::vector<int> rc(c->n_staging);
  for (size_t b = 0; b < n; b += c->n_staging) {
    const int m = static_cast<int>(std::min<size_t>(c->n_staging, n - b));
    for (int i = 0; i < m; ++i) {
      stage[i] = c->next_stage;
      c->next_stage = (c->next_stage + 1) % c->n_staging;
      if (c->stage_busy[stage[i]] && hipEventSynchronize(c->stage_ev[stage[i]]) != hipSuccess)
        return cache_fail(MOE_EHIP, "hipEventSynchronize failed");
    }
    auto read_one = [&](int i) {
      const size_t off = static_cast<size_t>(stage[i]) * c->stride;
      rc[i] = store_read(c->store, layer, jobs[b + i].e, c->staging + off, c->bounce ? c->bounce + off : nullptr);
    };
    std::vector<std::thread> pool;
    for (int i = 1; i < m; ++i) pool.emplace_back(read_one, i);
    read_one(0);
    for (std::thread& t : pool) t.join();
    for (int i = 0; i < m; ++i)
      if (rc[i] != MOE_OK) return rc[i];
    for (int i = 0; i < m; ++i) {
      const MissJob& j = jobs[b + i];
      if (wait_reader(cs, j, &waited) != MOE_OK) return MOE_EHIP;
      if (take_fault(c)) return cache_fail(MOE_EHIP, "injected copy failure");
      if (hipMemcpyAsync(c->pool + static_cast<size_t>(j.s) * c->stride,
                         c->staging + static_cast<size_t>(stage[i]) * c->stride, c->stride, hipMemcpyHostToDevice,
                         cs) != hipSuccess)
        return cache_fail(MOE_EHIP, "hipMemcpyAsync failed");
      if (hipEventRecord(c->stage_ev[stage[i]], cs) != hipSuccess) return cache_fail(MOE_EHIP, "hipEventRecord failed");
      c->stage_busy[stage[i]] = 1;
    }
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_store* moe_store_create(const char* path, int32_t n_layers, int32_t n_experts, int64_t stride,
                            int64_t blob_bytes) {
  if (!path || !store_shape_ok(n_layers, n_experts, stride, blob_bytes)) {
    cache_fail(MOE_EINVAL, "bad path or store shape (stride must be a positive multiple of 4096)");
    return nullptr;
  }
  const int fd = open(path, O_RDWR | O_CREAT | O_TRUNC | O_CLOEXEC, 0644);
  if (fd < 0) {
    io_fail("open of the store file", errno);
    return nullptr;
  }
  uint8_t head[kStoreHeader] = {};
  StoreHeader h;
  std::memcpy(h.magic, kStoreMagic, 8);
  h.n_layers = n_layers;
  h.n_experts = n_experts;
  h.stride = stride;
  h.blob_bytes = blob_bytes;
  std::memcpy(head, &h, sizeof(h));
  const int64_t total = kStoreHeader + static_cast<int64_t>(n_layers) * n_experts * stride;
  if (full_io([&](int64_t done, int64_t left) { return pwrite(fd, head + done, static_cast<size_t>(left), done); },
              kStoreHeader, "write of the store header") != MOE_OK) {
    close(fd);
    return nullptr;
  }
  if (ftruncate(fd, total) != 0) {
    io_fail("sizing of the store file", errno);
    close(fd);
    return nullptr;
  }
  moe_store* s = new moe_store;
  s->fd = fd;
  s->n_layers = n_layers;
  s->n_experts = n_experts;
  s->stride = stride;
  s->blob_bytes = blob_bytes;
  s->writable = true;
  return s;
}

moe_store* moe_store_open(const char* path, int32_t flags) {
  if (!path || (flags & ~MOE_STORE_DIRECT)) {
    cache_fail(MOE_EINVAL, "bad path or flags");
    return nullptr;
  }
  const bool direct = (flags & MOE_STORE_DIRECT) != 0;
  const int fd = open(path, O_RDONLY | O_CLOEXEC | (direct ? O_DIRECT : 0));
  if (fd < 0) {
    io_fail(direct ? "open of the store file with O_DIRECT" : "open of the store file", errno);
    return nullptr;
  }
  // the header is read through an aligned buffer (O_DIRECT needs one)
  void* head = nullptr;
  if (posix_memalign(&head, 4096, kStoreHeader) != 0) {
    cache_fail(MOE_EINVAL, "out of host memory");
    close(fd);
    return nullptr;
  }
  uint8_t* hb = static_cast<uint8_t*>(head);
  StoreHeader h;
  struct stat st;
  const int rc = full_io([&](int64_t done, int64_t left) { return pread(fd, hb + done, static_cast<size_t>(left), done); },
                         kStoreHeader, "read of the store header");
  std::memcpy(&h, hb, sizeof(h));
  free(head);
  if (rc != MOE_OK) {
    close(fd);
    return nullptr;
  }
  if (std::memcmp(h.magic, kStoreMagic, 8) != 0 || !store_shape_ok(h.n_layers, h.n_experts, h.stride, h.blob_bytes) ||
      fstat(fd, &st) != 0 ||
      st.st_size < kStoreHeader + static_cast<int64_t>(h.n_layers) * h.n_experts * h.stride) {
    cache_fail(MOE_EIO, "the file is not an expert store, or is shorter than its header says");
    close(fd);
    return nullptr;
  }
  void* bounce = nullptr;
  if (direct && posix_memalign(&bounce, 4096, static_cast<size_t>(h.stride)) != 0) {
    cache_fail(MOE_EINVAL, "out of host memory");
    close(fd);
    return nullptr;
  }
  moe_store* s = new moe_store;
  s->fd = fd;
  s->n_layers = h.n_layers;
  s->n_experts = h.n_experts;
  s->stride = h.stride;
  s->blob_bytes = h.blob_bytes;
  s->direct = direct;
  s->bounce = static_cast<uint8_t*>(bounce);
  return s;
}

int moe_store_info(const moe_store* s, int32_t* n_layers, int32_t* n_experts, int64_t* stride, int64_t* blob_bytes) {
  if (!s) return cache_fail(MOE_EINVAL, "store is NULL");
  if (n_layers) *n_layers = s->n_layers;
  if (n_experts) *n_experts = s->n_experts;
  if (stride) *stride = s->stride;
  if (blob_bytes) *blob_bytes = s->blob_bytes;
  return MOE_OK;
}

int moe_store_read(moe_store* s, int32_t layer, int32_t id, void* dst_host) {
  if (!s || !dst_host || layer < 0 || layer >= s->n_layers || id < 0 || id >= s->n_experts)
    return cache_fail(MOE_EINVAL, "bad store, destination, layer or id");
  return store_read(s, layer, id, dst_host, s->bounce);
}

int moe_store_write(moe_store* s, int32_t layer, int32_t id, const void* src_host) {
  if (!s || !src_host || layer < 0 || layer >= s->n_layers || id < 0 || id >= s->n_experts)
    return cache_fail(MOE_EINVAL, "bad store, source, layer or id");
  if (!s->writable) return cache_fail(MOE_EINVAL, "store opened read-only");
  const uint8_t* p = static_cast<const uint8_t*>(src_host);
  const int64_t off = blob_offset(s, layer, id);
  return full_io([&](int64_t done, int64_t left) { return pwrite(s->fd, p + done, static_cast<size_t>(left), off + done); },
                 s->stride, "pwrite of an expert blob");
}

void moe_store_close(moe_store* s) {
  if (!s) return;
  if (s->fd >= 0) close(s->fd);
  free(s->bounce);
  delete s;
}

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
  c->count.assign(static_cast<size_t>(n_layers) * n_experts, 0);
  c->pending.resize(n_layers);
  for (int32_t s = 0; s < n_slots; ++s) c->evictable.insert(c->key(s));
  if (!c->planning && hipEventCreateWithFlags(&c->last_copies, hipEventDisableTiming) != hipSuccess) {
    delete c;
    return nullptr;
  }
  return c;
}

moe_cache* moe_cache_create_from_store(int32_t n_slots, void* pool_base, moe_store* store, void* staging_pinned,
                                       int32_t n_staging) {
  if (!store || !pool_base || !staging_pinned || n_staging < 1 || n_staging > 64) {
    cache_fail(MOE_EINVAL, "bad store, pool, staging or staging count (1..64)");
    return nullptr;
  }
  // the store's stride is a multiple of 4096, so of 256 as the pool needs;
  // host_pinned stands in for "a source is given" until the store replaces it
  moe_cache* c = moe_cache_create(n_slots, store->stride, pool_base, staging_pinned, store->n_layers, store->n_experts);
  if (!c) {
    cache_fail(MOE_EINVAL, "bad slot count or pool alignment");
    return nullptr;
  }
  c->host = nullptr;
  c->store = store;
  c->staging = static_cast<uint8_t*>(staging_pinned);
  c->n_staging = n_staging;
  c->stage_ev.assign(n_staging, nullptr);
  c->stage_busy.assign(n_staging, 0);
  void* bounce = nullptr;
  if (store->direct) {
    if (posix_memalign(&bounce, 4096, static_cast<size_t>(n_staging) * store->stride) != 0) {
      moe_cache_destroy(c);
      cache_fail(MOE_EINVAL, "out of host memory");
      return nullptr;
    }
    c->bounce = static_cast<uint8_t*>(bounce);
  }
  for (int32_t j = 0; j < n_staging; ++j) {
    if (hipEventCreateWithFlags(&c->stage_ev[j], hipEventDisableTiming) != hipSuccess) {
      moe_cache_destroy(c);
      cache_fail(MOE_EHIP, "hipEventCreateWithFlags failed");
      return nullptr;
    }
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
  const int64_t hits0 = c->hits, misses0 = c->misses;
  std::vector<std::pair<int32_t, Slot>> hit_before;   // for the rollback of a failed call
  // hits first: they are held, so no miss of this call can evict them
  for (int32_t e = 0; e < E; ++e) {
    if (!need[e]) continue;
    const size_t le = static_cast<size_t>(layer) * E + e;
    const int32_t s = c->where[le];
    if (s < 0) continue;
    hit_before.emplace_back(s, c->slots[s]);
    c->hold(s);
    Slot& x = c->slots[s];
    c->count[le] += 1;
    x.uses = c->keep_counts ? c->count[le] : x.uses + 1;
    x.last = now;
    held.push_back(s);
    slot_table_host[e] = static_cast<int64_t>(s) * c->stride;
    ++c->hits;
  }
  // the policy first (slot of every miss), then the copies
  std::vector<MissJob> jobs;
  for (int32_t e = 0; e < E; ++e) {
    const size_t le = static_cast<size_t>(layer) * E + e;
    if (!need[e] || c->where[le] >= 0) continue;
    const int32_t s = std::get<5>(*c->evictable.begin());
    c->hold(s);
    Slot& x = c->slots[s];
    if (x.layer >= 0) {
      c->where[static_cast<size_t>(x.layer) * E + x.id] = -1;
      ++c->evictions;
    }
    jobs.push_back({e, s, x.reader});
    c->count[le] += 1;
    x.layer = layer;
    x.id = e;
    x.uses = c->keep_counts ? c->count[le] : 1;
    x.last = now;
    x.reader = nullptr;
    c->where[le] = s;
    held.push_back(s);
    slot_table_host[e] = static_cast<int64_t>(s) * c->stride;
    ++c->misses;
  }
  int rc = MOE_OK;
  if (c->planning) {
    for (size_t j = 0; j < jobs.size() && rc == MOE_OK; ++j)
      if (take_fault(c)) rc = cache_fail(MOE_EHIP, "injected copy failure");
  } else if (!jobs.empty()) {
    rc = c->store ? copy_from_store(c, layer, jobs, cs) : copy_from_host(c, layer, jobs, cs);
    // copies issued before a failure still run: later copies of this cache
    // stay behind them (issue order), whatever stream they use
    if (hipEventRecord(c->last_copies, cs) == hipSuccess) {
      c->any_copies = true;
      c->last_stream = cs;
    } else if (rc == MOE_OK) {
      rc = cache_fail(MOE_EHIP, "hipEventRecord failed");
    }
  }
  if (rc != MOE_OK) {
    // nothing of this call stays resident: the slots its misses took become
    // empty (keeping the event of their last reader, whom a later copy into
    // them must still wait for), and its holds are dropped
    for (const MissJob& j : jobs) {
      Slot& x = c->slots[j.s];
      c->where[static_cast<size_t>(layer) * E + j.e] = -1;
      c->count[static_cast<size_t>(layer) * E + j.e] -= 1;
      x.layer = -1;
      x.id = -1;
      x.uses = 0;
      x.last = -1;
      x.reader = j.reader;
    }
    for (int32_t e = 0; e < E; ++e)
      if (need[e] && c->where[static_cast<size_t>(layer) * E + e] >= 0)
        c->count[static_cast<size_t>(layer) * E + e] -= 1;
    for (const auto& hb : hit_before) {
      // back to the uses and last use the hit found (its hold is dropped below)
      c->slots[hb.first].uses = hb.second.uses;
      c->slots[hb.first].last = hb.second.last;
    }
    for (int32_t s : held) c->unhold(s);
    c->hits = hits0;
    c->misses = misses0;
    return rc;
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

int moe_cache_set_policy(moe_cache* c, int32_t flags) {
  if (!c || (flags & ~MOE_CACHE_KEEP_COUNTS)) return cache_fail(MOE_EINVAL, "bad cache or policy flags");
  c->keep_counts = (flags & MOE_CACHE_KEEP_COUNTS) != 0;
  return MOE_OK;
}

int moe_cache_inject_fault(moe_cache* c, int32_t nth_copy) {
  if (!c || nth_copy < -1) return cache_fail(MOE_EINVAL, "bad cache or copy index");
  c->fault_at = nth_copy;
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
  // nothing to report from here: destruction has no error path
  if (c->last_copies) (void)hipEventDestroy(c->last_copies);
  for (hipEvent_t ev : c->stage_ev)
    if (ev) (void)hipEventDestroy(ev);
  free(c->bounce);
  delete c;
}

const char* moe_cache_last_error(void) { return g_cache_err; }

}  // extern "C"
