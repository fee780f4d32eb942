// Exchanges between the blocks of the persistent decode kernels (gfx950).
//
// A value goes from one block to others as a tagged 64-bit word (tag << 32 |
// the value's bits), stored with a relaxed device-scope store, so it passes
// the writer's L2, and read with device-scope loads until the word carries the
// expected tag.  Tags only grow from call to call (per-block epoch counters),
// so a word left from an earlier call or layer never matches.  Also the
// direct global -> LDS copies the kernels use for operands they need later.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

typedef __attribute__((address_space(3))) uint32_t lds_w32;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) uint64_t lds_w64;
typedef __attribute__((address_space(3))) int64_t lds_i64;
typedef __attribute__((address_space(3))) uint16_t lds_w16;

__device__ __forceinline__ void store_tag(uint64_t* p, uint32_t bits, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One tagged word, read past this XCD's L2 (device scope).
__device__ __forceinline__ uint64_t load_tag(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tags only grow within a call and from call to call, so "at least" is a
// signed difference (safe across wrap-around).
__device__ __forceinline__ bool tag_ge(uint32_t f, uint32_t tag) { return static_cast<int32_t>(f - tag) >= 0; }

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Direct copies (global -> LDS, 16 or 4 bytes per lane) of `bytes` contiguous
// bytes at byte `src` of the buffer `rs` into `dst`.  Lane l of round j copies
// bytes [j W + l w, + w) (W = 64 w); a round that runs past `bytes` lands in
// the region's padding.
template <int W>
__device__ __forceinline__ void copy_lds(u32x4 rs, uint8_t* dst, uint32_t src, uint32_t bytes, int lane) {
  for (uint32_t j = 0; j < bytes; j += kWave * W)
    lds_load<W>(rs, dst + j, src + j + static_cast<uint32_t>(lane) * W, 0);
}

// Tagged words read by nthr threads: word i (reader rt takes i = rt + q nthr,
// q < PER) at addr(i), read until it carries `tag`; put(i, bits) stores its
// value.  Run by the reading waves only, under a branch on the wave index,
// with no barrier inside: the copy waves, whose direct loads are still in
// flight, must never execute the wait that follows these loads.  False on
// expiry.
template <int PER, typename A, typename F>
__device__ __forceinline__ bool read_tagged(int rt, int n, int nthr, uint32_t tag, uint32_t limit, A&& addr, F&& put) {
  const int tid = rt;
  uint32_t need = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (tid + q * nthr < n) need |= 1u << q;
  for (uint32_t spins = 0;; ++spins) {
    uint64_t w[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) w[q] = (need >> q) & 1u ? load_tag(addr(tid + q * nthr)) : 0ull;
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (((need >> q) & 1u) && static_cast<uint32_t>(w[q] >> 32) == tag) {
        put(tid + q * nthr, static_cast<uint32_t>(w[q]));
        need &= ~(1u << q);
      }
    if (__ballot(need != 0u) == 0) return true;
    if (spins >= limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

}  // namespace moe
