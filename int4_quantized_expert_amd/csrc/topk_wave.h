// Top-k selection of one token's router logits on one wave (gfx950, wave64).
//
// Ranks the experts by (logit descending, id ascending), so ties go to the
// lower id, and forms the renormalised weights p_i = exp(l_i - l_0) /
// sum_j exp(l_j - l_0) over the chosen logits in rank order.  Reading of the
// pages: the router picks the top k of E experts per token (Swiftlet README
// translation, "How it works"); the weights are the softmax over all experts
// renormalised over the chosen ones, whose full denominator cancels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace moe {

constexpr int kCandMax = 64;   // candidates ranked exactly before the fallback

// Monotone map from float to uint32 order keys (larger float, larger key);
// +0 and -0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) == 0) return 0x80000000u;          // +0 and -0 rank equal
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The float behind an order key (both zeros come back as +0, which leaves
// every difference taken with it unchanged; a NaN comes back as a NaN).
__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ uint64_t lane_mask_lt(int lane) { return lane == 0 ? 0ull : (~0ull >> (64 - lane)); }

// The value of lane (lane ^ S) within the wave, by lane moves (DPP, a
// swizzle, lane swaps) rather than an LDS round trip.
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v, int lane) {
  if constexpr (S == 1) {
    return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, false);   // quad_perm [1, 0, 3, 2]
  } else if constexpr (S == 2) {
    return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, false);   // quad_perm [2, 3, 0, 1]
  } else if constexpr (S == 4) {
    return __builtin_amdgcn_ds_swizzle(v, 0x1F | (4 << 10));     // bit mode, xor 4
  } else if constexpr (S == 8) {
    return __builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, false);  // row_ror:8 (xor 8 within a row)
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// Largest 64-bit word over the wave; every lane ends with it.
template <int S>
__device__ __forceinline__ uint64_t max_step(uint64_t c, int lane) {
  const uint64_t p = (static_cast<uint64_t>(lane_xor<S>(static_cast<uint32_t>(c >> 32), lane)) << 32) |
                     lane_xor<S>(static_cast<uint32_t>(c), lane);
  return p > c ? p : c;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t c, int lane) {
  c = max_step<1>(c, lane);
  c = max_step<2>(c, lane);
  c = max_step<4>(c, lane);
  c = max_step<8>(c, lane);
  c = max_step<16>(c, lane);
  return max_step<32>(c, lane);
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Top-k of one token on one wave.
//  1. A threshold from the per-lane maxima: the k-th largest lane maximum,
//     found on the top 14 bits of the order key two bits a step (three
//     independent ballots per step), is a lower bound of the k-th largest
//     logit, so every top-k logit is at or above it.
//  2. The candidates at or above it (usually a few more than k) are packed as
//     64-bit (key << 32 | ~id) words, so that "larger word" means "larger
//     logit, then lower id", and ranked exactly against each other.  The
//     ranks of the candidates and the indices of the other lanes form a
//     permutation of the lanes, so one lane permute hands rank r's logit and
//     id to lane r without a trip through LDS memory.
//  3. If more than kCandMax candidates qualify, k rounds of a wave arg-max
//     finish the job.
// Output: ids[0..k) and vals[0..k) = renormalised weights p_i, formed with the
// same operations and order as the staged kernel; lane r < k also returns the
// id of rank r.  lg, cand, ids and vals must be in LDS.  NJ = logits per lane
// (E <= 64 NJ); the code is straight-line over NJ so that every load and
// ballot is issued without waiting.
template <int NJ>
__device__ __forceinline__ int topk_wave_n(const float* lg_, int E, int k, int lane, uint64_t* cand_, int32_t* ids_,
                                           float* vals_) {
  const lds_f32* lg = (const lds_f32*)(lg_);
  typedef __attribute__((address_space(3))) uint64_t lds_u64;
  typedef __attribute__((address_space(3))) int32_t lds_i32;
  typedef __attribute__((address_space(3))) u32x4 lds_v4;
  lds_u64* cand = (lds_u64*)(cand_);
  lds_i32* ids = (lds_i32*)(ids_);
  lds_f32* vals = (lds_f32*)(vals_);
  float raw[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + j * kWave;
    raw[j] = lg[e < E ? e : 0];
  }
  uint32_t key[NJ];
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + j * kWave;
    const uint32_t kv = order_key(raw[j]);
    key[j] = e < E ? (kv > 1u ? kv : 1u) : 0u;   // every real entry ranks above "no entry"
    lm = key[j] > lm ? key[j] : lm;
  }
  // the largest theta (top 14 bits: sign, exponent and five mantissa bits,
  // candidates within about 3% of the bound) with at least k lane maxima at or above
  // it; a step settles two bits from the counts at three thresholds
  uint32_t theta = 0;
#pragma unroll
  for (int b = 30; b >= 18; b -= 2) {
    const uint32_t c1 = theta | (1u << b), c2 = theta | (2u << b), c3 = theta | (3u << b);
    const unsigned n1 = __popcll(__ballot(lm >= c1)), n2 = __popcll(__ballot(lm >= c2)),
                   n3 = __popcll(__ballot(lm >= c3));
    const unsigned kk = static_cast<unsigned>(k);
    theta = n3 >= kk ? c3 : n2 >= kk ? c2 : n1 >= kk ? c1 : theta;
  }
  // padding first (a wave's LDS writes land in program order, so the
  // candidates overwrite it): padding never outranks a candidate
  cand[lane] = 0ull;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool in = key[j] != 0u && key[j] >= theta;
    const uint64_t m = __ballot(in);
    const int pos = cnt + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
    const int id = lane + j * kWave;
    if (in && pos < kCandMax) cand[pos] = (static_cast<uint64_t>(key[j]) << 32) | static_cast<uint32_t>(~id);
    cnt += __popcll(m);
  }
  float v = 0.f;   // lane r < k: rank r's logit
  int myid = 0;    // lane r < k: rank r's id
  if (cnt <= kCandMax) {
    wave_sync_lds();
    const uint64_t mine = cand[lane];
    const lds_v4* c4 = (const lds_v4*)(cand);
    int rank = 0;
    // sixteen candidates per round, all eight reads requested together
    for (int d0 = 0; d0 < cnt; d0 += 16) {
      u32x4 q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = c4[d0 / 2 + i];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint64_t w0 = (static_cast<uint64_t>(q[i][1]) << 32) | q[i][0];
        const uint64_t w1 = (static_cast<uint64_t>(q[i][3]) << 32) | q[i][2];
        rank += (w0 > mine) ? 1 : 0;
        rank += (w1 > mine) ? 1 : 0;
      }
    }
    // candidates go to lane `rank` (ranks 0..cnt-1 are distinct), the other
    // lanes to themselves: a permutation of the lanes
    const bool cd = lane < cnt;
    const int id = static_cast<int>(~static_cast<uint32_t>(mine));
    float val = 0.f;
    if (cd && rank < k) {
      ids[rank] = id;
      val = key_float(static_cast<uint32_t>(mine >> 32));   // the logit, from its key
    }
    const int dst = 4 * (cd ? rank : lane);
    v = __int_as_float(__builtin_amdgcn_ds_permute(dst, __float_as_int(val)));
    myid = __builtin_amdgcn_ds_permute(dst, id);
  } else {
    // rare: more than kCandMax entries lie at or above the bound (many equal
    // logits, e.g. a zero input, where every logit is 0).  k rounds of a wave
    // arg-max over the unique words (key << 32 | ~id): larger key first, then
    // lower id; each round's maximum travels by lane moves, not through LDS.
    uint32_t taken = 0;
    for (int i = 0; i < k; ++i) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int e = lane + j * kWave;
        const uint64_t c = ((taken >> j) & 1u) || key[j] == 0u
                               ? 0ull
                               : (static_cast<uint64_t>(key[j]) << 32) | static_cast<uint32_t>(~e);
        best = c > best ? c : best;
      }
      best = wave_max_u64(best, lane);
      const int bid = static_cast<int>(~static_cast<uint32_t>(best));
      if ((bid & (kWave - 1)) == lane) taken |= 1u << (bid / kWave);
      if (lane == 0) ids[i] = bid;
      if (lane == i) myid = bid;
    }
    v = lg[lane < k ? myid : 0];
  }
  // p_i = exp(l_i - l_0) / sum_j exp(l_j - l_0), the sum in rank order from 0
  const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float ex = lane < k ? expf(v - top) : 0.f;
  float sum = 0.f;
  if (k <= 16) {
    // fixed lanes, no branches: lanes k..15 hold +0, and adding +0 to a sum
    // of non-negative terms leaves it unchanged, so the sum is the one in
    // rank order; the reads are independent, only the adds are chained
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), i));
  } else {
    for (int i = 0; i < k; ++i) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), i));
  }
  if (lane < k) vals[lane] = ex / sum;
  return myid;
}

__device__ __forceinline__ void topk_wave(const float* lg, int E, int k, int lane, uint64_t* cand, int32_t* ids,
                                          float* vals) {
  if (E <= 8 * kWave)
    topk_wave_n<8>(lg, E, k, lane, cand, ids, vals);
  else
    topk_wave_n<16>(lg, E, k, lane, cand, ids, vals);
}

}  // namespace moe
