// Device helpers shared by the MoE-layer kernels (gfx950, wave64).
//
// Numerics contract used by every kernel, so that different launch shapes of
// the same step give the same bits:
//   * A "segment" is 32 consecutive codes of one matrix row: 16 bytes of int4
//     (four little-endian words, low nibble first) or 32 bytes of int8.  A
//     group of 64 codes is two segments, so one segment has one scale/bias.
//   * Segment value = fmaf(s, qx, b * xs), where qx = sum_c q_c v_c is formed
//     as two float32 FMA chains (even and odd codes, each in code order) added
//     at the end, and xs = sum_c v_c is a float32 add chain in code order.
//     This is w.v with w = s q + b regrouped per group (affine dequantisation,
//     Swiftlet README translation, "Relation to TurboFieldfare").
//   * A row's segments are summed per lane in segment order, then across the
//     lanes of the row with symmetric pairwise steps (group_sum), which leave
//     the bitwise same total on every lane of the row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum : int { kF32 = 0, kBF16 = 1 };

constexpr int kWave = 64;
constexpr int kSegCodes = 32;

// Error flag bits kept in the workspace control words.
constexpr uint32_t kErrRange = 1u;     // bad slot offset or expert id; pair skipped
constexpr uint32_t kErrTimeout = 2u;   // a bounded in-kernel wait expired
constexpr uint32_t kErrF16 = 4u;       // prefill: a value rounded to float16 left its range (inf or NaN)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* base, size_t idx) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(base)[idx];
  } else {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  }
}

// Raw bits of one scale/bias value (float32 bits, or bf16 bits in the low
// half), converted only where used: a conversion right after the load would
// make the compiler wait for it there, serialising loads meant to overlap.
template <int DT>
__device__ __forceinline__ uint32_t load_raw(const void* base, size_t idx) {
  if constexpr (DT == kF32) {
    return static_cast<const uint32_t*>(base)[idx];
  } else {
    return static_cast<const uint16_t*>(base)[idx];
  }
}

template <int DT>
__device__ __forceinline__ float raw_value(uint32_t raw) {
  if constexpr (DT == kF32) {
    return __uint_as_float(raw);
  } else {
    return __uint_as_float(raw << 16);
  }
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *static_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}

// 32 activation values of one segment -> float registers.
template <int ACT>
using ActRaw = u32x4[ACT == kF32 ? 8 : 4];

// The raw 16-byte words of one 32-value activation segment; act_raw_f32
// converts them.  Split so that callers can request several segments before
// waiting for any.
template <int ACT>
__device__ __forceinline__ void load_act_raw(const void* row, int seg, ActRaw<ACT>& w) {
  const u32x4* p = ACT == kF32
                       ? reinterpret_cast<const u32x4*>(static_cast<const float*>(row) + seg * kSegCodes)
                       : reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + seg * kSegCodes);
#pragma unroll
  for (int i = 0; i < (ACT == kF32 ? 8 : 4); ++i) w[i] = p[i];
}

template <int ACT>
__device__ __forceinline__ void act_raw_f32(const ActRaw<ACT>& w, float (&v)[kSegCodes]) {
  if constexpr (ACT == kF32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[4 * i + 0] = __uint_as_float(w[i][0]);
      v[4 * i + 1] = __uint_as_float(w[i][1]);
      v[4 * i + 2] = __uint_as_float(w[i][2]);
      v[4 * i + 3] = __uint_as_float(w[i][3]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j + 0] = __uint_as_float(w[i][j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[i][j] & 0xffff0000u);
      }
    }
  }
}

template <int ACT>
__device__ __forceinline__ void load_act_seg(const void* row, int seg, float (&v)[kSegCodes]) {
  ActRaw<ACT> w;
  load_act_raw<ACT>(row, seg, w);
  act_raw_f32<ACT>(w, v);
}

// 32 float32 values (e.g. an h segment) from global memory.
__device__ __forceinline__ void load_f32_seg(const float* row, int seg, float (&v)[kSegCodes]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row + seg * kSegCodes);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 w = p[i];
    v[4 * i + 0] = __uint_as_float(w[0]);
    v[4 * i + 1] = __uint_as_float(w[1]);
    v[4 * i + 2] = __uint_as_float(w[2]);
    v[4 * i + 3] = __uint_as_float(w[3]);
  }
}

typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Direct (global -> LDS) buffer loads written as inline assembly.  Issued
// through the compiler's intrinsic, a direct load into one LDS stage makes
// the compiler wait for it before LDS reads it cannot prove to be of the other
// stage, which serialises the pipeline; the assembly form is invisible to it,
// and the kernels wait for their direct loads themselves (s_waitcnt 0, then a
// barrier when other waves read the copied bytes).  Lane l's bytes land at
// lds + BYTES * l.  M0 (the LDS base of the copy) is saved and restored around
// the load, and one wait state separates its write from the load.  The
// descriptor is the plain four-word form over [base, base + bytes); a load
// past its end reads zeros.
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const auto uni = [](uint32_t v) { return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(v)); };
  return u32x4{uni(static_cast<uint32_t>(b)), uni(static_cast<uint32_t>(b >> 32) & 0xffffu),
               uni(static_cast<uint32_t>(bytes)), 0x00020000u};
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <int BYTES>
__device__ __forceinline__ void lds_load(u32x4 rs, uint8_t* lds, uint32_t voff, int soff) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte direct loads");
  const uint32_t la = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)lds)));
  const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(soff));
  uint32_t saved;
  if constexpr (BYTES == 16)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(la), "v"(voff), "s"(rs), "s"(so)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(la), "v"(voff), "s"(rs), "s"(so)
        : "memory");
}


// 32 floats of one segment from LDS (p points into shared memory; the cast
// makes the compiler use LDS instructions rather than generic ones).
__device__ __forceinline__ void load_lds_seg(const float* p, int seg, float (&v)[kSegCodes]) {
  const lds_u32x4* q = reinterpret_cast<const lds_u32x4*>((const lds_f32*)(p) + seg * kSegCodes);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 w = q[i];
    v[4 * i + 0] = __uint_as_float(w[0]);
    v[4 * i + 1] = __uint_as_float(w[1]);
    v[4 * i + 2] = __uint_as_float(w[2]);
    v[4 * i + 3] = __uint_as_float(w[3]);
  }
}

__device__ __forceinline__ float seg_sum(const float (&v)[kSegCodes]) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kSegCodes; ++c) s += v[c];
  return s;
}

// Packed codes of one segment: one u32x4 for int4, two for int8.
template <int BITS>
struct Seg {
  u32x4 w[BITS / 4];
};

template <int BITS>
__device__ __forceinline__ Seg<BITS> load_codes(const uint8_t* p) {
  Seg<BITS> s;
#pragma unroll
  for (int i = 0; i < BITS / 4; ++i) s.w[i] = load16_stream(p + 16 * i);
  return s;
}

// The same loads through an address known to be global memory (a pointer
// rebuilt from integers, e.g. after readfirstlane, is otherwise generic and
// compiles to FLAT loads, which also count against the LDS wait counter).
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) const uint32_t g_u32;
typedef __attribute__((address_space(1))) const uint16_t g_u16;

template <int BITS>
__device__ __forceinline__ Seg<BITS> load_codes_g(uint64_t addr) {
  Seg<BITS> s;
#pragma unroll
  for (int i = 0; i < BITS / 4; ++i) s.w[i] = __builtin_nontemporal_load(reinterpret_cast<g_u32x4*>(addr + 16 * i));
  return s;
}

template <int DT>
__device__ __forceinline__ uint32_t load_raw_g(uint64_t addr) {
  if constexpr (DT == kF32) return *reinterpret_cast<g_u32*>(addr);
  else return *reinterpret_cast<g_u16*>(addr);
}

__device__ __forceinline__ float seg_value(float s, float b, float qx, float xs) {
  return fmaf(s, qx, b * xs);
}

// DPP move of a float within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// v + v of lane l ^ D for D = 16 or 32, on gfx950's v_permlane16/32_swap: with
// both operands holding v, the swap leaves the two addends of every lane in
// the two results (no LDS round trip, unlike a bpermute).
template <int D>
__device__ __forceinline__ float swap_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (D == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

// Sum over aligned groups of `width` lanes (power of two <= 64).  Each step
// adds the value of a partner lane that adds ours back (mirror within 16,
// mirror within 8, reversal within 4, swap of neighbours; then xor 16, 32),
// so every lane of a group ends with the bitwise same total.  The first four
// steps are DPP moves and the last two lane swaps, so no step takes an LDS
// round trip.
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 16) v += dpp_f32<0x140>(v);   // row_mirror
  if (width >= 8) v += dpp_f32<0x141>(v);    // row_half_mirror
  if (width >= 4) v += dpp_f32<0x1B>(v);     // quad_perm [3, 2, 1, 0]
  if (width >= 2) v += dpp_f32<0xB1>(v);     // quad_perm [1, 0, 3, 2]
  if (width >= 32) v = swap_sum<16>(v);
  if (width >= 64) v = swap_sum<32>(v);
  return v;
}

// group_sum for a width known at compile time: the same steps in the same
// order, without the run-time tests.
template <int W>
__device__ __forceinline__ float group_sum_w(float v) {
  if constexpr (W >= 16) v += dpp_f32<0x140>(v);
  if constexpr (W >= 8) v += dpp_f32<0x141>(v);
  if constexpr (W >= 4) v += dpp_f32<0x1B>(v);
  if constexpr (W >= 2) v += dpp_f32<0xB1>(v);
  if constexpr (W >= 32) v = swap_sum<16>(v);
  if constexpr (W >= 64) v = swap_sum<32>(v);
  return v;
}

// Gate and up row sums of one row at once.  Full-wave rows (width 64): one
// lane swap leaves gate pairs in lanes 0-31 and up pairs in lanes 32-63, the
// rest of the reduction runs within each half, and lanes 0 and 32 hand the
// totals to the whole wave.  Narrower rows: two group_sums.  Every lane ends
// with its row's totals.
template <int W>
__device__ __forceinline__ void gu_sums_w(float accg, float accu, int width, float& g, float& u) {
  if (W == kWave || (W == 0 && width == kWave)) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(accg), __float_as_uint(accu), false, false);
    const float v = group_sum_w<32>(__uint_as_float(r[0]) + __uint_as_float(r[1]));
    g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));   // the builtin takes int: move bits
    u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  } else if constexpr (W == 0) {
    g = group_sum(accg, width);
    u = group_sum(accu, width);
  } else {
    g = group_sum_w<W>(accg);
    u = group_sum_w<W>(accu);
  }
}

__device__ __forceinline__ void gu_sums(float accg, float accu, int width, float& g, float& u) {
  gu_sums_w<0>(accg, accu, width, g, u);
}

// silu(a) = a / (1 + e^-a) on the hardware exp and reciprocal (about one ulp each).
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

__device__ __forceinline__ float sigmoid(float a) { return 1.0f / (1.0f + expf(-a)); }

__device__ __forceinline__ void raise_error(uint32_t* flags, uint32_t bit) {
  __hip_atomic_fetch_or(flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A blob offset is usable if it is non-negative, 256-byte aligned and the
// whole blob fits in the pool.
__device__ __forceinline__ bool slot_ok(int64_t off, int64_t blob_bytes, int64_t pool_bytes) {
  return off >= 0 && (off & 255) == 0 && off <= pool_bytes - blob_bytes;
}

// Passes of row_lanes rows a wave takes per task in the GEMV kernels.
constexpr int kMaxPass = 4;

// ---------------------------------------------------------------------------
// Lane layout for a row of `cols` codes split into 32-code segments:
// spr = cols / 32 segments per row.  If spr >= 64 one wave covers one row and
// lane L takes segments L, L + 64, ... (nsl = spr / 64 of them).  Otherwise a
// wave covers 64 / spr rows at once and lane L takes segment L % spr of row
// L / spr.
struct RowLanes {
  int spr;      // segments per row
  int rpp;      // rows per wave pass
  int width;    // lanes summed per row
  int sub_row;  // this lane's row within a pass
  int seg0;     // this lane's first segment
};

// cols is a power of two >= 64 (the descriptor checks enforce it), so the
// divisions reduce to shifts and masks.
__device__ __forceinline__ RowLanes row_lanes(int cols, int lane) {
  RowLanes r;
  const int sh = __builtin_ctz(static_cast<unsigned>(cols)) - 5;   // log2(cols / kSegCodes)
  r.spr = 1 << sh;
  if (r.spr >= kWave) {
    r.rpp = 1;
    r.width = kWave;
    r.sub_row = 0;
    r.seg0 = lane;
  } else {
    r.rpp = kWave >> sh;
    r.width = r.spr;
    r.sub_row = lane >> sh;
    r.seg0 = lane & (r.spr - 1);
  }
  return r;
}

// Multi-token segment dot: converts each code once and feeds NT FMA chains per
// parity; per token the result is bitwise the single-token seg_qdot.
template <int BITS, int NT>
__device__ __forceinline__ void seg_qdot_nt(const Seg<BITS>& s_in, const float (&v)[NT][kSegCodes], float (&out)[NT]) {
  // Opaque copy of the packed codes: keeps the compiler from hoisting the
  // code->float conversions out of the callers' token loops, which would hold
  // 32 floats per segment in registers instead of 4 words.
  Seg<BITS> s;
#pragma unroll
  for (int i = 0; i < BITS / 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = s_in.w[i][j];
      asm volatile("" : "+v"(w));
      s.w[i][j] = w;
    }
  }
  float a0[NT], a1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) { a0[t] = 0.f; a1[t] = 0.f; }
  if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = s.w[0][k];
      uint32_t lo = w & 0x0f0f0f0fu;
      uint32_t hi = (w >> 4) & 0x0f0f0f0fu;
      // opaque masked words: the byte conversions below then map to single
      // v_cvt_f32_ubyte{0..3} instead of a bit-field extract plus a conversion
      asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float qe = static_cast<float>((lo >> (8 * j)) & 0xffu);
        const float qo = static_cast<float>((hi >> (8 * j)) & 0xffu);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          a0[t] = fmaf(qe, v[t][8 * k + 2 * j], a0[t]);
          a1[t] = fmaf(qo, v[t][8 * k + 2 * j + 1], a1[t]);
        }
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = s.w[h][k];
        const float q0 = static_cast<float>(w & 0xffu);
        const float q1 = static_cast<float>((w >> 8) & 0xffu);
        const float q2 = static_cast<float>((w >> 16) & 0xffu);
        const float q3 = static_cast<float>(w >> 24);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          a0[t] = fmaf(q0, v[t][16 * h + 4 * k + 0], a0[t]);
          a1[t] = fmaf(q1, v[t][16 * h + 4 * k + 1], a1[t]);
          a0[t] = fmaf(q2, v[t][16 * h + 4 * k + 2], a0[t]);
          a1[t] = fmaf(q3, v[t][16 * h + 4 * k + 3], a1[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) out[t] = a0[t] + a1[t];
}

// bf16 activations with int4 codes: the segment dot on v_dot2_f32_bf16.
// Each code q becomes the bf16 value 128 + q (exact: 128 + q < 256 needs 8
// significant bits), pairs (q_2j, q_2j+1) side by side as the raw activation
// words hold (x_2j, x_2j+1).  One instruction then adds two products, both
// exact in float32, and  D = sum (128 + q) x,  so  sum q x = D - 128 sum x.
struct QPairs {
  uint32_t p[16];
};

__device__ __forceinline__ QPairs qpairs_bf16(const Seg<4>& s_in) {
  constexpr uint32_t kHi = 0x43434343u;   // 0x43 is the high byte of bf16 128.0
  QPairs o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w = s_in.w[0][k];
    asm volatile("" : "+v"(w));           // keep the conversion where the caller uses it
    const uint32_t lo = w & 0x0f0f0f0fu;          // bytes: q0 q2 q4 q6
    const uint32_t hi = (w >> 4) & 0x0f0f0f0fu;   // bytes: q1 q3 q5 q7
    const uint32_t t0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // q0 q1 q2 q3
    const uint32_t t1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // q4 q5 q6 q7
    o.p[4 * k + 0] = __builtin_amdgcn_perm(kHi, t0, 0x04010400u);     // (128 + q0, 128 + q1)
    o.p[4 * k + 1] = __builtin_amdgcn_perm(kHi, t0, 0x04030402u);     // (128 + q2, 128 + q3)
    o.p[4 * k + 2] = __builtin_amdgcn_perm(kHi, t1, 0x04010400u);
    o.p[4 * k + 3] = __builtin_amdgcn_perm(kHi, t1, 0x04030402u);
  }
  return o;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// D = sum over the segment of (128 + q) x, two chains of eight.
__device__ __forceinline__ float dot2_seg(const QPairs& q, const ActRaw<kBF16>& x) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0 = dot2_bf16(q.p[4 * i + 0], x[i][0], a0);
    a1 = dot2_bf16(q.p[4 * i + 1], x[i][1], a1);
    a0 = dot2_bf16(q.p[4 * i + 2], x[i][2], a0);
    a1 = dot2_bf16(q.p[4 * i + 3], x[i][3], a1);
  }
  return a0 + a1;
}

// sum x of a raw bf16 segment, on the same instruction (pairs times (1, 1)).
__device__ __forceinline__ float xsum_bf16(const ActRaw<kBF16>& x) {
  constexpr uint32_t kOnes = 0x3f803f80u;
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0 = dot2_bf16(kOnes, x[i][0], a0);
    a1 = dot2_bf16(kOnes, x[i][1], a1);
    a0 = dot2_bf16(kOnes, x[i][2], a0);
    a1 = dot2_bf16(kOnes, x[i][3], a1);
  }
  return a0 + a1;
}

// One segment's affine contribution s sum q x + b sum x from D and sum x.
__device__ __forceinline__ float seg_value_d2(float s, float b, float d, float xs) {
  return seg_value(s, b, d - 128.f * xs, xs);
}

// Raw bf16 segment of an activation row held in LDS.
__device__ __forceinline__ void load_lds_act_bf16(const uint8_t* row, int seg, ActRaw<kBF16>& w) {
  const lds_u32x4* p = reinterpret_cast<const lds_u32x4*>((const __attribute__((address_space(3))) uint8_t*)(row) +
                                                          seg * kSegCodes * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = p[i];
}

// Blob plane offsets (see include/moe_layer.h): Q bytes of codes and S bytes
// of scales per matrix, all three matrices the same size.
struct Planes {
  int64_t q;   // codes bytes of one matrix
  int64_t s;   // scale bytes of one matrix
  int64_t blob;
};

__host__ __device__ inline Planes planes_of(int hidden, int inter, int bits, int sb_dtype) {
  Planes p;
  p.q = static_cast<int64_t>(hidden) * inter * bits / 8;
  p.s = static_cast<int64_t>(hidden) * (inter / 64) * (sb_dtype == kF32 ? 4 : 2);
  p.blob = 3 * p.q + 6 * p.s;
  return p;
}

}  // namespace moe
