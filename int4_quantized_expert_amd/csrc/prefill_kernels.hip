// Prefill path: one MoE layer over many tokens at once (gfx950).
//
// The pages' method is the same as in decode -- softmax router, top-k, expert
// SwiGLU with MLX-affine group-quantized weights, a weighted combine plus a
// sigmoid-gated shared expert (Swiftlet README translation, "How it works";
// linlog.top article, "Why MoE can stream") -- but with ~40 tokens per expert
// the expert products become small dense GEMMs, so they run on MFMA:
//
//   k_pf_router    logits = x R^T on v_mfma_f32_16x16x32_bf16 (exact bf16
//                  products, fp32 accumulation)
//   (k_topk)       the staged path's per-token top-k and renormalisation
//   k_pf_dispatch  each pair's place in its expert's list, the list starts
//                  and a table of tiles of up to 64 pairs of one expert
//   k_pf_xprep     x to float16, stored in the k order the MFMA operands use;
//                  also writes the pair lists
//   k_pf_gateup    per tile: h = silu(Wg x) * (Wu x), h in float16
//   k_pf_down      per tile: partial = Wd h, fp32 sums stored as float16 per
//                  (pair, output row)
//   (k_combine)    the staged path's ordered combine with the shared expert
//
// Expert weights are dequantized straight into MFMA A operands: each int4/int8
// code becomes 1024 + q in float16 by OR-ing it into the mantissa of 1024
// (exact), 1024 is subtracted (exact) and w = s * q + b is formed by one
// float16 FMA, i.e. rounded once.  Activations (bf16 inputs, exact in float16
// within its range) and h are float16; every product accumulates in fp32.
//
// MFMA 16x16x32 operand layout (gfx950): lane l supplies row/column l % 16 and
// eight k values 8 (l / 16) .. +7 of A and B; D row 4 (l / 16) + i, column
// l % 16 lands in lane l, element i.  The sum over k does not care which k a
// slot stands for, as long as A and B agree, so within each 128-wide step of k
// lane quarter q takes k = 32 q .. 32 q + 31 (contiguous bytes per lane) and
// within each 8 codes the slot order is the one the dequantization produces.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {
namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk = kPrefillChunk;   // pairs per tile (4 MFMA column blocks)
constexpr int kGuRows = 128;            // gate/up rows (each) per block: 4 waves x 32
constexpr int kDnRows = 256;            // down rows per row block: 4 waves x 64
constexpr int kDownGroup = 2;           // row blocks per down block (int4, bf16 scales)
constexpr int kSlice = 256;             // k staged in LDS per step
constexpr int kDispThreads = 1024;
constexpr int kDispBatch = 8;           // dispatch: id loads in flight per lane

__device__ __forceinline__ uint32_t h2_bits(h2v v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h2v bits_h2(uint32_t v) { return __builtin_bit_cast(h2v, v); }

// Slot order of 8 consecutive k inside one MFMA operand, as produced by the
// dequantization: int4 words give pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7); int8
// words give (k0,k2) (k1,k3) (k4,k6) (k5,k7).  permute8 puts float16
// activations in the same order.

// Position of the 16-byte chunk holding natural 8-group g8 (k = 8 g8 ..) in
// the MFMA k order: inside each 128-wide step (16 groups), group 4 q + j goes
// to 4 j + q, so lane quarter q reads chunk 4 j + q for MFMA step j.
__device__ __forceinline__ int chunk_of(int g8) { return (g8 & ~15) | ((g8 & 3) << 2) | ((g8 >> 2) & 3); }

// Eight float16 values in natural k order -> slot order.
template <int BITS>
__device__ __forceinline__ u32x4 permute8(u32x4 v) {
  const uint32_t a = v[0], b = v[1], c = v[2], d = v[3];   // (k0,k1) (k2,k3) (k4,k5) (k6,k7)
  u32x4 o;
  if constexpr (BITS == 4) {
    o[0] = (a & 0xffffu) | (c << 16);            // (k0, k4)
    o[1] = (a >> 16) | (c & 0xffff0000u);        // (k1, k5)
    o[2] = (b & 0xffffu) | (d << 16);            // (k2, k6)
    o[3] = (b >> 16) | (d & 0xffff0000u);        // (k3, k7)
  } else {
    o[0] = (a & 0xffffu) | (b << 16);            // (k0, k2)
    o[1] = (a >> 16) | (b & 0xffff0000u);        // (k1, k3)
    o[2] = (c & 0xffffu) | (d << 16);            // (k4, k6)
    o[3] = (c >> 16) | (d & 0xffff0000u);        // (k5, k7)
  }
  return o;
}

// (w & mask) | magic in one v_and_or_b32.  gfx9 VOP3 instructions read at
// most one scalar or literal operand, so the compiler splits the expression
// into two instructions when both constants are literals; here the mask is a
// scalar and the magic number comes from a vector register.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic_v) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(w), "s"(mask), "v"(magic_v));
  return d;
}

// Dequantize 8 int4 codes (one word, low nibble first) into an A operand.
// magic_v holds 0x64006400 (float16 1024 in both halves).
__device__ __forceinline__ h8v dq_int4(uint32_t w, h2v s, h2v b, uint32_t magic_v) {
  const uint32_t hi = w >> 8;
  const h2v m1024 = {-1024.0f16, -1024.0f16}, r16 = {0.0625f16, 0.0625f16}, m64 = {-64.0f16, -64.0f16};
  const h2v q0 = bits_h2(and_or(w, 0x000F000Fu, magic_v)) + m1024;                          // (q0, q4)
  const h2v q1 = __builtin_elementwise_fma(bits_h2(and_or(w, 0x00F000F0u, magic_v)), r16, m64);   // (q1, q5)
  const h2v q2 = bits_h2(and_or(hi, 0x000F000Fu, magic_v)) + m1024;                         // (q2, q6)
  const h2v q3 = __builtin_elementwise_fma(bits_h2(and_or(hi, 0x00F000F0u, magic_v)), r16, m64);  // (q3, q7)
  u32x4 o;
  o[0] = h2_bits(__builtin_elementwise_fma(q0, s, b));
  o[1] = h2_bits(__builtin_elementwise_fma(q1, s, b));
  o[2] = h2_bits(__builtin_elementwise_fma(q2, s, b));
  o[3] = h2_bits(__builtin_elementwise_fma(q3, s, b));
  return __builtin_bit_cast(h8v, o);
}

// Dequantize 8 int8 codes (two words, low byte first) into an A operand.
__device__ __forceinline__ h8v dq_int8(uint32_t w0, uint32_t w1, h2v s, h2v b, uint32_t magic_v) {
  const h2v m1024 = {-1024.0f16, -1024.0f16};
  const h2v q0 = bits_h2(and_or(w0, 0x00FF00FFu, magic_v)) + m1024;          // (q0, q2)
  const h2v q1 = bits_h2(and_or(w0 >> 8, 0x00FF00FFu, magic_v)) + m1024;     // (q1, q3)
  const h2v q2 = bits_h2(and_or(w1, 0x00FF00FFu, magic_v)) + m1024;          // (q4, q6)
  const h2v q3 = bits_h2(and_or(w1 >> 8, 0x00FF00FFu, magic_v)) + m1024;     // (q5, q7)
  u32x4 o;
  o[0] = h2_bits(__builtin_elementwise_fma(q0, s, b));
  o[1] = h2_bits(__builtin_elementwise_fma(q1, s, b));
  o[2] = h2_bits(__builtin_elementwise_fma(q2, s, b));
  o[3] = h2_bits(__builtin_elementwise_fma(q3, s, b));
  return __builtin_bit_cast(h8v, o);
}

// True if either float16 half of w is inf or NaN (exponent all ones): a value
// rounded to float16 here left the range the prefill path needs.
__device__ __forceinline__ bool f16_bad(uint32_t w) {
  return (w & 0x7c00u) == 0x7c00u || (w & 0x7c000000u) == 0x7c000000u;
}

__device__ __forceinline__ f4v mfma16(h8v a, h8v b, f4v c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// ---------------------------------------------------------------------------
// Shared-expert gate sigmoid(g . x_t) of token t, on one wave, fp32 (the
// staged path's order: a segment's FMA chain per lane, then the wave sum).
__device__ __forceinline__ void pf_gate_token(const void* __restrict__ x, const void* __restrict__ gvec,
                                              float* __restrict__ gate, int t, int H, int lane) {
  const uint8_t* xr = static_cast<const uint8_t*>(x) + static_cast<size_t>(t) * H * 2;
  float acc = 0.f;
  for (int sg = lane; sg < H / kSegCodes; sg += kWave) {
    float a[kSegCodes], g[kSegCodes];
    load_act_seg<kBF16>(xr, sg, a);
    load_act_seg<kBF16>(gvec, sg, g);
#pragma unroll
    for (int c = 0; c < kSegCodes; ++c) acc = fmaf(a[c], g[c], acc);
  }
  acc = group_sum(acc, kWave);
  if (lane == 0) gate[t] = sigmoid(acc);
}

// ---------------------------------------------------------------------------
// Pair lists by expert, pass 1 (one block).  Each pair takes the next place in
// its expert's list with an LDS atomic increment (places follow the order the
// increments land in; no value depends on it, since every pair's columns and
// output rows are its own).  A scan of the counts gives each expert's list
// start; the distinct experts (ascending id), their list starts and the tile
// table follow: expert rank u gets ceil(n_u / 64) tiles, then the shared
// expert ceil(T / 64) tiles of consecutive tokens.  Pass 2 (in k_pf_xprep,
// spread over the grid) writes every pair at its expert's start plus its
// place.
__global__ __launch_bounds__(kDispThreads) void k_pf_dispatch(const int32_t* __restrict__ ids, int T, int k, int E,
                                                             int32_t* __restrict__ erank, int32_t* __restrict__ estart,
                                                             int32_t* __restrict__ ucount, int32_t* __restrict__ uniq,
                                                             int32_t* __restrict__ ustart, int32_t* __restrict__ tstart,
                                                             int32_t* __restrict__ tile_u, int32_t* __restrict__ meta,
                                                             uint32_t* __restrict__ flags) {
  __shared__ int cnt[kDispThreads];
  __shared__ int ws_c[kDispThreads / kWave], ws_u[kDispThreads / kWave], ws_t[kDispThreads / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int np = T * k;
  cnt[tid] = 0;
  __syncthreads();
  // kDispBatch pairs per thread in flight: all loads before any use
  for (int b0 = 0; b0 < np; b0 += kDispBatch * kDispThreads) {
    int ev[kDispBatch];
#pragma unroll
    for (int v = 0; v < kDispBatch; ++v) {
      const int p = b0 + v * kDispThreads + tid;
      ev[v] = ids[p < np ? p : 0];
    }
#pragma unroll
    for (int v = 0; v < kDispBatch; ++v) {
      const int p = b0 + v * kDispThreads + tid;
      if (p >= np) continue;
      const int e = ev[v];
      const bool ok = e >= 0 && e < E;
      if (!ok) raise_error(flags, kErrRange);
      erank[p] = ok ? atomicAdd(&cnt[e], 1) : -1;
    }
  }
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int u = c > 0 ? 1 : 0;
  const int nt = (c + kChunk - 1) / kChunk;
  int ic = c, iu = u, it = nt;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int oc = __shfl_up(ic, m, kWave), ou = __shfl_up(iu, m, kWave), ot = __shfl_up(it, m, kWave);
    if (lane >= m) { ic += oc; iu += ou; it += ot; }
  }
  if (lane == kWave - 1) { ws_c[w] = ic; ws_u[w] = iu; ws_t[w] = it; }
  __syncthreads();
  if (w == 0) {
    const int nw = kDispThreads / kWave;
    int vc = lane < nw ? ws_c[lane] : 0, vu = lane < nw ? ws_u[lane] : 0, vt = lane < nw ? ws_t[lane] : 0;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int oc = __shfl_up(vc, m, kWave), ou = __shfl_up(vu, m, kWave), ot = __shfl_up(vt, m, kWave);
      if (lane >= m) { vc += oc; vu += ou; vt += ot; }
    }
    if (lane < nw) { ws_c[lane] = vc; ws_u[lane] = vu; ws_t[lane] = vt; }
  }
  __syncthreads();
  const int start = (w > 0 ? ws_c[w - 1] : 0) + ic - c;
  const int rank = (w > 0 ? ws_u[w - 1] : 0) + iu - u;
  const int tile0 = (w > 0 ? ws_t[w - 1] : 0) + it - nt;
  if (tid < E) estart[tid] = start;
  if (tid < E && u) {
    uniq[rank] = tid;
    ustart[rank] = start;
    tstart[rank] = tile0;
    for (int i = 0; i < nt; ++i) tile_u[tile0 + i] = rank;
  }
  if (tid == kDispThreads - 1) {
    const int U = ws_u[kDispThreads / kWave - 1];
    const int routed = ws_t[kDispThreads / kWave - 1];
    const int shared_tiles = (T + kChunk - 1) / kChunk;
    *ucount = U;
    ustart[U] = ws_c[kDispThreads / kWave - 1];
    tstart[U] = routed;
    tstart[U + 1] = routed + shared_tiles;
    for (int i = 0; i < shared_tiles; ++i) tile_u[routed + i] = U;
    meta[0] = routed + shared_tiles;
  }
}

// ---------------------------------------------------------------------------
// x [T, H] bf16 -> float16 in MFMA k order, one thread per 8 values.
// The grid also writes the pair lists (pass 2 of the dispatch).
template <int BITS>
__global__ __launch_bounds__(kThreads) void k_pf_xprep(const uint16_t* __restrict__ x, u32x4* __restrict__ x16, int T,
                                                      int H, const int32_t* __restrict__ ids,
                                                      const int32_t* __restrict__ erank,
                                                      const int32_t* __restrict__ estart, int np,
                                                      int32_t* __restrict__ plist, const void* __restrict__ gvec,
                                                      float* __restrict__ gate, uint32_t* __restrict__ flags) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (size_t p = i; p < static_cast<size_t>(np); p += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int r = erank[p];
    if (r >= 0) plist[estart[ids[p]] + r] = static_cast<int32_t>(p);
  }
  // the shared-expert gates: wave 0 of block b takes tokens b, b + grid, ...
  if (threadIdx.x < kWave)
    for (int t = blockIdx.x; t < T; t += gridDim.x) pf_gate_token(x, gvec, gate, t, H, threadIdx.x);
  const int g_row = H / 8;
  if (i >= static_cast<size_t>(T) * g_row) return;
  const size_t t = i / g_row;
  const int g8 = static_cast<int>(i % g_row);
  const u32x4 v = load16(x + t * H + 8 * g8);
  u32x4 h;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const _Float16 lo = static_cast<_Float16>(__uint_as_float(v[m] << 16));
    const _Float16 hi = static_cast<_Float16>(__uint_as_float(v[m] & 0xffff0000u));
    h[m] = h2_bits(h2v{lo, hi});
  }
  if (f16_bad(h[0]) || f16_bad(h[1]) || f16_bad(h[2]) || f16_bad(h[3])) raise_error(flags, kErrF16);
  x16[t * g_row + chunk_of(g8)] = permute8<BITS>(h);
}

// ---------------------------------------------------------------------------
// Expert tiles.
struct PfArgs {
  const u32x4* x16;        // [T, H / 8] chunks in MFMA k order
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  const int32_t* ucount;
  const int32_t* uniq;
  const int32_t* ustart;
  const int32_t* plist;
  const int32_t* tstart;
  const int32_t* tile_u;
  const int32_t* meta;
  _Float16* h;             // [T k + T, hs] natural k order
  _Float16* partial;       // [T k + T, H]
  uint32_t* flags;
  int64_t pool_bytes;
  int T, k, H, E, I, SI, hs;
  int n_rt;                // blocks per tile in this launch
  int n_g;                 // down: 256-row blocks per block
  int slots_x;             // blocks resident at once on one XCD (0: no half blocks)
};

struct Tile {
  const uint8_t* blob;
  int rows_or_k;   // gate/up rows (I or SI), or the down contraction length
  int n;           // pairs in the tile
  int first;       // first plist position (routed) or first token (shared)
  bool shared;
  bool ok;
};

// The hardware hands consecutive blocks of a grid to the 8 XCDs in turn, and
// each XCD has its own L2.  Blocks are renumbered so that XCD x runs a
// contiguous range of (tile, row block) pairs in order: the row blocks of one
// tile then run on one XCD at about the same time and read the tile's
// activations through the same L2.  An XCD holds slots_x blocks at once, so
// the last (per mod slots_x) pairs of its range would run as a part-empty
// round; when that is at most half a round they run instead as twice as many
// half blocks (half = 0, 1; -1 for a whole block), which halves that round's
// length.  The grid is a multiple of kXcds blocks with at least
// kXcds (per + slots_x) of them; the spare ones return at once.
constexpr int kXcds = 8;

__device__ __forceinline__ bool block_map(const PfArgs& a, int* ti, int* rb, int* half) {
  const int nb = a.meta[0] * a.n_rt;
  const int per = (nb + kXcds - 1) / kXcds;
  const int idx = blockIdx.x / kXcds;
  const int tail = a.slots_x > 0 && per % a.slots_x <= a.slots_x / 2 ? per % a.slots_x : 0;
  const int full = per - tail;
  int item;
  if (idx < full) {
    item = idx;
    *half = -1;
  } else if (idx < full + 2 * tail) {
    item = full + (idx - full) / 2;
    *half = (idx - full) % 2;
  } else {
    return false;
  }
  const int logical = (blockIdx.x % kXcds) * per + item;
  if (logical >= nb) return false;
  *ti = logical / a.n_rt;
  *rb = logical % a.n_rt;
  return true;
}

// Uniform per block: which expert and which pairs this tile covers.
template <int BITS, int SB>
__device__ __forceinline__ bool tile_of(const PfArgs& a, int ti, Tile* tl) {
  if (ti >= a.meta[0]) return false;
  const int u = a.tile_u[ti];
  const int U = *a.ucount;
  const int chunk = ti - a.tstart[u];
  tl->shared = u == U;
  if (tl->shared) {
    tl->blob = a.shared;
    tl->rows_or_k = a.SI;
    tl->first = chunk * kChunk;
    tl->n = min(kChunk, a.T - tl->first);
    tl->ok = true;
  } else {
    const int beg = a.ustart[u] + chunk * kChunk;
    tl->first = beg;
    tl->n = min(kChunk, a.ustart[u + 1] - beg);
    tl->rows_or_k = a.I;
    const int64_t off = a.slot_table[a.uniq[u]];
    tl->ok = slot_ok(off, planes_of(a.H, a.I, BITS, SB).blob, a.pool_bytes);
    tl->blob = a.pool + (tl->ok ? off : 0);
  }
  return true;
}

__device__ __forceinline__ void tile_pairs(const PfArgs& a, const Tile& tl, int tid, int* s_pair, int* s_tok) {
  if (tid < tl.n) {
    const int p = tl.shared ? a.T * a.k + tl.first + tid : a.plist[tl.first + tid];
    s_pair[tid] = p;
    s_tok[tid] = tl.shared ? tl.first + tid : p / a.k;
  }
}

// Weights are read through a buffer descriptor over the tile's blob: each load
// takes this lane's byte offset (its row, its k quarter) and a wave-uniform
// offset (matrix plane, 16-row block, k step) in a scalar register, so the
// per-block addressing costs no vector registers.  Offsets past the blob read
// zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t blob_rsrc(const uint8_t* blob, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), 0,
                                           static_cast<int>(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
}

constexpr int kNonTemporal = 2;   // buffer-load cache policy: streamed once

// This lane's weights of one 128-k step for one 16-row MFMA block: its 32
// codes (int4: one 16-byte word, int8: two) and a scale and a bias word.  A
// 128-k step spans two 64-groups; lane quarter q uses group q / 2.  float32
// scales: the word is that group's value.  bf16 scales: the word holds both
// groups (low half first) and the lane picks its half with v_perm when it
// converts (sb_value); the four lanes of a row then load one shared word.
template <int BITS>
struct StepW {
  u32x4 c[BITS / 4];
  uint32_t s, b;
};

// Where one 16-row block's planes start (wave-uniform byte offsets in the
// blob) and where this lane's row starts inside them.
struct BlockOffsets {
  int code, scale, bias;   // uniform
};
struct LaneOffsets {
  int code, sb;            // per lane: row and k quarter (row only for bf16 scales)
  uint32_t sel;            // bf16 scales: v_perm selector of this lane's group half
};

template <int BITS, int SB>
__device__ __forceinline__ LaneOffsets lane_offsets(int lrow, int rbytes, int sbrow, int q) {
  LaneOffsets lo;
  lo.code = lrow * rbytes + 32 * q * BITS / 8;
  lo.sb = lrow * sbrow + (SB == kF32 ? (q >> 1) * 4 : 0);
  lo.sel = (q >> 1) ? 0x03020c0cu : 0x01000c0cu;   // bf16 bits -> top half of a float32, low half zero
  return lo;
}

// Float value of a scale or bias word for this lane.
template <int SB>
__device__ __forceinline__ float sb_value(uint32_t word, uint32_t sel) {
  if constexpr (SB == kF32) return __uint_as_float(word);
  else return __uint_as_float(__builtin_amdgcn_perm(0u, word, sel));
}

template <int BITS, int SB>
__device__ __forceinline__ void load_step(StepW<BITS>& w, __amdgpu_buffer_rsrc_t rs, LaneOffsets lo, BlockOffsets bo,
                                          int kb) {
  constexpr int sbsz = SB == kF32 ? 4 : 2;
#pragma unroll
  for (int i = 0; i < BITS / 4; ++i)
    w.c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo.code,
                                                                             bo.code + kb * BITS / 8 + 16 * i,
                                                                             kNonTemporal));
  w.s = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.sb, bo.scale + (kb / 64) * sbsz, 0);
  w.b = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.sb, bo.bias + (kb / 64) * sbsz, 0);
}

// Both 128-k steps of a 256-k slice (int4): the codes are one 128-byte line
// per row, and bf16 scales of the slice's four groups are one 8-byte word.
template <int SB>
__device__ __forceinline__ void load_slice4(StepW<4>& w0, StepW<4>& w1, __amdgpu_buffer_rsrc_t rs, LaneOffsets lo,
                                            BlockOffsets bo, int kb) {
  w0.c[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo.code, bo.code + kb / 2, kNonTemporal));
  w1.c[0] = __builtin_bit_cast(u32x4,
                               __builtin_amdgcn_raw_buffer_load_b128(rs, lo.code, bo.code + kb / 2 + 64, kNonTemporal));
  if constexpr (SB == kF32) {
    w0.s = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.sb, bo.scale + (kb / 64) * 4, 0);
    w1.s = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.sb, bo.scale + (kb / 64 + 2) * 4, 0);
    w0.b = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.sb, bo.bias + (kb / 64) * 4, 0);
    w1.b = __builtin_amdgcn_raw_buffer_load_b32(rs, lo.sb, bo.bias + (kb / 64 + 2) * 4, 0);
  } else {
    const auto sv = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.sb, bo.scale + (kb / 64) * 2, 0);
    const auto bv = __builtin_amdgcn_raw_buffer_load_b64(rs, lo.sb, bo.bias + (kb / 64) * 2, 0);
    w0.s = sv[0];
    w1.s = sv[1];
    w0.b = bv[0];
    w1.b = bv[1];
  }
}

// The codes alone of both 128-k steps of a 256-k slice (int4; the scales come
// through LDS).
__device__ __forceinline__ void load_codes4(StepW<4>& w0, StepW<4>& w1, __amdgpu_buffer_rsrc_t rs, LaneOffsets lo,
                                            BlockOffsets bo, int kb) {
  w0.c[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo.code, bo.code + kb / 2, kNonTemporal));
  w1.c[0] = __builtin_bit_cast(u32x4,
                               __builtin_amdgcn_raw_buffer_load_b128(rs, lo.code, bo.code + kb / 2 + 64, kNonTemporal));
}

__device__ __forceinline__ h2v splat_h2(float v) {
  const _Float16 h = static_cast<_Float16>(v);
  return h2v{h, h};
}

// A operand of MFMA k-step j.
template <int BITS>
__device__ __forceinline__ h8v step_operand(const StepW<BITS>& w, int j, h2v s, h2v b, uint32_t magic_v) {
  if constexpr (BITS == 4) {
    return dq_int4(w.c[0][j], s, b, magic_v);
  } else {
    const u32x4& cw = w.c[j >> 1];
    return dq_int8(cw[(2 * j) & 3], cw[(2 * j + 1) & 3], s, b, magic_v);
  }
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Calls f(IntC<nt>) for the tile's number of 16-column MFMA blocks, so that
// every loop over column blocks has a compile-time trip count.
template <typename F>
__device__ __forceinline__ void with_nt(int nt, F&& f) {
  switch (nt) {
    case 1: f(IntC<1>{}); break;
    case 2: f(IntC<2>{}); break;
    case 3: f(IntC<3>{}); break;
    default: f(IntC<4>{}); break;
  }
}

// Activation staging shared by both expert kernels.  One staged 256-k slice is
// chunk-major in LDS: [32 chunks in MFMA k order][64 columns][16 bytes], so the
// B operand of one MFMA (16 columns, one chunk per lane quarter) is four runs
// of 256 contiguous bytes.  The rows are copied global -> LDS by the gfx950
// direct loads (global_load_lds_dwordx4: lane l's 16 bytes land at the
// wave-uniform LDS address + 16 l), so they never pass through registers.
// Lane l copies column (pair) l, wave w chunks 8 w .. 8 w + 7.  Lanes past
// the tile's pairs copy column 0 again: MFMA columns are independent, and
// those columns are never written out.
constexpr int kChunkBytes = kChunk * 16;              // one chunk of all 64 columns
constexpr int kStageBytes = (kSlice / 8) * kChunkBytes;

// int4 codes with bf16 scales: the scale and bias words of a slice are copied
// into LDS with the slice's activations (direct 4-byte loads), instead of
// being held in registers one slice ahead.  Per wave and slice: [m][scale,
// bias][32 rows][2 words] for gate/up (word S holds the two groups of 128-k
// step S), [scale, bias][64 rows][2 words] for down: 1 KB per wave.
constexpr int kSbWave = 1024;
constexpr int kSbStage = 4 * kSbWave;
template <int BITS, int SB>
constexpr bool kLdsSb = BITS == 4 && SB == kBF16;

typedef __attribute__((address_space(3))) void lds_void;

// src: this lane's column at the wave's first chunk of slice 0 (bytes).
__device__ __forceinline__ void stage_slice(const uint8_t* src, int ks, uint8_t* stage, int w) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_global_load_lds(src + ks * 2 + 16 * i, (lds_void*)(stage + (8 * w + i) * kChunkBytes), 16, 0, 0);
}

// The direct copies of a stage must have landed, for every wave, before any
// wave reads it: wait for all of this wave's memory operations, then barrier.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

__device__ __forceinline__ h8v stage_b(const uint8_t* stage, int S, int j, int ct, int r, int q) {
  return *reinterpret_cast<const h8v*>(stage + (16 * S + 4 * j + q) * kChunkBytes + (16 * ct + r) * 16);
}


// Row-pair staging: one direct-load instruction brings two rows' 256-k
// slices (2 x 512 bytes, whole cache lines) into a 1 KB block of LDS; lane L
// copies chunk (L % 32) ^ (row & 7) of row 2 i + L / 32, so chunk c of a row
// sits at position 32 (row % 2) + (c ^ (row & 7)) of its block.  Sixteen
// lanes reading one chunk of sixteen consecutive rows then spread over all
// banks.  A 64-row slice is 32 blocks, 8 per wave.
__device__ __forceinline__ int pair_pos(int row, int chunk) {
  return (row >> 1) * kChunkBytes + (32 * (row & 1) + (chunk ^ (row & 7))) * 16;
}

// row_src: this lane's row (row 2 i + lane / 32 of each of the wave's blocks
// i = 8 w .. 8 w + 7, i.e. row 16 w + 2 j + lane / 32 for j < 8) at chunk
// (lane % 32) ^ (row & 7) of slice 0, given for each j.
struct PairRows {
  const uint8_t* src[8];
};

__device__ __forceinline__ void stage_pairs(const PairRows& pr, int ks, uint8_t* stage, int w) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_global_load_lds(pr.src[j] + ks * 2, (lds_void*)(stage + (8 * w + j) * kChunkBytes), 16, 0, 0);
}

// Row-pair staging of the activation rows of a tile (layout of pair_pos):
// this lane's byte offsets, one per block it copies, from a buffer
// descriptor over the whole activation array (under 2^31 bytes); the k
// offset of the slice is a scalar.
struct PairOffs {
  uint32_t off[8];
};

template <typename RowStart>
__device__ __forceinline__ PairOffs pair_offsets(int w, int lane, RowStart row_start) {
  PairOffs po;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 16 * w + 2 * j + (lane >> 5);
    po.off[j] = row_start(row) + 16u * static_cast<uint32_t>((lane & 31) ^ (row & 7));
  }
  return po;
}

__device__ __forceinline__ void stage_pairs(u32x4 src, const PairOffs& po, int ks, uint8_t* stage, int w) {
#pragma unroll
  for (int j = 0; j < 8; ++j) lds_load<16>(src, stage + (8 * w + j) * kChunkBytes, po.off[j], ks * 2);
}

// B operand reads of a row-pair staged slice: lane (r, q) reads chunk
// 16 S + 4 j + q of row 16 ct + r.  Rows 16 ct + r share r & 7 and the xor
// only touches a chunk's low three bits, so every read is one of two per-lane
// bases (by j % 2) plus a constant.
struct PairRead {
  int even, odd;
};

__device__ __forceinline__ PairRead pair_read(int r, int q) {
  const int row_part = (r >> 1) * kChunkBytes + 32 * (r & 1) * 16;
  return {row_part + (q ^ (r & 7)) * 16, row_part + ((4 + q) ^ (r & 7)) * 16};
}

__device__ __forceinline__ h8v stage_b_pair(const uint8_t* stage, const PairRead& pr, int S, int j, int ct) {
  return *reinterpret_cast<const h8v*>(stage + ((j & 1) ? pr.odd : pr.even) + ct * 8 * kChunkBytes + S * 256 +
                                       (j >> 1) * 128);
}

// Router logits [T, E] = x [T, H] . R [E, H]^T: bf16 operands (exact
// products), fp32 sums, on v_mfma_f32_16x16x32_bf16.  Block: 64 experts x 64
// tokens; wave w owns experts 16 w .. +15 for the 64 tokens (four column
// blocks).  Both operands are staged a 256-k slice at a time into LDS with
// row-pair direct loads (natural k order for both), two stages, one barrier
// per slice.  Blocks are renumbered so that
// XCD x runs a contiguous range of (token block, expert block) pairs,
// token-major: an XCD's blocks share their token tiles and the router matrix
// through its L2.
__global__ __launch_bounds__(kThreads) void k_pf_router(const uint16_t* __restrict__ x, const uint16_t* __restrict__ R,
                                                       float* __restrict__ logits, int T, int H, int E) {
  __shared__ __align__(16) uint8_t rs0[kStageBytes];
  __shared__ __align__(16) uint8_t rs1[kStageBytes];
  __shared__ __align__(16) uint8_t xs0[kStageBytes];
  __shared__ __align__(16) uint8_t xs1[kStageBytes];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int neb = (E + 63) / 64, nb = neb * ((T + 63) / 64);
  const int per = (nb + kXcds - 1) / kXcds;
  const int idx = blockIdx.x / kXcds;
  if (idx >= per) return;
  const int logical = (blockIdx.x % kXcds) * per + idx;
  if (logical >= nb) return;
  const int tb = logical / neb, eb = logical % neb;
  const int r = lane & 15, q = lane >> 4;
  // this lane's rows and chunks for the row-pair direct loads, clamped into
  // range (the sums of a clamped row are never stored)
  PairRows rsrc, xsrc;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 16 * w + 2 * j + (lane >> 5);              // row of the tile
    const int chunk = (lane & 31) ^ (row & 7);
    const int e_row = min(eb * 64 + row, E - 1), t_row = min(tb * 64 + row, T - 1);
    rsrc.src[j] = reinterpret_cast<const uint8_t*>(R + static_cast<size_t>(e_row) * H) + chunk * 16;
    xsrc.src[j] = reinterpret_cast<const uint8_t*>(x + static_cast<size_t>(t_row) * H) + chunk * 16;
  }
  f4v acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f4v{0.f, 0.f, 0.f, 0.f};
  auto mult = [&](const uint8_t* rst, const uint8_t* xst) {
#pragma unroll
    for (int st = 0; st < kSlice / 32; ++st) {
      const b8v A = *reinterpret_cast<const b8v*>(rst + pair_pos(16 * w + r, 4 * st + q));
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const b8v B = *reinterpret_cast<const b8v*>(xst + pair_pos(16 * ct + r, 4 * st + q));
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[ct], 0, 0, 0);
      }
    }
  };
  const int nsl = H / kSlice;
  stage_pairs(rsrc, 0, rs0, w);
  stage_pairs(xsrc, 0, xs0, w);
  stage_barrier();
  for (int sl = 0; sl < nsl; sl += 2) {
    if (sl + 1 < nsl) {
      stage_pairs(rsrc, (sl + 1) * kSlice, rs1, w);
      stage_pairs(xsrc, (sl + 1) * kSlice, xs1, w);
    }
    mult(rs0, xs0);
    stage_barrier();
    if (sl + 1 < nsl) {
      if (sl + 2 < nsl) {
        stage_pairs(rsrc, (sl + 2) * kSlice, rs0, w);
        stage_pairs(xsrc, (sl + 2) * kSlice, xs0, w);
      }
      mult(rs1, xs1);
      stage_barrier();
    }
  }
  // D row 4 q + i (expert), column r (token) of each column block
  const int e0 = eb * 64 + w * 16 + 4 * q;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int t = tb * 64 + 16 * ct + r;
    if (t < T) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e0 + i < E) logits[static_cast<size_t>(t) * E + e0 + i] = acc[ct][i];
    }
  }
}

// Natural k (0..7) that MFMA slot s of an 8-group stands for; see permute8.
template <int BITS>
__device__ __forceinline__ int slot_k(int s) {
  if constexpr (BITS == 4) return (s >> 1) + 4 * (s & 1);
  else return (s & 4) + ((s >> 1) & 1) + 2 * (s & 1);
}

// Gate/up: block = (tile, 128-row block); wave w owns rows 32 w .. +31 of gate
// and of up (two 16-row MFMA blocks each) for the tile's pairs (up to 4 column
// blocks).  h leaves in the down kernel's operand order: inside each 16-row
// block, MFMA row 4 q + i computes natural row 8 (q / 2) + slot_k(4 (q % 2) +
// i), so lane quarter q's four results are four consecutive slots of 8-group
// 2 b + q / 2, stored at chunk position chunk_of of that group.
// Software-pipelined over 256-k slices: while a slice is multiplied, the next
// slice's weights (registers) and activations (direct copies into the other
// LDS stage) are in flight; one barrier per slice.  Rows (I or SI) are
// multiples of 256, so every wave of a block has rows.
template <int BITS, int SB>
__global__ __launch_bounds__(kThreads, 2) void k_pf_gateup(PfArgs a) {
  constexpr bool kLsb = kLdsSb<BITS, SB>;
  __shared__ __align__(16) uint8_t xs0[kStageBytes + (kLsb ? kSbStage : 0)];
  __shared__ __align__(16) uint8_t xs1[kStageBytes + (kLsb ? kSbStage : 0)];
  __shared__ int s_pair[kChunk], s_tok[kChunk];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  int ti, rb, half;
  if (!block_map(a, &ti, &rb, &half)) return;
  Tile tl;
  if (!tile_of<BITS, SB>(a, ti, &tl)) return;
  const int rows = tl.rows_or_k;
  if (rb * kGuRows >= rows) return;
  if (!tl.ok) {
    if (tid == 0 && rb == 0) raise_error(a.flags, kErrRange);
    return;
  }
  tile_pairs(a, tl, tid, s_pair, s_tok);
  const int n = tl.n;
  const Planes P = planes_of(a.H, rows, BITS, SB);
  const __amdgpu_buffer_rsrc_t rs = blob_rsrc(tl.blob, P.blob);
  const int r = lane & 15, q = lane >> 4;
  const uint32_t magic_v = __builtin_amdgcn_readfirstlane(0x64006400);   // kept in a vector register by and_or
  constexpr int sbsz = SB == kF32 ? 4 : 2;
  const int rbytes = a.H * BITS / 8;
  const int sbrow = (a.H / 64) * sbsz;
  const int lrow = 8 * (r >> 3) + slot_k<BITS>(r & 7);          // this lane's row inside a 16-row block
  const LaneOffsets lo = lane_offsets<BITS, SB>(lrow, rbytes, sbrow, q);
  // RR 16-row MFMA blocks of gate and of up per wave: 2 for a whole block of
  // 128 rows, 1 for a half block (rows 64 half .. +64 of the row block)
  auto body = [&](auto rrc) {
    constexpr int RR = decltype(rrc)::value;
    const int wrow = rb * kGuRows + (half < 0 ? 0 : 64 * half) + w * 16 * RR;   // first row of the wave (uniform)
    BlockOffsets bo[2][RR];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int rr = 0; rr < RR; ++rr) {
        const int row = wrow + 16 * rr;
        bo[m][rr] = {static_cast<int>(m * P.q) + row * rbytes, static_cast<int>(3 * P.q + m * P.s) + row * sbrow,
                     static_cast<int>(3 * P.q + (3 + m) * P.s) + row * sbrow};
      }
    __syncthreads();   // s_tok ready
    const uint8_t* xsrc = reinterpret_cast<const uint8_t*>(a.x16) +
                          static_cast<size_t>(s_tok[lane < n ? lane : 0]) * a.H * 2 + w * 8 * 16;
    // int4 with bf16 scales: activations staged as row pairs (whole lines per
    // direct load)
    const u32x4 xrs = raw_rsrc(a.x16, static_cast<int64_t>(a.T) * a.H * 2);
    const u32x4 rsa = raw_rsrc(tl.blob, P.blob);
    PairOffs xo;
    if constexpr (kLsb)
      xo = pair_offsets(w, lane, [&](int row) {
        return static_cast<uint32_t>(s_tok[row < n ? row : 0]) * static_cast<uint32_t>(a.H * 2);
      });
    const PairRead prd = pair_read(r, q);
    auto stage_x = [&](int ks, uint8_t* stage) {
      if constexpr (kLsb) stage_pairs(xrs, xo, ks, stage, w);
      else stage_slice(xsrc, ks, stage, w);
    };
    auto load_w = [&](StepW<BITS> (&dst)[2][RR], int kb) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rr = 0; rr < RR; ++rr) load_step<BITS, SB>(dst[m][rr], rs, lo, bo[m][rr], kb);
    };
    auto load_w2 = [&](StepW<BITS> (&d0)[2][RR], StepW<BITS> (&d1)[2][RR], int kb) {
      if constexpr (kLsb) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int rr = 0; rr < RR; ++rr) load_codes4(d0[m][rr], d1[m][rr], rs, lo, bo[m][rr], kb);
      } else if constexpr (BITS == 4) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int rr = 0; rr < RR; ++rr) load_slice4<SB>(d0[m][rr], d1[m][rr], rs, lo, bo[m][rr], kb);
      }
    };
    // the wave's 32 rows' scale and bias words of the slice at kb: lane l
    // copies word l % 2 of row l / 2 of one plane
    const uint32_t sb_lane = static_cast<uint32_t>((lane >> 1) * sbrow + 4 * (lane & 1));
    auto stage_sb = [&](int kb, uint8_t* stage) {
      if constexpr (kLsb) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const int soff = static_cast<int>(3 * P.q + (sb ? 3 + m : m) * P.s) + wrow * sbrow + (kb / 64) * 2;
            lds_load<4>(rsa, stage + kStageBytes + w * kSbWave + (2 * m + sb) * 256, sb_lane, soff);
          }
      }
    };
    with_nt((n + 15) / 16, [&](auto ntc) {
      constexpr int NT = decltype(ntc)::value;
      f4v acc[2][RR][NT];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rr = 0; rr < RR; ++rr)
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) acc[m][rr][ct] = f4v{0.f, 0.f, 0.f, 0.f};
      // One 128-k step S (0 or 1) of the slice staged in `stage`.
      auto mult = [&](int S, const uint8_t* stage, const StepW<BITS> (&wv)[2][RR]) {
        h2v sc[2][RR], bc[2][RR];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int rr = 0; rr < RR; ++rr) {
            if constexpr (kLsb) {
              const uint8_t* sw = stage + kStageBytes + w * kSbWave + 2 * m * 256 + (16 * rr + lrow) * 8;
              const uint2 sv = *reinterpret_cast<const uint2*>(sw), bv = *reinterpret_cast<const uint2*>(sw + 256);
              sc[m][rr] = splat_h2(sb_value<SB>(S ? sv.y : sv.x, lo.sel));
              bc[m][rr] = splat_h2(sb_value<SB>(S ? bv.y : bv.x, lo.sel));
            } else {
              sc[m][rr] = splat_h2(sb_value<SB>(wv[m][rr].s, lo.sel));
              bc[m][rr] = splat_h2(sb_value<SB>(wv[m][rr].b, lo.sel));
            }
          }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h8v B[NT];
#pragma unroll
          for (int ct = 0; ct < NT; ++ct)
            B[ct] = kLsb ? stage_b_pair(stage, prd, S, j, ct) : stage_b(stage, S, j, ct, r, q);
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int rr = 0; rr < RR; ++rr) {
              const h8v A = step_operand<BITS>(wv[m][rr], j, sc[m][rr], bc[m][rr], magic_v);
#pragma unroll
              for (int ct = 0; ct < NT; ++ct) acc[m][rr][ct] = mfma16(A, B[ct], acc[m][rr][ct]);
            }
        }
      };
      if constexpr (BITS == 4) {
        // int4: a 128-k step is half of each row's 128-byte line; both steps of
        // the next slice are requested together so that lines are fetched whole.
        // The two register sets alternate roles from slice to slice.
        StepW<BITS> wa[2][RR], wa2[2][RR], wb[2][RR], wb2[2][RR];
        const int nsl = a.H / kSlice;
        auto slice = [&](int sl, const uint8_t* cur, uint8_t* nxt, const StepW<BITS> (&c1)[2][RR],
                         const StepW<BITS> (&c2)[2][RR], StepW<BITS> (&n1)[2][RR], StepW<BITS> (&n2)[2][RR]) {
          const bool more = sl + 1 < nsl;
          if (more) {
            stage_x((sl + 1) * kSlice, nxt);
            stage_sb((sl + 1) * kSlice, nxt);
            load_w2(n1, n2, (sl + 1) * kSlice);
          }
          mult(0, cur, c1);
          mult(1, cur, c2);
          stage_barrier();
        };
        stage_x(0, xs0);
        stage_sb(0, xs0);
        load_w2(wa, wa2, 0);
        stage_barrier();
        for (int sl = 0; sl < nsl; sl += 2) {
          slice(sl, xs0, xs1, wa, wa2, wb, wb2);
          if (sl + 1 < nsl) slice(sl + 1, xs1, xs0, wb, wb2, wa, wa2);
        }
      } else {
        // int8: one 128-k step already covers whole lines; prefetch one step
        // ahead, alternating two register sets.  The number of steps is even.
        StepW<BITS> wa[2][RR], wb[2][RR];
        const int nst = a.H / 128;
        auto step = [&](int st, int S, const uint8_t* cur, uint8_t* nxt, const StepW<BITS> (&cw)[2][RR],
                        StepW<BITS> (&nw)[2][RR]) {
          if (S == 0 && st + 2 < nst) stage_slice(xsrc, (st + 2) * 128, nxt, w);
          if (st + 1 < nst) load_w(nw, (st + 1) * 128);
          mult(S, cur, cw);
          if (S == 1) stage_barrier();
        };
        stage_slice(xsrc, 0, xs0, w);
        load_w(wa, 0);
        stage_barrier();
        for (int st = 0; st < nst; st += 4) {
          step(st, 0, xs0, xs1, wa, wb);
          step(st + 1, 1, xs0, xs1, wb, wa);
          if (st + 2 < nst) {
            step(st + 2, 0, xs1, xs0, wa, wb);
            step(st + 3, 1, xs1, xs0, wb, wa);
          }
        }
      }
      // h = silu(gate) * up, float16, four consecutive slots per lane
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int c = 16 * ct + r;
        if (c < n) {
          _Float16* hr = a.h + static_cast<size_t>(s_pair[c]) * a.hs;
#pragma unroll
          for (int rr = 0; rr < RR; ++rr) {
            const int g8 = (wrow + 16 * rr) / 8 + (q >> 1);
            uint32_t o[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const _Float16 h0 = static_cast<_Float16>(silu(acc[0][rr][ct][2 * i]) * acc[1][rr][ct][2 * i]);
              const _Float16 h1 = static_cast<_Float16>(silu(acc[0][rr][ct][2 * i + 1]) * acc[1][rr][ct][2 * i + 1]);
              o[i] = h2_bits(h2v{h0, h1});
            }
            if (f16_bad(o[0]) || f16_bad(o[1])) raise_error(a.flags, kErrF16);
            *reinterpret_cast<uint2*>(hr + 8 * chunk_of(g8) + 4 * (q & 1)) = make_uint2(o[0], o[1]);
          }
        }
      }
    });
  };
  if (half < 0) body(IntC<2>{});
  else body(IntC<1>{});
}

// Down: block = (tile, n_g consecutive 256-row blocks of H); wave w owns
// rows 64 w .. +63 (four 16-row MFMA blocks) of each row block for the tile's
// pairs.  h rows arrive in operand order and are staged like x.  Writes the
// fp32 sums rounded to float16 partial rows (half the bytes written here and
// read back by the combine; like x and h, values must stay inside the float16
// range); a tile of an unusable blob writes zeros, so that expert contributes
// nothing.
// int4 with bf16 scales: the block walks its row blocks one 256-k slice
// ("step") at a time with the next step's codes in registers and its scales
// and h slice in the other LDS stage; with K <= 512 the h tile stays
// resident after the first two steps.  Other formats: one row block per
// block, pipelined over slices like the gate/up kernel.
template <int BITS, int SB>
__global__ __launch_bounds__(kThreads, 2) void k_pf_down(PfArgs a) {
  constexpr bool kLsb = kLdsSb<BITS, SB>;
  __shared__ __align__(16) uint8_t hs0[kStageBytes + (kLsb ? kSbStage : 0)];
  __shared__ __align__(16) uint8_t hs1[kStageBytes + (kLsb ? kSbStage : 0)];
  __shared__ int s_pair[kChunk], s_tok[kChunk];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  int ti, rb, half;
  if (!block_map(a, &ti, &rb, &half)) return;
  Tile tl;
  if (!tile_of<BITS, SB>(a, ti, &tl)) return;
  const int K = tl.rows_or_k;
  const int n = tl.n;
  // a half block is one of the n_g = 2 row blocks (rb counts row blocks then)
  const int G = half < 0 ? a.n_g : 1;
  if (half >= 0) rb = rb * a.n_g + half;
  tile_pairs(a, tl, tid, s_pair, s_tok);
  __syncthreads();
  const int r = lane & 15, q = lane >> 4;
  if (!tl.ok) {
    // zero this block's output rows of the tile's pairs
    const int span = G * kDnRows;
    for (int i = tid; i < n * (span / 4); i += kThreads) {
      const int c = i / (span / 4), col = (i % (span / 4)) * 4;
      *reinterpret_cast<uint2*>(a.partial + static_cast<size_t>(s_pair[c]) * a.H + rb * span + col) =
          make_uint2(0u, 0u);
    }
    return;
  }
  const Planes P = planes_of(a.H, K, BITS, SB);   // down is [H, K]
  const __amdgpu_buffer_rsrc_t rs = blob_rsrc(tl.blob, P.blob);
  const uint32_t magic_v = __builtin_amdgcn_readfirstlane(0x64006400);
  constexpr int sbsz = SB == kF32 ? 4 : 2;
  const int rbytes = K * BITS / 8;
  const int sbrow = (K / 64) * sbsz;
  const int wrow = rb * G * kDnRows + w * 64;   // the wave's first row in the first row block
  const LaneOffsets lo = lane_offsets<BITS, SB>(r, rbytes, sbrow, q);
  BlockOffsets bo[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = wrow + 16 * rr;
    bo[rr] = {static_cast<int>(2 * P.q) + row * rbytes, static_cast<int>(3 * P.q + 2 * P.s) + row * sbrow,
              static_cast<int>(3 * P.q + 5 * P.s) + row * sbrow};
  }
  const uint8_t* hsrc = reinterpret_cast<const uint8_t*>(a.h) +
                        static_cast<size_t>(s_pair[lane < n ? lane : 0]) * a.hs * 2 + w * 8 * 16;
  const u32x4 hrs = raw_rsrc(a.h, (static_cast<int64_t>(a.T) * a.k + a.T) * a.hs * 2);
  const u32x4 rsa = raw_rsrc(tl.blob, P.blob);
  PairOffs ho;
  if constexpr (kLsb)
    ho = pair_offsets(w, lane, [&](int row) {
      return static_cast<uint32_t>(s_pair[row < n ? row : 0]) * static_cast<uint32_t>(a.hs * 2);
    });
  const PairRead prd = pair_read(r, q);
  auto load_w = [&](StepW<BITS> (&dst)[4], int kb) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) load_step<BITS, SB>(dst[rr], rs, lo, bo[rr], kb);
  };
  auto load_w2 = [&](StepW<BITS> (&d0)[4], StepW<BITS> (&d1)[4], int kb) {
    if constexpr (BITS == 4) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) load_slice4<SB>(d0[rr], d1[rr], rs, lo, bo[rr], kb);
    }
  };
  with_nt((n + 15) / 16, [&](auto ntc) {
    constexpr int NT = decltype(ntc)::value;
    f4v acc[4][NT];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) acc[rr][ct] = f4v{0.f, 0.f, 0.f, 0.f};
    // One 128-k step S of the slice in `stage`; scale words from registers or,
    // with kLsb, from the stage's scale area.
    auto mult = [&](int S, const uint8_t* stage, const StepW<BITS> (&wv)[4]) {
      h2v sc[4], bc[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        if constexpr (kLsb) {
          const uint8_t* sw = stage + kStageBytes + w * kSbWave + (16 * rr + r) * 8;
          const uint2 sv = *reinterpret_cast<const uint2*>(sw), bv = *reinterpret_cast<const uint2*>(sw + 512);
          sc[rr] = splat_h2(sb_value<SB>(S ? sv.y : sv.x, lo.sel));
          bc[rr] = splat_h2(sb_value<SB>(S ? bv.y : bv.x, lo.sel));
        } else {
          sc[rr] = splat_h2(sb_value<SB>(wv[rr].s, lo.sel));
          bc[rr] = splat_h2(sb_value<SB>(wv[rr].b, lo.sel));
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h8v B[NT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
          B[ct] = kLsb ? stage_b_pair(stage, prd, S, j, ct) : stage_b(stage, S, j, ct, r, q);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const h8v A = step_operand<BITS>(wv[rr], j, sc[rr], bc[rr], magic_v);
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) acc[rr][ct] = mfma16(A, B[ct], acc[rr][ct]);
        }
      }
    };
    // partial rows of the row block whose first wave row is row0
    auto store = [&](int row0) {
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const int c = 16 * ct + r;
        if (c < n) {
          _Float16* pr = a.partial + static_cast<size_t>(s_pair[c]) * a.H + row0 + 4 * q;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const h2v lo = {static_cast<_Float16>(acc[rr][ct][0]), static_cast<_Float16>(acc[rr][ct][1])};
            const h2v hi = {static_cast<_Float16>(acc[rr][ct][2]), static_cast<_Float16>(acc[rr][ct][3])};
            if (f16_bad(h2_bits(lo)) || f16_bad(h2_bits(hi))) raise_error(a.flags, kErrF16);
            *reinterpret_cast<uint2*>(pr + 16 * rr) = make_uint2(h2_bits(lo), h2_bits(hi));
          }
        }
      }
    };
    if constexpr (kLsb) {
      const int nsl = K / kSlice;
      const int nsteps = G * nsl;
      // step st: row block st / nsl (rows from wrow + that * kDnRows), slice st % nsl
      const uint32_t sb_lane = static_cast<uint32_t>((lane >> 1) * sbrow + 4 * (lane & 1));
      auto stage_step = [&](int st, uint8_t* stage) {
        const int g = st / nsl, ks = (st % nsl) * kSlice;
        if (nsl > 2 || st < 2) stage_pairs(hrs, ho, ks, stage, w);   // else the stage already holds it
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int soff = static_cast<int>(3 * P.q + (sb ? 5 : 2) * P.s) +
                             (wrow + g * kDnRows + 32 * half) * sbrow + (ks / 64) * 2;
            lds_load<4>(rsa, stage + kStageBytes + w * kSbWave + sb * 512 + half * 256, sb_lane, soff);
          }
      };
      auto load_codes = [&](StepW<BITS> (&d0)[4], StepW<BITS> (&d1)[4], int st) {
        const int g = st / nsl, ks = (st % nsl) * kSlice;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          load_codes4(d0[rr], d1[rr], rs, lo, BlockOffsets{bo[rr].code + g * kDnRows * rbytes, 0, 0}, ks);
      };
      StepW<BITS> wa[4], wa2[4], wb[4], wb2[4];
      auto step = [&](int st, const uint8_t* cur, uint8_t* nxt, const StepW<BITS> (&c1)[4],
                      const StepW<BITS> (&c2)[4], StepW<BITS> (&n1)[4], StepW<BITS> (&n2)[4]) {
        if (st + 1 < nsteps) {
          stage_step(st + 1, nxt);
          load_codes(n1, n2, st + 1);
        }
        mult(0, cur, c1);
        mult(1, cur, c2);
        if (st % nsl == nsl - 1) {
          store(wrow + (st / nsl) * kDnRows);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) acc[rr][ct] = f4v{0.f, 0.f, 0.f, 0.f};
        }
        stage_barrier();
      };
      stage_step(0, hs0);
      load_codes(wa, wa2, 0);
      stage_barrier();
      for (int st = 0; st < nsteps; st += 2) {
        step(st, hs0, hs1, wa, wa2, wb, wb2);
        if (st + 1 < nsteps) step(st + 1, hs1, hs0, wb, wb2, wa, wa2);
      }
    } else if constexpr (BITS == 4) {
      StepW<BITS> wa[4], wa2[4], wb[4], wb2[4];
      const int nsl = K / kSlice;
      auto slice = [&](int sl, const uint8_t* cur, uint8_t* nxt, const StepW<BITS> (&c1)[4],
                       const StepW<BITS> (&c2)[4], StepW<BITS> (&n1)[4], StepW<BITS> (&n2)[4]) {
        const bool more = sl + 1 < nsl;
        if (more) {
          stage_slice(hsrc, (sl + 1) * kSlice, nxt, w);
          load_w2(n1, n2, (sl + 1) * kSlice);
        }
        mult(0, cur, c1);
        mult(1, cur, c2);
        stage_barrier();
      };
      stage_slice(hsrc, 0, hs0, w);
      load_w2(wa, wa2, 0);
      stage_barrier();
      for (int sl = 0; sl < nsl; sl += 2) {
        slice(sl, hs0, hs1, wa, wa2, wb, wb2);
        if (sl + 1 < nsl) slice(sl + 1, hs1, hs0, wb, wb2, wa, wa2);
      }
      store(wrow);
    } else {
      StepW<BITS> wa[4], wb[4];
      const int nst = K / 128;
      auto step = [&](int st, int S, const uint8_t* cur, uint8_t* nxt, const StepW<BITS> (&cw)[4],
                      StepW<BITS> (&nw)[4]) {
        if (S == 0 && st + 2 < nst) stage_slice(hsrc, (st + 2) * 128, nxt, w);
        if (st + 1 < nst) load_w(nw, (st + 1) * 128);
        mult(S, cur, cw);
        if (S == 1) stage_barrier();
      };
      stage_slice(hsrc, 0, hs0, w);
      load_w(wa, 0);
      stage_barrier();
      for (int st = 0; st < nst; st += 4) {
        step(st, 0, hs0, hs1, wa, wb);
        step(st + 1, 1, hs0, hs1, wb, wa);
        if (st + 2 < nst) {
          step(st + 2, 0, hs1, hs0, wa, wb);
          step(st + 3, 1, hs1, hs0, wb, wa);
        }
      }
      store(wrow);
    }
  });
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers.

bool prefill_supported(const moe_desc& d, int T) {
  // weight offsets inside a blob are 32-bit buffer offsets
  const int wide = d.inter > d.shared_inter ? d.inter : d.shared_inter;
  const bool blob_fits = planes_of(d.hidden, wide, d.bits, d.sb_dtype).blob < (int64_t{1} << 31);
  // activations read through 32-bit buffer offsets
  const int64_t h_bytes = (static_cast<int64_t>(T) * d.top_k + T) * wide * 2;
  const bool act_fits = static_cast<int64_t>(T) * d.hidden * 2 < (int64_t{1} << 31) && h_bytes < (int64_t{1} << 31);
  return T >= kPrefillMinT && d.act_dtype == kBF16 && d.hidden % kSlice == 0 && d.inter % kSlice == 0 &&
         d.shared_inter % kSlice == 0 && d.n_experts <= 1024 && blob_fits && act_fits;
}

static int last_error() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

int launch_prefill_router(const Call& c, int32_t* ids2, float* wts2) {
  const moe_desc& d = c.d;
  float* logits = reinterpret_cast<float*>(c.ws + c.L.logits);
  int32_t* ids = reinterpret_cast<int32_t*>(c.ws + c.L.ids);
  float* wts = reinterpret_cast<float*>(c.ws + c.L.wts);
  const int nb = ((d.n_experts + 63) / 64) * ((c.T + 63) / 64);
  const dim3 grid(static_cast<unsigned>((nb + kXcds - 1) / kXcds * kXcds));
  launch_kernel(k_pf_router, grid, dim3(kThreads), 0, c.stream, static_cast<const uint16_t*>(c.x),
                static_cast<const uint16_t*>(c.router_w), logits, c.T, d.hidden, d.n_experts);
  if (last_error()) return MOE_EHIP;
  return launch_topk(c, logits, ids, wts, ids2, wts2);
}

// Blocks for up to max_tiles tiles of n_rt row blocks, rounded up to a
// multiple of the XCD count, plus room for the half blocks (see block_map).
static unsigned xcd_grid(int max_tiles, int n_rt, int slots_x) {
  const unsigned nb = static_cast<unsigned>(max_tiles) * n_rt;
  return (nb + kXcds - 1) / kXcds * kXcds + kXcds * static_cast<unsigned>(slots_x);
}

// Blocks of a prefill GEMM kernel resident at once on one XCD (two per CU),
// per device; 0 if the device cannot be queried.
static int xcd_slots() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < kXcds) return 0;
    cached[dev] = 2 * cus / kXcds;
  }
  return cached[dev];
}

template <int BITS, int SB>
static void launch_tiles(const PfArgs& base, const Call& c) {
  const moe_desc& d = c.d;
  PfArgs a = base;
  a.n_rt = (d.inter > d.shared_inter ? d.inter : d.shared_inter) / kGuRows;
  a.slots_x = xcd_slots();
  launch_kernel(k_pf_gateup<BITS, SB>, dim3(xcd_grid(c.L.max_tiles, a.n_rt, a.slots_x)), dim3(kThreads), 0,
                c.stream, a);
  a.n_g = kLdsSb<BITS, SB> && (d.hidden / kDnRows) % kDownGroup == 0 ? kDownGroup : 1;
  a.n_rt = d.hidden / (kDnRows * a.n_g);
  a.slots_x = a.n_g == 2 ? xcd_slots() : 0;   // a half block is one of two row blocks
  launch_kernel(k_pf_down<BITS, SB>, dim3(xcd_grid(c.L.max_tiles, a.n_rt, a.slots_x)), dim3(kThreads), 0,
                c.stream, a);
}

int launch_prefill_experts(const Call& c) {
  const moe_desc& d = c.d;
  uint8_t* ws = c.ws;
  const WsLayout& L = c.L;
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.ctrl);
  float* gate = reinterpret_cast<float*>(ws + L.gate);
  _Float16* partial = reinterpret_cast<_Float16*>(ws + L.partial);
  PfArgs a;
  a.x16 = reinterpret_cast<const u32x4*>(ws + L.p_x16);
  a.slot_table = c.slot_table;
  a.pool = c.pool;
  a.shared = c.shared;
  a.ucount = reinterpret_cast<const int32_t*>(ws + L.ucount);
  a.uniq = reinterpret_cast<const int32_t*>(ws + L.uniq);
  a.ustart = reinterpret_cast<const int32_t*>(ws + L.ustart);
  a.plist = reinterpret_cast<const int32_t*>(ws + L.plist);
  a.tstart = reinterpret_cast<const int32_t*>(ws + L.p_tstart);
  a.tile_u = reinterpret_cast<const int32_t*>(ws + L.p_tile);
  a.meta = reinterpret_cast<const int32_t*>(ws + L.p_meta);
  a.h = reinterpret_cast<_Float16*>(ws + L.h);
  a.partial = partial;
  a.flags = flags;
  a.pool_bytes = d.pool_bytes;
  a.T = c.T;
  a.k = d.top_k;
  a.H = d.hidden;
  a.E = d.n_experts;
  a.I = d.inter;
  a.SI = d.shared_inter;
  a.hs = L.hstride;
  a.n_rt = 1;
  a.n_g = 1;
  a.slots_x = 0;

  const void* gvec = c.shared + d.shared_stride;
  int32_t* estart = reinterpret_cast<int32_t*>(ws + L.p_estart);
  int32_t* erank = reinterpret_cast<int32_t*>(ws + L.p_erank);
  launch_kernel(k_pf_dispatch, dim3(1), dim3(kDispThreads), 0, c.stream, c.ids, c.T, d.top_k, d.n_experts, erank,
                estart, const_cast<int32_t*>(a.ucount), const_cast<int32_t*>(a.uniq), const_cast<int32_t*>(a.ustart),
                const_cast<int32_t*>(a.tstart), const_cast<int32_t*>(a.tile_u), const_cast<int32_t*>(a.meta), flags);
  const size_t nchunk = static_cast<size_t>(c.T) * d.hidden / 8;
  const dim3 xgrid(static_cast<unsigned>((nchunk + kThreads - 1) / kThreads));
  u32x4* x16 = reinterpret_cast<u32x4*>(ws + L.p_x16);
  const uint16_t* x = static_cast<const uint16_t*>(c.x);
  const int np = c.T * d.top_k;
  int32_t* plist = const_cast<int32_t*>(a.plist);
  if (d.bits == 4)
    launch_kernel(k_pf_xprep<4>, xgrid, dim3(kThreads), 0, c.stream, x, x16, c.T, d.hidden, c.ids,
                  static_cast<const int32_t*>(erank), static_cast<const int32_t*>(estart), np, plist, gvec, gate, a.flags);
  else
    launch_kernel(k_pf_xprep<8>, xgrid, dim3(kThreads), 0, c.stream, x, x16, c.T, d.hidden, c.ids,
                  static_cast<const int32_t*>(erank), static_cast<const int32_t*>(estart), np, plist, gvec, gate, a.flags);
  if (d.bits == 4 && d.sb_dtype == kBF16) launch_tiles<4, kBF16>(a, c);
  else if (d.bits == 4) launch_tiles<4, kF32>(a, c);
  else if (d.sb_dtype == kBF16) launch_tiles<8, kBF16>(a, c);
  else launch_tiles<8, kF32>(a, c);
  if (last_error()) return MOE_EHIP;
  return launch_combine(c, partial, gate);
}

}  // namespace moe
