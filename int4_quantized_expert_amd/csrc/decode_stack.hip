// Persistent decode of a stack of MoE layers, one token per layer (gfx950).
//
// One launch runs L layers in order on a grid of one resident 512-thread
// block per CU.  Per layer:
//   R  router rows, the shared expert's gate/up rows and sigmoid(g . x), from
//      operands already in LDS (copied there while the previous layer ran)
//   K  every block gathers the E logits and takes top-k and the renormalised
//      weights itself, all eight waves at once
//   G  the routed gate/up rows, an equal share per block, every load of a
//      wave requested at once; meanwhile one wave copies the block's down
//      operands (its output rows of each chosen expert) into LDS
//   H  every block gathers h (k routed rows, the shared row, the gate)
//   D  down rows from LDS, ordered combine, output (and, in a chain, the next
//      layer's input x + y, exchanged like h)
// Blocks exchange data only through tagged 64-bit words: the value's bits
// and a per-layer tag, written with relaxed device-scope stores and read with
// device-scope loads until every word a block needs carries the tag.  Words
// are written in several replicas, each read by a fraction of the blocks.
// Every wait is bounded; on expiry the kernel raises kErrTimeout and skips
// all later waits.
//
// Work inside a layer needs every block resident at once (checked with the
// occupancy query when the plan is made).  Across layers, one exchange per
// layer (h) orders everything: a block writes a layer's words only after it
// has read every block's h of the layer before, so a buffer is never
// overwritten while another block may still read it.
//
// The arithmetic of every row (segment FMA chains, v_dot2 on exact bf16
// codes, the symmetric lane reductions, the combine order) is that of the
// staged kernels, so both give the same bits.
//
// Sources: routing to k of E experts plus a shared expert in every layer, and
// the whole layer stack run per token on the GPU (Swiftlet README
// translation, "How it works" and "Status"); int4 affine group quantization
// with byte-addressed kernels and 64-bit offsets (same page, "Relation to
// TurboFieldfare"); the decode loop reported as bound by dispatch rather than
// by expert reads (linlog.top article, "Capability limits").
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {

namespace {

constexpr int kH = 2048;                   // hidden size this kernel is built for
constexpr int kI = 512;                    // routed and shared intermediate size
constexpr int kThr = 512;
constexpr int kNW = kThr / kWave;          // 8 waves per block
constexpr int kGW = 6;                     // waves 0..5 take the phase-G rows
constexpr int kWaveStatic = 6;             // copies the next layer's static operands
constexpr int kWaveDown = 7;               // copies the routed down operands
constexpr int kSegI = kI / kSegCodes;      // 16 segments per down row
constexpr int kRpp = kWave / kSegI;        // 4 down rows per wave pass
constexpr int kPad = kSegCodes + 4;        // staged h: floats per segment (bank spread)
constexpr int64_t kQ = int64_t(kH) * kI / 2;        // code bytes of one matrix
constexpr int64_t kS = int64_t(kH) * (kI / 64) * 2; // bf16 scale bytes of one matrix
constexpr int64_t kBlob = 3 * kQ + 6 * kS;
constexpr int kRowQ = kH / 2;              // code bytes of a gate/up row
constexpr int kDRowQ = kI / 2;             // code bytes of a down row
constexpr int kDRowSB = (kI / 64) * 2;     // scale (or bias) bytes of a down row
constexpr int kLgRep = 8, kHRep = 4, kXRep = 8;   // copies of the exchanged words
constexpr int kFlagRep = 16;                        // copies of the per-block flags
constexpr int kMaxNb = 512;                         // blocks whose flags one wave polls
constexpr int kMaxK = 10, kMaxRpb = 4, kMaxSpb = 4, kMaxRb = 16, kMaxG = 4, kMaxE = 512;
constexpr int kMaxHn = (kMaxK + 1) * kI + 1;        // exchanged h words: k routed rows, shared row, gate
constexpr int kRdWaves = 6;                         // waves that read exchanged words (0..5)
constexpr int kRdThr = kRdWaves * kWave;
constexpr int kFlLg = 0, kFlH = 1, kFlX = 2;        // flag kinds

// Bytes of LDS per region, rounded so that 256-byte direct-load rounds that
// run past a region's end land in its own padding.
__host__ __device__ constexpr uint32_t r256(uint32_t n) { return (n + 255u) / 256u * 256u; }

struct SLds {
  // static operands of one layer (two copies, by layer parity)
  uint32_t p_x, p_rr, p_suq, p_susb, p_sdq, p_sdsb, p_slot, p_gv, p_bytes;
  uint32_t p[2];
  uint32_t d, d_per;   // routed down operands: [k][d_per] = codes [rb][256], scales [rb][8], biases [rb][8]
  uint32_t hs;         // staged h [(k + 1) * kSegI][kPad] floats
  uint32_t hsum;       // [(k + 1) * kSegI] segment sums
  uint32_t lg;         // [kMaxE] logits
  uint32_t cand;       // [kWave] packed top-k candidates (wave 0)
  uint32_t misc;       // see below
  uint32_t part;       // [(k + 1) * rb] partial down sums
  uint32_t total;
};

// misc words (32-bit each)
constexpr int kMIds = 0;              // [kMaxK] chosen experts by rank
constexpr int kMVals = kMIds + kMaxK; // [kMaxK] chosen logits, then weights
constexpr int kMSig = kMVals + kMaxK; // sigmoid(g . x)
constexpr int kMOk = kMSig + 1;       // result of the last flag wait
constexpr int kMRd = kMOk + 1;        // [kRdWaves] results of the reading waves
constexpr int kMOff = 64;             // [kMaxK] int64 blob offsets by rank (8-byte aligned)
constexpr int kMWords = kMOff + 2 * kMaxK;

__host__ __device__ inline SLds stack_lds(int E, int k, int rpb, int spb, int rb) {
  SLds s{};
  uint32_t o = 0;
  s.p_x = o;    o += r256(kH * 2);
  s.p_rr = o;   o += r256(static_cast<uint32_t>(rpb) * kH * 2);
  s.p_suq = o;  o += r256(static_cast<uint32_t>(spb) * 2 * kRowQ);
  s.p_susb = o; o += r256(static_cast<uint32_t>(spb) * 4 * (kH / 64) * 2);
  s.p_sdq = o;  o += r256(static_cast<uint32_t>(rb) * kDRowQ);
  s.p_sdsb = o; o += r256(static_cast<uint32_t>(rb) * 2 * kDRowSB);
  s.p_slot = o; o += r256(static_cast<uint32_t>(E) * 8);
  s.p_gv = o;   o += r256(kH * 2);
  s.p_bytes = o;
  s.p[0] = 0;
  s.p[1] = s.p_bytes;
  uint32_t t = 2 * s.p_bytes;
  s.d_per = r256(static_cast<uint32_t>(rb) * (kDRowQ + 2 * kDRowSB));
  s.d = t;      t += static_cast<uint32_t>(k) * s.d_per;
  s.hs = t;     t += static_cast<uint32_t>(k + 1) * kSegI * kPad * 4;
  s.hsum = t;   t += r256(static_cast<uint32_t>(k + 1) * kSegI * 4);
  s.lg = t;     t += kMaxE * 4;
  s.cand = t;   t += kNW * kWave * 8;
  s.misc = t;   t += r256(kMWords * 4);
  s.part = t;   t += r256(static_cast<uint32_t>(k + 1) * rb * 4 + static_cast<uint32_t>(rb) * 2);
  s.total = t;
  return s;
}

typedef __attribute__((address_space(3))) uint32_t lds_w32;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) uint64_t lds_w64;
typedef __attribute__((address_space(3))) int64_t lds_i64;
typedef __attribute__((address_space(3))) uint16_t lds_w16;

__device__ __forceinline__ void store_tag(uint64_t* p, uint32_t bits, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct StackArgs {
  const uint8_t* x;          // layer l's input at x + l * x_stride (layer 0 only when chained)
  int64_t x_stride;
  const uint8_t* router;     // [E, H] bf16 per layer
  int64_t r_stride;
  const uint8_t* slots;      // int64 [E] per layer
  int64_t s_stride;
  const uint8_t* pool;
  int64_t pool_bytes;
  const uint8_t* shared;     // shared blob + gate vector per layer
  int64_t sh_stride;         // bytes between layers' shared buffers
  int64_t gv_off;            // gate vector offset inside one
  uint8_t* out;
  int64_t out_stride;
  uint8_t* x_chain;          // chained: x_chain + l * xc_stride = x_l + y_l (layer l + 1's input)
  int64_t xc_stride;
  int32_t* ids_out;          // optional [L][k]
  float* wts_out;            // optional [L][k]
  uint64_t* lg;              // [kLgRep][kMaxE] tagged logits
  uint64_t* hx;              // [kHRep][kMaxHn] tagged h rows (ranks 0..k-1, shared), then the gate
  uint64_t* xx;              // [kXRep][kH / 2] tagged next-layer input (two bf16 per word)
  uint32_t* flags;           // [3][kFlagRep][kMaxNb] per-block exchange flags
  uint32_t* ctrl;            // [0] error flags
  uint32_t* epochs;          // per-block call counters
  int L, E, k, nb, rpb, spb, rb, gpb, hn;
  int out_bf16;
  uint32_t spin_limit;
};

// Direct copies (global -> LDS, 16 or 4 bytes per lane) of `bytes` contiguous
// bytes at byte `src` of the buffer `rs` into `dst`.  Lane l of round j copies
// bytes [j W + l w, + w) (W = 64 w); a round that runs past `bytes` lands in
// the region's padding.
template <int W>
__device__ __forceinline__ void copy_lds(u32x4 rs, uint8_t* dst, uint32_t src, uint32_t bytes, int lane) {
  for (uint32_t j = 0; j < bytes; j += kWave * W)
    lds_load<W>(rs, dst + j, src + j + static_cast<uint32_t>(lane) * W, 0);
}

// The static operands of layer l (those that do not depend on its routing)
// into LDS copy `p`: its slot table, this block's router rows, shared
// gate/up rows and shared down rows, the gate vector (block 0) and, unless
// the input comes from the chain, x.  Issued by one wave; that wave waits for
// them (s_waitcnt vmcnt(0)) before the barrier that precedes their use.
__device__ __forceinline__ void issue_static(const StackArgs& a, const SLds& S, uint8_t* lds, int p, int l,
                                             int lane) {
  uint8_t* P = lds + p * S.p_bytes;
  const int b = blockIdx.x;
  // slot table
  copy_lds<16>(raw_rsrc(a.slots + l * a.s_stride, int64_t(a.E) * 8), P + S.p_slot, 0, a.E * 8, lane);
  // router rows
  {
    const u32x4 rs = raw_rsrc(a.router + l * a.r_stride, int64_t(a.E) * kH * 2);
    for (int j = 0; j < a.rpb; ++j) {
      const int e = b * a.rpb + j;
      if (e < a.E) copy_lds<16>(rs, P + S.p_rr + j * kH * 2, static_cast<uint32_t>(e) * kH * 2, kH * 2, lane);
    }
  }
  const uint8_t* sh = a.shared + l * a.sh_stride;
  const u32x4 rsh = raw_rsrc(sh, kBlob);
  // shared gate/up rows r = b * spb + j: gate codes then up codes per unit
  for (int j = 0; j < a.spb; ++j) {
    const int r = b * a.spb + j;
    if (r >= kI) continue;
    copy_lds<16>(rsh, P + S.p_suq + (2 * j) * kRowQ, static_cast<uint32_t>(r) * kRowQ, kRowQ, lane);
    copy_lds<16>(rsh, P + S.p_suq + (2 * j + 1) * kRowQ, static_cast<uint32_t>(kQ + r * kRowQ), kRowQ, lane);
  }
  // their scales and biases: [gate s, up s, gate b, up b][spb rows][32 groups] bf16
  {
    const uint32_t per = static_cast<uint32_t>(a.spb) * (kH / 64) * 2;   // bytes per plane
    const uint32_t base = static_cast<uint32_t>(b * a.spb) * (kH / 64) * 2;
    for (uint32_t j = 0; j < 4 * per; j += kWave * 4) {
      const uint32_t q = j + static_cast<uint32_t>(lane) * 4;
      const uint32_t plane = q / per, within = q - plane * per;
      const uint32_t poff = static_cast<uint32_t>(3 * kQ) + (plane < 2 ? plane : plane + 1) * static_cast<uint32_t>(kS);
      lds_load<4>(rsh, P + S.p_susb + j, poff + base + within, 0);
    }
  }
  // shared down rows [row_lo, row_lo + rb): codes, then [scales | biases]
  {
    const int row_lo = b * a.rb;
    copy_lds<16>(rsh, P + S.p_sdq, static_cast<uint32_t>(2 * kQ + row_lo * kDRowQ), a.rb * kDRowQ, lane);
    const uint32_t per = static_cast<uint32_t>(a.rb) * kDRowSB;
    for (uint32_t j = 0; j < 2 * per; j += kWave * 4) {
      const uint32_t q = j + static_cast<uint32_t>(lane) * 4;
      const uint32_t plane = q / per, within = q - plane * per;
      const uint32_t poff = static_cast<uint32_t>(3 * kQ + (plane == 0 ? 2 : 5) * kS);
      lds_load<4>(rsh, P + S.p_sdsb + j, poff + static_cast<uint32_t>(row_lo) * kDRowSB + within, 0);
    }
  }
  if (b == 0) copy_lds<16>(raw_rsrc(sh + a.gv_off, kH * 2), P + S.p_gv, 0, kH * 2, lane);
  if (l == 0 || a.x_chain == nullptr)
    copy_lds<16>(raw_rsrc(a.x + l * a.x_stride, kH * 2), P + S.p_x, 0, kH * 2, lane);
}

// The routed down operands of this block's rows: for rank i, rows
// [row_lo, row_lo + rb) of expert ids[i]'s down matrix (codes, scales,
// biases).  An unusable blob offset reads zeros.
__device__ __forceinline__ void issue_down(const StackArgs& a, const SLds& S, uint8_t* lds, int lane) {
  const lds_i64* roff = (const lds_i64*)(reinterpret_cast<lds_w32*>((lds_w32*)(lds + S.misc)) + kMOff);
  const int row_lo = blockIdx.x * a.rb;
  const uint32_t per = static_cast<uint32_t>(a.rb) * kDRowSB;
  for (int i = 0; i < a.k; ++i) {
    const int64_t off = roff[i];
    const bool ok = slot_ok(off, kBlob, a.pool_bytes);
    const u32x4 rs = raw_rsrc(a.pool + (ok ? off : 0), ok ? kBlob : 0);
    uint8_t* D = lds + S.d + i * S.d_per;
    copy_lds<16>(rs, D, static_cast<uint32_t>(2 * kQ + row_lo * kDRowQ), a.rb * kDRowQ, lane);
    for (uint32_t j = 0; j < 2 * per; j += kWave * 4) {
      const uint32_t q = j + static_cast<uint32_t>(lane) * 4;
      const uint32_t plane = q / per, within = q - plane * per;
      const uint32_t poff = static_cast<uint32_t>(3 * kQ + (plane == 0 ? 2 : 5) * kS);
      lds_load<4>(rs, D + a.rb * kDRowQ + j, poff + static_cast<uint32_t>(row_lo) * kDRowSB + within, 0);
    }
  }
}

// Exchanges.  A producer block stores its words (value bits and the layer's
// tag), then, once every wave of the block has issued them (the caller's
// barrier), raises its flag: the tag in every copy of the block's flag word.
// A reader polls the flags of all blocks with one wave (1 KB per try), then
// reads the words once; a flag may be seen before the words it follows, so a
// word with an older tag is read again.  Polling the flags instead of the
// words keeps the traffic of waiting blocks small while the other blocks
// still stream their operands.  Every wait is bounded.
__device__ __forceinline__ void raise_flag(const StackArgs& a, int kind, uint32_t tag, int wave, int lane) {
  if (wave == 0 && lane < kFlagRep)
    __hip_atomic_store(a.flags + (kind * kFlagRep + lane) * kMaxNb + blockIdx.x, tag, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// True once every block's flag of `kind` carries `tag`; false on expiry (or
// when an earlier wait expired).
__device__ __forceinline__ bool wait_flags(const StackArgs& a, int kind, uint32_t tag, bool dead, lds_w32* misc,
                                           int wave, int lane) {
  if (wave == 0) {
    bool ok = !dead;
    if (ok) {
      const uint32_t* r = a.flags + (kind * kFlagRep + blockIdx.x % kFlagRep) * kMaxNb;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(r), 0, kMaxNb * 4, 0x00020000);
      for (uint32_t spins = 0;; ++spins) {
        bool all = true;
        for (int j = lane * 4; j < a.nb; j += kWave * 4) {   // scope of device (sc1)
          const u32x4 f = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, j * 4, 0, 16));
#pragma unroll
          for (int q = 0; q < 4; ++q) all = all && (j + q >= a.nb || f[q] == tag);
        }
        if (__ballot(!all) == 0) break;
        if (spins >= a.spin_limit) { ok = false; break; }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (lane == 0) misc[kMOk] = ok ? 1u : 0u;
  }
  __syncthreads();
  return misc[kMOk] != 0u;
}

// The n tagged words at `src` (thread t of the first nthr takes words
// t + q nthr, q < PER), read until each carries `tag`; put(i, bits) stores
// word i's value.  Run by the reading waves only, under a branch on the wave
// index, with no barrier inside: the copy waves, whose direct loads are still
// in flight, must never execute the wait that follows these loads.  False on
// expiry.
template <int PER, typename F>
__device__ __forceinline__ bool read_tagged(const uint64_t* src, int n, int nthr, uint32_t tag, uint32_t limit,
                                            F&& put) {
  const int tid = threadIdx.x;
  uint32_t need = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (tid + q * nthr < n) need |= 1u << q;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(src), 0, n * 8, 0x00020000);
  for (uint32_t spins = 0;; ++spins) {
    uint64_t w[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q)   // scope of device (sc1): past this XCD's L2, where the writers' stores went
      w[q] = (need >> q) & 1u
                 ? __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rs, (tid + q * nthr) * 8, 0, 16))
                 : 0ull;
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

// After a barrier: true if every reading wave's read succeeded.
__device__ __forceinline__ bool reads_ok(const lds_w32* misc) {
  bool ok = true;
#pragma unroll
  for (int w = 0; w < kRdWaves; ++w) ok = ok && misc[kMRd + w] != 0u;
  return ok;
}

template <int OUT>
__global__ __launch_bounds__(kThr) void k_decode_stack(StackArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SLds S = stack_lds(a.E, a.k, a.rpb, a.spb, a.rb);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x;
  const int E = a.E, k = a.k;
  lds_w32* misc = (lds_w32*)(lds + S.misc);
  float* const lg = reinterpret_cast<float*>(lds + S.lg);
  const uint32_t epoch = a.epochs[b];
  bool dead = false;
  bool bad = false;   // a routed blob offset was unusable (its pair contributes nothing)

  if (wave == kWaveStatic) {
    issue_static(a, S, lds, 0, 0, lane);
    wait_vm0();
  }
  __syncthreads();

  for (int l = 0; l < a.L; ++l) {
    const uint32_t tag = epoch + 1u + static_cast<uint32_t>(l);
    const int p = l & 1;
    uint8_t* P = lds + p * S.p_bytes;
    const uint8_t* xl = P + S.p_x;                           // this layer's input (bf16)

    // ------------------------------------------------------------------ R
    // per lane: its 32-value segment of x (lane = segment for H = 2048)
    ActRaw<kBF16> xr;
    load_lds_act_bf16(xl, lane, xr);
    const float xs = xsum_bf16(xr);
    for (int j = wave; j < a.rpb + a.spb; j += kNW) {
      if (j < a.rpb) {
        const int e = b * a.rpb + j;
        if (e >= E) continue;
        float v[kSegCodes], r[kSegCodes];
        act_raw_f32<kBF16>(xr, v);
        ActRaw<kBF16> rw;
        load_lds_act_bf16(P + S.p_rr + j * kH * 2, lane, rw);
        act_raw_f32<kBF16>(rw, r);
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < kSegCodes; ++c) acc = fmaf(v[c], r[c], acc);
        acc = group_sum(acc, kWave);
        if (lane < kLgRep) store_tag(a.lg + static_cast<size_t>(lane) * kMaxE + e, __float_as_uint(acc), tag);
      } else {
        const int u = j - a.rpb;
        const int r = b * a.spb + u;
        if (r >= kI) continue;
        Seg<4> cg, cu;
        cg.w[0] = *(const lds_u32x4*)((const lds_u8*)(P + S.p_suq + (2 * u) * kRowQ) + 16 * lane);
        cu.w[0] = *(const lds_u32x4*)((const lds_u8*)(P + S.p_suq + (2 * u + 1) * kRowQ) + 16 * lane);
        const uint32_t per = static_cast<uint32_t>(a.spb) * (kH / 64);   // bf16 values per plane
        const lds_w16* sb = (const lds_w16*)(P + S.p_susb);
        const int gi = u * (kH / 64) + lane / 2;
        const float sg = bf16_to_f32(sb[gi]), su = bf16_to_f32(sb[per + gi]);
        const float bg = bf16_to_f32(sb[2 * per + gi]), bu = bf16_to_f32(sb[3 * per + gi]);
        const QPairs pg = qpairs_bf16(cg), pu = qpairs_bf16(cu);
        float accg = 0.f, accu = 0.f;
        accg += seg_value_d2(sg, bg, dot2_seg(pg, xr), xs);
        accu += seg_value_d2(su, bu, dot2_seg(pu, xr), xs);
        float g, uu;
        gu_sums_w<kWave>(accg, accu, kWave, g, uu);
        const float h = silu(g) * uu;
        if (lane < kHRep) store_tag(a.hx + static_cast<size_t>(lane) * kMaxHn + k * kI + r, __float_as_uint(h), tag);
      }
    }
    if (b == 0 && wave == kNW - 1) {
      // sigmoid(g . x), as the staged path forms it
      float acc = 0.f;
      {
        float xv[kSegCodes], gv[kSegCodes];
        act_raw_f32<kBF16>(xr, xv);
        ActRaw<kBF16> gw;
        load_lds_act_bf16(P + S.p_gv, lane, gw);
        act_raw_f32<kBF16>(gw, gv);
#pragma unroll
        for (int c = 0; c < kSegCodes; ++c) acc = fmaf(xv[c], gv[c], acc);
      }
      acc = group_sum(acc, kWave);
      const float sgm = sigmoid(acc);
      if (lane < kHRep) store_tag(a.hx + static_cast<size_t>(lane) * kMaxHn + (k + 1) * kI, __float_as_uint(sgm), tag);
    }

    // ------------------------------------------------------------------ K
    __syncthreads();                 // every wave's logit stores are issued
    raise_flag(a, kFlLg, tag, wave, lane);
    {
      bool ok = wait_flags(a, kFlLg, tag, dead, misc, wave, lane);
      if (ok && wave < kRdWaves) {
        const bool r = read_tagged<(kMaxE + kRdThr - 1) / kRdThr>(
            a.lg + static_cast<size_t>(b % kLgRep) * kMaxE, E, kRdThr, tag, a.spin_limit,
            [&](int i, uint32_t bits) { ((lds_f32*)(lg))[i] = __uint_as_float(bits); });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok(misc));
    }
    // top-k on wave 0 (the staged kernels' wave top-k: a bound from the lane
    // maxima, the candidates above it ranked exactly, the weights in rank
    // order), then the chosen experts' blob offsets; one barrier for all
    if (wave == 0) {
      topk_wave_n<8>(lg, E, k, lane, reinterpret_cast<uint64_t*>(lds + S.cand),
                     reinterpret_cast<int32_t*>(reinterpret_cast<uint32_t*>(lds + S.misc) + kMIds),
                     reinterpret_cast<float*>(reinterpret_cast<uint32_t*>(lds + S.misc) + kMVals));
      const lds_i64* slot = (const lds_i64*)(P + S.p_slot);
      if (lane < k) {
        const int e = static_cast<int>(misc[kMIds + lane]);
        ((lds_i64*)(misc + kMOff))[lane] = slot[e];
        if (b == 0) {
          if (a.ids_out) a.ids_out[static_cast<size_t>(l) * k + lane] = e;
          if (a.wts_out) a.wts_out[static_cast<size_t>(l) * k + lane] = __uint_as_float(misc[kMVals + lane]);
        }
      }
    }
    __syncthreads();

    // ------------------------------------------------------------------ G
    {
      const int g0 = b * a.gpb;
      const int g1 = min(g0 + a.gpb, k * kI);
      const lds_i64* roff = (const lds_i64*)(misc + kMOff);
      Seg<4> cg[kMaxG], cu[kMaxG];
      uint32_t sg[kMaxG], su[kMaxG], bg[kMaxG], bu[kMaxG];
      bool live[kMaxG], vv[kMaxG];
      int ii[kMaxG], rr[kMaxG];
      if (wave < kGW) {
#pragma unroll
        for (int j = 0; j < kMaxG; ++j) {
          const int u0 = g0 + wave + kGW * j;
          live[j] = u0 < g1;
          const int u = live[j] ? u0 : g0;
          ii[j] = u / kI;
          rr[j] = u % kI;
          const int64_t off0 = roff[ii[j]];
          const int64_t off = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off0 >> 32))) << 32) |
                              static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off0)));
          vv[j] = slot_ok(off, kBlob, a.pool_bytes);
          if (live[j] && !vv[j]) bad = true;
          // one descriptor over the blob (an unusable one reads zeros); the
          // plane offsets go in the scalar offset, the lane's in the vector one
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<uint8_t*>(a.pool + (vv[j] ? off : 0)), 0, vv[j] ? static_cast<int>(kBlob) : 0, 0x00020000);
          const int qo = rr[j] * kRowQ + 16 * lane;
          cg[j].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qo, 0, 2));
          cu[j].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qo, kQ, 2));
          const int si = (rr[j] * (kH / 64) + lane / 2) * 2;
          sg[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ, 0);
          su[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + kS, 0);
          bg[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 3 * kS, 0);
          bu[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 4 * kS, 0);
        }
      }
      __syncthreads();   // the down copies start after every phase-G load is requested
      if (wave < kGW) {
#pragma unroll
        for (int j = 0; j < kMaxG; ++j) {
          if (!live[j]) continue;
          const QPairs pg = qpairs_bf16(cg[j]), pu = qpairs_bf16(cu[j]);
          float accg = 0.f, accu = 0.f;
          accg += seg_value_d2(raw_value<kBF16>(sg[j]), raw_value<kBF16>(bg[j]), dot2_seg(pg, xr), xs);
          accu += seg_value_d2(raw_value<kBF16>(su[j]), raw_value<kBF16>(bu[j]), dot2_seg(pu, xr), xs);
          float g, uu;
          gu_sums_w<kWave>(accg, accu, kWave, g, uu);
          const float h = vv[j] ? silu(g) * uu : 0.f;
          if (lane < kHRep)
            store_tag(a.hx + static_cast<size_t>(lane) * kMaxHn + ii[j] * kI + rr[j], __float_as_uint(h), tag);
        }
      } else if (wave == kWaveDown) {
        issue_down(a, S, lds, lane);
      } else if (wave == kWaveStatic && l + 1 < a.L) {
        // the next layer's static operands: into the other copy, free since
        // the layer before this one ended
        issue_static(a, S, lds, p ^ 1, l + 1, lane);
      }
    }

    // ------------------------------------------------------------------ H
    __syncthreads();                 // every wave's h stores are issued
    raise_flag(a, kFlH, tag, wave, lane);
    if (wave == kWaveDown) wait_vm0();
    {
      float* hs = reinterpret_cast<float*>(lds + S.hs);
      const int nh = (k + 1) * kI + 1;
      // waves 0..5 read (wave 6 still has the static copies in flight)
      bool ok = wait_flags(a, kFlH, tag, dead, misc, wave, lane);
      if (ok && wave < kRdWaves) {
        const bool r = read_tagged<(kMaxHn + kRdThr - 1) / kRdThr>(
            a.hx + static_cast<size_t>(b % kHRep) * kMaxHn, nh, kRdThr, tag, a.spin_limit, [&](int i, uint32_t bits) {
              if (i < (k + 1) * kI) {
                const int row = i / kI, c = i % kI;
                ((lds_f32*)(hs))[(row * kSegI + c / kSegCodes) * kPad + c % kSegCodes] = __uint_as_float(bits);
              } else {
                misc[kMSig] = bits;
              }
            });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok(misc));
      // segment sums of the staged rows, in the order seg_sum uses
      float* hsum = reinterpret_cast<float*>(lds + S.hsum);
      for (int j = tid; j < (k + 1) * kSegI; j += kThr) {
        float v[kSegCodes];
        load_lds_seg(hs + static_cast<size_t>(j) * kPad, 0, v);
        ((lds_f32*)(hsum))[j] = seg_sum(v);
      }
      __syncthreads();
    }

    // ------------------------------------------------------------------ D
    {
      const int row_lo = b * a.rb;
      const int npass = a.rb / kRpp;
      const int ntask = (k + 1) * npass;
      const int sub = lane / kSegI, seg = lane % kSegI;
      const lds_i64* roff = (const lds_i64*)(misc + kMOff);
      const float* hs = reinterpret_cast<const float*>(lds + S.hs);
      const float* hsum = reinterpret_cast<const float*>(lds + S.hsum);
      float* part = reinterpret_cast<float*>(lds + S.part);
      for (int t = wave; t < ntask; t += kNW) {
        const int i = t / npass, pp = t % npass;
        const int rloc = pp * kRpp + sub;
        const uint8_t* base = i < k ? lds + S.d + i * S.d_per : nullptr;
        const uint8_t* q8 = i < k ? base : P + S.p_sdq;
        const uint8_t* sb8 = i < k ? base + a.rb * kDRowQ : P + S.p_sdsb;
        Seg<4> code;
        code.w[0] = *(const lds_u32x4*)((const lds_u8*)(q8) + rloc * kDRowQ + 16 * seg);
        const lds_w16* sbw = (const lds_w16*)(sb8);
        const int gi = rloc * (kI / 64) + seg / 2;
        const float sc = bf16_to_f32(sbw[gi]);
        const float bi = bf16_to_f32(sbw[a.rb * (kI / 64) + gi]);
        float hv[1][kSegCodes];
        load_lds_seg(hs + (static_cast<size_t>(i) * kSegI + seg) * kPad, 0, hv[0]);
        const float hsv = ((const lds_f32*)(hsum))[i * kSegI + seg];
        float qv[1];
        seg_qdot_nt<4, 1>(code, hv, qv);
        float acc = 0.f;
        acc += seg_value(sc, bi, qv[0], hsv);
        const float v = group_sum(acc, kSegI);
        const bool valid = i == k || slot_ok(roff[i], kBlob, a.pool_bytes);
        if (seg == 0) ((lds_f32*)(part))[i * a.rb + rloc] = valid ? v : 0.f;
      }
      __syncthreads();
      // ordered combine: ranks ascending, then the gated shared expert
      const float sgm = __uint_as_float(misc[kMSig]);
      if (tid < a.rb && row_lo + tid < kH) {
        const int n = row_lo + tid;
        float acc = 0.f;
        for (int i = 0; i < k; ++i)
          acc = fmaf(__uint_as_float(misc[kMVals + i]), ((const lds_f32*)(part))[i * a.rb + tid], acc);
        acc = fmaf(sgm, ((const lds_f32*)(part))[k * a.rb + tid], acc);
        uint8_t* o = a.out + l * a.out_stride;
        if constexpr (OUT == kF32) reinterpret_cast<float*>(o)[n] = acc;
        else reinterpret_cast<uint16_t*>(o)[n] = f32_to_bf16(acc);
        if (a.x_chain) {
          // the stack step x + y: fp32 sum, nearest-even bf16
          const float xv = bf16_to_f32(((const lds_w16*)(xl))[n]);
          const uint16_t xn = f32_to_bf16(xv + acc);
          reinterpret_cast<uint16_t*>(a.x_chain + l * a.xc_stride)[n] = xn;
          ((lds_w16*)(lds + S.part))[(k + 1) * a.rb * 2 + tid] = xn;   // staged for the tagged words
        }
      }
    }

    // ------------------------------------------------------------------ next input
    if (a.x_chain && l + 1 < a.L) {
      __syncthreads();
      const uint32_t ntag = tag + 1u;    // the next layer's tag marks its input
      const int row_lo = b * a.rb;
      const lds_w16* xn = (const lds_w16*)(lds + S.part) + (k + 1) * a.rb * 2;
      const int nw = a.rb / 2;
      if (tid < nw * kXRep) {
        const int w = tid % nw, rep = tid / nw;
        const uint32_t bits = static_cast<uint32_t>(xn[2 * w]) | (static_cast<uint32_t>(xn[2 * w + 1]) << 16);
        store_tag(a.xx + static_cast<size_t>(rep) * (kH / 2) + row_lo / 2 + w, bits, ntag);
      }
      __syncthreads();               // every x store is issued
      raise_flag(a, kFlX, ntag, wave, lane);
      lds_w32* xd = (lds_w32*)(lds + (p ^ 1) * S.p_bytes + S.p_x);
      bool ok = wait_flags(a, kFlX, ntag, dead, misc, wave, lane);
      if (ok && wave < kRdWaves) {
        const bool r = read_tagged<(kH / 2 + kRdThr - 1) / kRdThr>(
            a.xx + static_cast<size_t>(b % kXRep) * (kH / 2), kH / 2, kRdThr, ntag, a.spin_limit,
            [&](int i, uint32_t bits) { xd[i] = bits; });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok(misc));
    }
    if (wave == kWaveStatic) wait_vm0();
    __syncthreads();
  }

  if (bad && lane == 0) raise_error(a.ctrl, kErrRange);
  if (dead && tid == 0) raise_error(a.ctrl, kErrTimeout);
  // every block read its counter at its start; advance them (the ones past
  // the grid by block 0), so that all counters stay equal
  if (tid == 0) a.epochs[b] = epoch + static_cast<uint32_t>(a.L);
  if (b == 0)
    for (int j = a.nb + tid; j < kFusedMaxBlocks; j += kThr) a.epochs[j] = a.epochs[j] + static_cast<uint32_t>(a.L);
}

}  // namespace

bool stack_supported(const moe_desc& d) {
  return d.hidden == kH && d.inter == kI && d.shared_inter == kI && d.bits == 4 && d.act_dtype == kBF16 &&
         d.sb_dtype == kBF16 && d.n_experts <= kMaxE && d.top_k <= kMaxK;
}

size_t stack_ws_lg() { return static_cast<size_t>(kLgRep) * kMaxE * 8; }
size_t stack_ws_h() { return static_cast<size_t>(kHRep) * kMaxHn * 8; }
size_t stack_ws_x() { return static_cast<size_t>(kXRep) * (kH / 2) * 8; }
size_t stack_ws_flags() { return static_cast<size_t>(3) * kFlagRep * kMaxNb * 4; }

// Grid and LDS of the stack kernel on the current device: one block per CU,
// each CU's share of rows an exact multiple of a down pass.
int stack_plan(const moe_desc& d, StackPlan* plan) {
  int dev = 0, cus = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ENODEV;
  if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return MOE_ENODEV;
  const int nb = cus;
  if (nb < 1 || nb > kMaxNb || kH % nb) return MOE_EINVAL;
  const int rb = kH / nb;
  const int rpb = (d.n_experts + nb - 1) / nb, spb = (kI + nb - 1) / nb;
  const int gpb = (d.top_k * kI + nb - 1) / nb;
  if (rb % kRpp || rb > kMaxRb || rpb > kMaxRpb || spb > kMaxSpb || gpb > kGW * kMaxG || rpb + spb > kNW - 1)
    return MOE_EINVAL;
  const SLds S = stack_lds(d.n_experts, d.top_k, rpb, spb, rb);
  if (S.total > static_cast<uint32_t>(lds_max)) return MOE_EINVAL;
  const void* fn = d.out_dtype == kF32 ? reinterpret_cast<const void*>(k_decode_stack<kF32>)
                                       : reinterpret_cast<const void*>(k_decode_stack<kBF16>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(S.total)) != hipSuccess)
    return MOE_EHIP;
  int fit = 0;
  const hipError_t e = d.out_dtype == kF32
                           ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, k_decode_stack<kF32>, kThr, S.total)
                           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, k_decode_stack<kBF16>, kThr, S.total);
  if (e != hipSuccess) return MOE_EHIP;
  if (fit < 1) return MOE_EINVAL;
  plan->nb = nb;
  plan->rb = rb;
  plan->rpb = rpb;
  plan->spb = spb;
  plan->gpb = gpb;
  plan->lds = S.total;
  return MOE_OK;
}

int launch_decode_stack(const StackCall& c, const StackPlan& plan) {
  const moe_desc& d = c.d;
  StackArgs a;
  a.x = static_cast<const uint8_t*>(c.x);
  a.x_stride = c.x_stride;
  a.router = static_cast<const uint8_t*>(c.router_w);
  a.r_stride = c.router_stride;
  a.slots = reinterpret_cast<const uint8_t*>(c.slot_table);
  a.s_stride = c.slot_stride;
  a.pool = c.pool;
  a.pool_bytes = d.pool_bytes;
  a.shared = c.shared;
  a.sh_stride = c.shared_stride;
  a.gv_off = d.shared_stride;
  a.out = static_cast<uint8_t*>(c.out);
  a.out_stride = c.out_stride;
  a.x_chain = static_cast<uint8_t*>(c.x_chain);
  a.xc_stride = c.chain_stride;
  a.ids_out = c.ids_out;
  a.wts_out = c.wts_out;
  a.lg = reinterpret_cast<uint64_t*>(c.ws + c.L.s_lg);
  a.hx = reinterpret_cast<uint64_t*>(c.ws + c.L.s_h);
  a.xx = reinterpret_cast<uint64_t*>(c.ws + c.L.s_x);
  a.flags = reinterpret_cast<uint32_t*>(c.ws + c.L.s_flags);
  a.ctrl = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  a.epochs = reinterpret_cast<uint32_t*>(c.ws + c.L.f_epoch);
  a.L = c.n_layers;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.nb = plan.nb;
  a.rpb = plan.rpb;
  a.spb = plan.spb;
  a.rb = plan.rb;
  a.gpb = plan.gpb;
  a.hn = (d.top_k + 1) * kI + 1;
  a.out_bf16 = d.out_dtype == kBF16;
  a.spin_limit = 1u << 21;
  if (d.out_dtype == kF32)
    launch_kernel(k_decode_stack<kF32>, dim3(plan.nb), dim3(kThr), plan.lds, c.stream, a);
  else
    launch_kernel(k_decode_stack<kBF16>, dim3(plan.nb), dim3(kThr), plan.lds, c.stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
