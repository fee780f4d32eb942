// Persistent decode of a stack of MoE layers, one token per layer (gfx950).
//
// One launch runs L layers in order on a grid of 256 resident 512-thread
// blocks (one per CU).  The blocks form eight groups of 32 (block b is in
// group b % 8; the dispatcher sends block b to XCD b % 8, so a group is one
// XCD).  The work of a layer is divided so that every block has the same
// share and most exchanges stay inside a group:
//   * whole units: routed rank r < 8 lives in group r (its 512 gate/up row
//     pairs, 16 per block, and its 2048 down rows, 64 per block);
//   * split units: ranks 8 and 9 (k = 10) each live in four groups (0..3 and
//     4..7): 4 row pairs and 16 down rows per block;
//   * the shared expert: its gate/up rows in phase R on every block (two per
//     block, from LDS), its down rows 8 per block.
// Per layer:
//   R  two router rows and two shared gate/up rows per block, from LDS
//      (copied there while the previous layer ran); block 0 also sigma(g . x);
//      meanwhile one wave requests the next layer's static operands into the
//      other LDS copy
//   K  every block reads the E logits and takes top-k and the renormalised
//      weights itself (one wave)
//   G  the block's gate/up row pairs of its whole and split unit, every load
//      of a wave requested at once; meanwhile one wave copies the block's
//      down rows of its three units into LDS
//   H  h of the whole unit (from the group), the split unit (from its four
//      groups) and the shared expert (from R)
//   D  the block's 88 down rows, stored as row sums per unit
// The ordered combine (ranks ascending, then sigma times the shared unit)
// reads every unit's row sums: unchained, block b finishes rows 8b..8b+7 of
// layer l while the next layer's top-k runs (the last layer at the end);
// chained, every group finishes all rows and exchanges the next input within
// the group.
//
// Blocks exchange data only through tagged 64-bit words: the value's bits and
// the layer's tag, written with relaxed device-scope stores and read with
// device-scope loads, each word read again (after a short sleep) until it
// carries the tag; no flags.  Reading a block's word of layer l orders
// everything that block did before writing it, and every block writes logit
// words in phase R (E is a multiple of 256), so a block that has read the
// logits of layer l + 1 knows every block has finished layer l's reads.
// Regions written before that point and read after it (the logits, the
// shared h, the row sums) alternate between two copies by layer parity.
// Every wait is bounded; on expiry the kernel raises kErrTimeout and skips
// all later waits, so the grid always drains.
//
// Work inside a layer needs every block resident at once (checked with the
// occupancy query when the plan is made).
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
#include "stack_common.h"
#include "topk_wave.h"

namespace moe {

namespace {

constexpr int kH = 2048;                   // hidden size this kernel is built for
constexpr int kI = 512;                    // routed and shared intermediate size
constexpr int kThr = 512;
constexpr int kNW = kThr / kWave;          // 8 waves per block
constexpr int kNG = 8;                     // block groups (block b in group b % 8)
constexpr int kNM = 32;                    // blocks per group
constexpr int kNB = kNG * kNM;             // blocks in the grid
constexpr int kQuads = 2;                  // ranks 8 and 9: split units, over groups 0..3 and 4..7
constexpr int kQG = kNG / kQuads;          // groups per split unit (4)
constexpr int kHPM = kI / kNM;             // gate/up row pairs of a whole unit per block (16)
constexpr int kDPM = kH / kNM;             // down rows of a whole unit per block (64)
constexpr int kSHP = kI / (kQG * kNM);     // gate/up row pairs of a split unit per block (4)
constexpr int kSDR = kH / (kQG * kNM);     // down rows of a split unit per block (16)
constexpr int kFR = kH / kNB;              // shared down rows per block, and output rows a block
                                           // finishes when unchained (8)
constexpr int kGA = 4;                     // waves 0..3 compute phase G
constexpr int kPW = kHPM / kGA;            // whole-unit pairs per phase-G wave (4), plus one split pair
constexpr int kWaveStatic = 6;             // copies the next layer's static operands
constexpr int kWaveDown = 7;               // copies the down operands
constexpr int kWaveFin = 1;                // finishes the previous layer's rows (unchained)
constexpr int kSegI = kI / kSegCodes;      // 16 segments per down row
constexpr int kRpp = kWave / kSegI;        // 4 down rows per wave pass
constexpr int kPad = kSegCodes + 4;        // staged h: floats per segment (bank spread)
constexpr int64_t kQ = int64_t(kH) * kI / 2;        // code bytes of one matrix
constexpr int64_t kS = int64_t(kH) * (kI / 64) * 2; // bf16 scale bytes of one matrix
constexpr int64_t kBlob = 3 * kQ + 6 * kS;
constexpr int kRowQ = kH / 2;              // code bytes of a gate/up row
constexpr int kDRowQ = kI / 2;             // code bytes of a down row
constexpr int kDRowSB = (kI / 64) * 2;     // scale (or bias) bytes of a down row
constexpr uint32_t kDRowB = kDRowQ + 2 * kDRowSB;   // LDS bytes of one staged down row
constexpr int kLgRep = 8;                  // copies of the exchanged logits
constexpr int kMaxK = 10, kMaxRpb = 2, kSpb = kI / kNB, kMaxE = kNB * kMaxRpb;
constexpr int kTopC = 16;                  // top-k candidates each wave keeps
constexpr int kRdWaves = 6;                // waves that read exchanged words (0..5)
constexpr int kRdThr = kRdWaves * kWave;
constexpr int kSigW = (kMaxK + 1) * kH;    // sigma's word in a row-sum copy
constexpr int kPartW = kSigW + 64;         // words of one row-sum copy
static_assert(kSpb == 2 && kSHP == kGA && kPW % 2 == 0 && kMaxK <= kNG + kQuads && kFR == 8, "grid shape");

// Exchange regions (word offsets into the one tagged-word buffer).
constexpr size_t kXLg = 0;                                      // [2][kLgRep][kMaxE] logits
constexpr size_t kXSh = kXLg + size_t(2) * kLgRep * kMaxE;      // [2][kI] shared h
constexpr size_t kXHx = kXSh + size_t(2) * kI;                  // [kNG][kI] h of each group's whole unit
constexpr size_t kXHq = kXHx + size_t(kNG) * kI;                // [kQuads][kI] h of the split units
constexpr size_t kXPart = kXHq + size_t(kQuads) * kI;           // [2][kPartW] row sums by unit, then sigma
constexpr size_t kXWords = kXPart + size_t(2) * kPartW;

// Bytes of LDS per region, rounded so that 256-byte direct-load rounds that
// run past a region's end land in its own padding.
__host__ __device__ constexpr uint32_t r256(uint32_t n) { return (n + 255u) / 256u * 256u; }

struct SLds {
  // static operands of one layer (two copies, by layer parity)
  uint32_t p_x, p_rr, p_suq, p_susb, p_slot, p_gv, p_bytes;
  uint32_t d[3];   // down rows of the whole, split and shared unit: codes [n][256 B], scales [n][16 B],
                   // biases [n][16 B] (n = 64, 16, 8)
  uint32_t hs;     // [3][kSegI][kPad] floats: h of the whole, split and shared unit
  uint32_t hsum;   // [3][kSegI] floats: the segment sums of hs
  uint32_t lg;     // [kMaxE] logits
  uint32_t cand;   // [8 waves][16] top-k candidates
  uint32_t misc;   // see below
  uint32_t fin;    // [kMaxK + 1][kDPM] row sums being combined, then sigma
  uint32_t xn;     // [kDPM] bf16 next-layer input rows (chained)
  uint32_t total;
};

// misc words (32-bit each)
constexpr int kMIds = 0;               // [kMaxK] chosen experts by rank
constexpr int kMVals = 16;             // [2][kMaxK] chosen logits, then weights, by layer parity
constexpr int kMSig = kMVals + 2 * kMaxK;   // sigmoid(g . x) of this layer (block 0)
constexpr int kMFin = kMSig + 1;       // result of the finishing wave's reads
constexpr int kMRd = kMFin + 1;        // [kRdWaves] results of the reading waves
constexpr int kMOff = 64;              // [kMaxK] int64 blob offsets by rank (8-byte aligned)
constexpr int kMWords = kMOff + 2 * kMaxK;

__host__ __device__ inline SLds stack_lds(int E, int rpb) {
  SLds s{};
  uint32_t o = 0;
  s.p_x = o;    o += r256(kH * 2);
  s.p_rr = o;   o += r256(static_cast<uint32_t>(rpb) * kH * 2);
  s.p_suq = o;  o += r256(kSpb * 2 * kRowQ);
  s.p_susb = o; o += r256(kSpb * 4 * (kH / 64) * 2);
  s.p_slot = o; o += r256(static_cast<uint32_t>(E) * 8);
  s.p_gv = o;   o += r256(kH * 2);
  s.p_bytes = o;
  uint32_t t = 2 * s.p_bytes;
  s.d[0] = t;   t += kDPM * kDRowB;
  s.d[1] = t;   t += kSDR * kDRowB;
  s.d[2] = t;   t += kFR * kDRowB;
  s.hs = t;     t += 3 * kSegI * kPad * 4;
  s.hsum = t;   t += r256(3 * kSegI * 4);
  s.lg = t;     t += kMaxE * 4;
  s.cand = t;   t += kNW * kTopC * 8;
  s.misc = t;   t += r256(kMWords * 4);
  s.fin = t;    t += r256(((kMaxK + 1) * kDPM + 1) * 4);
  s.xn = t;     t += r256(kDPM * 2);
  s.total = t;
  return s;
}

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
  uint64_t* xw;              // tagged words, regions at kX*
  uint64_t* xx;              // [kNG][kH / 2] tagged next-layer input of each group (two bf16 per word)
  uint32_t* ctrl;            // [0] error flags
  uint32_t* epochs;          // per-block call counters
  int L, E, k, rpb;
  uint32_t spin_limit;
};

// n down rows from row r0 of the blob behind `rs` into LDS at D: codes
// [n][256 B], then scales [n][16 B] and biases [n][16 B] (4-byte direct loads,
// 256 bytes a round: n * 32 bytes is a whole number of rounds).
__device__ __forceinline__ void copy_down_rows(u32x4 rs, uint8_t* D, int r0, int n, int lane) {
  copy_lds<16>(rs, D, static_cast<uint32_t>(2 * kQ + r0 * kDRowQ), n * kDRowQ, lane);
  const uint32_t per = static_cast<uint32_t>(n) * kDRowSB;
  for (uint32_t j = 0; j < 2 * per; j += kWave * 4) {
    const uint32_t q = j + static_cast<uint32_t>(lane) * 4;
    const uint32_t plane = q / per, within = q - plane * per;
    const uint32_t poff = static_cast<uint32_t>(3 * kQ + (plane == 0 ? 2 : 5) * kS);
    lds_load<4>(rs, D + n * kDRowQ + j, poff + static_cast<uint32_t>(r0) * kDRowSB + within, 0);
  }
}

// The static operands of layer l (those that do not depend on its routing)
// into LDS copy `p`: its slot table, this block's router rows and shared
// gate/up rows, the gate vector (block 0) and, unless the input comes from
// the chain, x.  Direct-to-LDS loads: cheap to request, slow to
// land (few in flight per CU), so one wave requests them a layer ahead and
// waits for them (s_waitcnt vmcnt(0)) only at the end of the layer.
__device__ __forceinline__ void issue_static(const StackArgs& a, const SLds& S, uint8_t* lds, int p, int l,
                                             int lane) {
  uint8_t* P = lds + p * S.p_bytes;
  const int b = blockIdx.x;
  copy_lds<16>(raw_rsrc(a.slots + l * a.s_stride, int64_t(a.E) * 8), P + S.p_slot, 0, a.E * 8, lane);
  {
    const u32x4 rs = raw_rsrc(a.router + l * a.r_stride, int64_t(a.E) * kH * 2);
    for (int j = 0; j < a.rpb; ++j) {
      const int e = b * a.rpb + j;
      if (e < a.E) copy_lds<16>(rs, P + S.p_rr + j * kH * 2, static_cast<uint32_t>(e) * kH * 2, kH * 2, lane);
    }
  }
  const uint8_t* sh = a.shared + l * a.sh_stride;
  const u32x4 rsh = raw_rsrc(sh, kBlob);
  // shared gate/up rows r = b * kSpb + j: gate codes then up codes per unit
  for (int j = 0; j < kSpb; ++j) {
    const int r = b * kSpb + j;
    copy_lds<16>(rsh, P + S.p_suq + (2 * j) * kRowQ, static_cast<uint32_t>(r) * kRowQ, kRowQ, lane);
    copy_lds<16>(rsh, P + S.p_suq + (2 * j + 1) * kRowQ, static_cast<uint32_t>(kQ + r * kRowQ), kRowQ, lane);
  }
  // their scales and biases: [gate s, up s, gate b, up b][kSpb rows][32 groups] bf16
  {
    constexpr uint32_t per = kSpb * (kH / 64) * 2;   // bytes per plane
    const uint32_t base = static_cast<uint32_t>(b * kSpb) * (kH / 64) * 2;
    for (uint32_t j = 0; j < 4 * per; j += kWave * 4) {
      const uint32_t q = j + static_cast<uint32_t>(lane) * 4;
      const uint32_t plane = q / per, within = q - plane * per;
      const uint32_t poff = static_cast<uint32_t>(3 * kQ) + (plane < 2 ? plane : plane + 1) * static_cast<uint32_t>(kS);
      lds_load<4>(rsh, P + S.p_susb + j, poff + base + within, 0);
    }
  }
  if (b == 0) copy_lds<16>(raw_rsrc(sh + a.gv_off, kH * 2), P + S.p_gv, 0, kH * 2, lane);
  if (l == 0 || a.x_chain == nullptr)
    copy_lds<16>(raw_rsrc(a.x + l * a.x_stride, kH * 2), P + S.p_x, 0, kH * 2, lane);
}

// Blob of unit u (a routed rank below k, else the shared expert) and whether
// its offset is usable; an unusable blob reads zeros.
__device__ __forceinline__ const uint8_t* unit_blob(const StackArgs& a, const lds_w32* misc, int u, int l, bool& ok) {
  if (u >= a.k) {
    ok = true;
    return a.shared + l * a.sh_stride;
  }
  const int64_t off0 = ((const lds_i64*)(misc + kMOff))[u];
  const int64_t off = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off0 >> 32))) << 32) |
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(off0)));
  ok = slot_ok(off, kBlob, a.pool_bytes);
  return a.pool + (ok ? off : 0);
}

// The block's down rows of its whole unit (rows [64 m, + 64) of rank g), its
// split unit (rows [512 (g % 4) + 16 m, + 16) of rank 8 + g / 4) and the shared
// expert (rows [256 g + 8 m, + 8)), into LDS.
__device__ __forceinline__ void issue_down(const StackArgs& a, const SLds& S, uint8_t* lds, const lds_w32* misc,
                                           int grp, int mem, bool has_w, bool has_s, int l, int lane) {
  bool ok;
  if (has_w) {
    const uint8_t* blob = unit_blob(a, misc, grp, l, ok);
    copy_down_rows(raw_rsrc(blob, ok ? kBlob : 0), lds + S.d[0], mem * kDPM, kDPM, lane);
  }
  if (has_s) {
    const uint8_t* blob = unit_blob(a, misc, kNG + grp / kQG, l, ok);
    copy_down_rows(raw_rsrc(blob, ok ? kBlob : 0), lds + S.d[1], (grp % kQG) * (kH / kQG) + mem * kSDR, kSDR, lane);
  }
  copy_down_rows(raw_rsrc(a.shared + l * a.sh_stride, kBlob), lds + S.d[2], grp * (kH / kNG) + mem * kFR, kFR, lane);
}

// After a barrier: true if every reading wave's read succeeded.
__device__ __forceinline__ bool reads_ok(const lds_w32* misc) {
  bool ok = true;
#pragma unroll
  for (int w = 0; w < kRdWaves; ++w) ok = ok && misc[kMRd + w] != 0u;
  return ok;
}

// Unchained: one wave finishes rows [8 b, 8 b + 8) of layer lf, the ordered
// combine of the row sums of every unit (tag `tg`) with the weights of that
// layer.  False if a word never arrived.
template <int OUT>
__device__ __forceinline__ bool finish_rows(const StackArgs& a, const SLds& S, uint8_t* lds, int lf, uint32_t tg,
                                            int lane) {
  const lds_w32* misc = (const lds_w32*)(lds + S.misc);
  lds_f32* fin = (lds_f32*)(lds + S.fin);
  const uint64_t* part = a.xw + kXPart + static_cast<size_t>(lf & 1) * kPartW;
  const int k = a.k, row0 = blockIdx.x * kFR;
  const int n = (k + 1) * kFR + 1;   // row sums of every unit, then sigma
  uint32_t need = 0;
  for (int q = 0; q < 2; ++q)
    if (lane + q * kWave < n) need |= 1u << q;
  for (uint32_t spins = 0;; ++spins) {
    uint64_t w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = lane + q * kWave;
      const size_t at = i < n - 1 ? static_cast<size_t>(i / kFR) * kH + row0 + i % kFR : static_cast<size_t>(kSigW);
      w[q] = (need >> q) & 1u ? load_tag(part + at) : 0ull;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (((need >> q) & 1u) && static_cast<uint32_t>(w[q] >> 32) == tg) {
        fin[lane + q * kWave] = __uint_as_float(static_cast<uint32_t>(w[q]));
        need &= ~(1u << q);
      }
    if (__ballot(need != 0u) == 0) break;
    if (spins >= a.spin_limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  wave_sync_lds();
  if (lane < kFR) {
    const lds_f32* vals = (const lds_f32*)(misc + kMVals + (lf & 1) * kMaxK);
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc = fmaf(vals[i], fin[i * kFR + lane], acc);
    acc = fmaf(fin[n - 1], fin[k * kFR + lane], acc);
    uint8_t* o = a.out + lf * a.out_stride;
    if constexpr (OUT == kF32) reinterpret_cast<float*>(o)[row0 + lane] = acc;
    else reinterpret_cast<uint16_t*>(o)[row0 + lane] = f32_to_bf16(acc);
  }
  return true;
}

template <int OUT>
__global__ __launch_bounds__(kThr) void k_decode_stack(StackArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const SLds S = stack_lds(a.E, a.rpb);
  int tid = threadIdx.x;
  int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x;
  const int grp = b % kNG, mem = b / kNG;
  const int E = a.E, k = a.k;
  lds_w32* misc = (lds_w32*)(lds + S.misc);
  float* const lg = reinterpret_cast<float*>(lds + S.lg);
  const uint32_t epoch = a.epochs[b];
  bool dead = false;
  bool bad = false;   // a routed blob offset was unusable (its unit contributes nothing)
  // this block's units: the whole unit (rank g), the split unit (rank
  // 8 + g / 4, a quarter of it per group) and an eighth of the shared down
  const bool has_w = grp < k;
  const int ur_s = kNG + grp / kQG;
  const bool has_s = ur_s < k;

  if (tid == 0) misc[kMFin] = 1u;
  if (wave == kWaveStatic) {
    issue_static(a, S, lds, 0, 0, lane);
    wait_vm0();
  }
  __syncthreads();

  for (int l = 0; l < a.L; ++l) {
    // lane-derived addresses are formed again in every layer instead of being
    // held in registers across the loop (which spills them to scratch)
    asm volatile("" : "+v"(lane), "+v"(tid));
    const uint32_t tag = epoch + 1u + static_cast<uint32_t>(l);
    const int p = l & 1;                                     // copy of the exchange regions
    uint8_t* P = lds + p * S.p_bytes;                        // this layer's static operands
    const uint8_t* xl = P + S.p_x;                           // this layer's input (bf16)
    uint64_t* const lgw = a.xw + kXLg + static_cast<size_t>(p) * kLgRep * kMaxE;
    uint64_t* const shw = a.xw + kXSh + static_cast<size_t>(p) * kI;
    uint64_t* const part = a.xw + kXPart + static_cast<size_t>(p) * kPartW;

    // ------------------------------------------------------------------ R
    // the next layer's static operands into the other copy, free since the
    // layer before this one ended (waited for at the end of this one)
    if (wave == kWaveStatic && l + 1 < a.L) issue_static(a, S, lds, p ^ 1, l + 1, lane);
    // per lane: its 32-value segment of x (lane = segment for H = 2048)
    ActRaw<kBF16> xr;
    load_lds_act_bf16(xl, lane, xr);
    const float xs = xsum_bf16(xr);
    for (int j = wave; j < a.rpb + kSpb; j += kNW) {
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
        if (lane < kLgRep) store_tag(lgw + static_cast<size_t>(lane) * kMaxE + e, __float_as_uint(acc), tag);
      } else {
        const int u = j - a.rpb;
        const int r = b * kSpb + u;
        Seg<4> cg, cu;
        cg.w[0] = *(const lds_u32x4*)((const lds_u8*)(P + S.p_suq + (2 * u) * kRowQ) + 16 * lane);
        cu.w[0] = *(const lds_u32x4*)((const lds_u8*)(P + S.p_suq + (2 * u + 1) * kRowQ) + 16 * lane);
        constexpr uint32_t per = kSpb * (kH / 64);   // bf16 values per plane
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
        if (lane == 0) store_tag(shw + r, __float_as_uint(h), tag);
      }
    }
    if (b == 0 && wave == kNW - 1) {
      // sigmoid(g . x), as the staged path forms it; stored with the row sums
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
      if (lane == 0) misc[kMSig] = __float_as_uint(sigmoid(acc));
    }

    // ------------------------------------------------------------------ K
    __syncthreads();                 // every wave's logit stores are issued
    {
      bool ok = !dead;
      if (ok && wave < kRdWaves) {
        const uint64_t* src = lgw + static_cast<size_t>(b % kLgRep) * kMaxE;
        const bool r = read_tagged<(kMaxE + kRdThr - 1) / kRdThr>(
            tid, E, kRdThr, tag, a.spin_limit, [&](int i) { return src + i; },
            [&](int i, uint32_t bits) { ((lds_f32*)(lg))[i] = __uint_as_float(bits); });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok(misc));
    }
    // top-k on wave 0 (a bound from the lane maxima, the candidates above it
    // ranked exactly, the weights in rank order), then the chosen experts'
    // blob offsets; meanwhile wave 1 finishes the previous layer's rows
    if (wave == 0) {
      const int e = topk_wave_n<8>(lg, E, k, lane, reinterpret_cast<uint64_t*>(lds + S.cand),
                                   reinterpret_cast<int32_t*>(reinterpret_cast<uint32_t*>(lds + S.misc) + kMIds),
                                   reinterpret_cast<float*>(reinterpret_cast<uint32_t*>(lds + S.misc) + kMVals + p * kMaxK));
      const lds_i64* slot = (const lds_i64*)(P + S.p_slot);
      if (lane < k) {   // lane r holds rank r's id
        ((lds_i64*)(misc + kMOff))[lane] = slot[e];
        if (b == 0) {
          if (a.ids_out) a.ids_out[static_cast<size_t>(l) * k + lane] = e;
          if (a.wts_out) a.wts_out[static_cast<size_t>(l) * k + lane] = __uint_as_float(misc[kMVals + p * kMaxK + lane]);
        }
      }
    } else if (wave == kWaveFin) {
      if (l > 0 && !a.x_chain && !dead) {
        const bool r = finish_rows<OUT>(a, S, lds, l - 1, tag - 1u, lane);
        if (lane == 0) misc[kMFin] = r ? 1u : 0u;
      }
    }
    __syncthreads();
    dead = dead || misc[kMFin] == 0u;

    // ------------------------------------------------------------------ G
    {
      // waves 0..3 (the older wave of each SIMD, which issues first): pairs
      // w + 4 j (j < 4) of the whole unit's [16 m, 16 m + 16) and pair w of
      // the split unit's [128 (g % 4) + 4 m, + 4).  One descriptor per unit,
      // every load requested before any compute; an absent unit's descriptor
      // is empty and reads zeros.
      const bool gw = wave < kGA && (has_w || has_s);
      auto pair_row = [&](int j) {
        return j < kPW ? mem * kHPM + wave + kGA * j : (grp % kQG) * (kI / kQG) + mem * kSHP + wave;
      };
      Seg<4> cg[kPW + 1], cu[kPW + 1];
      uint32_t sg[kPW + 1], su[kPW + 1], bg[kPW + 1], bu[kPW + 1];
      bool vw = false, vs = false;
      if (gw) {
        bool okw = false, oks = false;
        const uint8_t* blw = has_w ? unit_blob(a, misc, grp, l, okw) : a.pool;
        const uint8_t* bls = has_s ? unit_blob(a, misc, ur_s, l, oks) : a.pool;
        if ((has_w && !okw) || (has_s && !oks)) bad = true;
        vw = okw;
        vs = oks;
        // the plane offsets go in the scalar offset, the lane's in the vector one
        const __amdgpu_buffer_rsrc_t rsw =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blw), 0, okw ? static_cast<int>(kBlob) : 0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rss =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(bls), 0, oks ? static_cast<int>(kBlob) : 0, 0x00020000);
#pragma unroll
        for (int j = 0; j <= kPW; ++j) {
          const __amdgpu_buffer_rsrc_t rs = j < kPW ? rsw : rss;
          const int rr = pair_row(j);
          const int qo = rr * kRowQ + 16 * lane;
          cg[j].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qo, 0, 2));
          cu[j].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qo, kQ, 2));
          const int si = (rr * (kH / 64) + lane / 2) * 2;
          sg[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ, 0);
          su[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + kS, 0);
          bg[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 3 * kS, 0);
          bu[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 4 * kS, 0);
        }
      }
      __syncthreads();   // the down copies start after every phase-G load is requested
      if (gw) {
        uint64_t* const hw = a.xw + kXHx + static_cast<size_t>(grp) * kI;
        uint64_t* const hq = a.xw + kXHq + static_cast<size_t>(grp / kQG) * kI;
        auto pair_h = [&](int j, bool v) {
          const QPairs pg = qpairs_bf16(cg[j]), pu = qpairs_bf16(cu[j]);
          float accg = 0.f, accu = 0.f, g, uu;
          accg += seg_value_d2(raw_value<kBF16>(sg[j]), raw_value<kBF16>(bg[j]), dot2_seg(pg, xr), xs);
          accu += seg_value_d2(raw_value<kBF16>(su[j]), raw_value<kBF16>(bu[j]), dot2_seg(pu, xr), xs);
          gu_sums_w<kWave>(accg, accu, kWave, g, uu);
          return v ? silu(g) * uu : 0.f;
        };
        if (has_w) {
          // two pairs at a time, with no branch between them
#pragma unroll
          for (int j = 0; j < kPW; j += 2) {
            const float h0 = pair_h(j, vw), h1 = pair_h(j + 1, vw);
            if (lane == 0) {
              store_tag(hw + pair_row(j), __float_as_uint(h0), tag);
              store_tag(hw + pair_row(j + 1), __float_as_uint(h1), tag);
            }
          }
        }
        if (has_s) {
          const float h = pair_h(kPW, vs);
          if (lane == 0) store_tag(hq + pair_row(kPW), __float_as_uint(h), tag);
        }
      } else if (wave == kWaveDown) {
        issue_down(a, S, lds, misc, grp, mem, has_w, has_s, l, lane);
      }
    }

    // ------------------------------------------------------------------ H, D
    __syncthreads();                 // every wave's h stores are issued
    if (wave == kWaveDown) wait_vm0();
    {
      float* hs = reinterpret_cast<float*>(lds + S.hs);
      // waves 0..5 read (wave 6 still has the static copies in flight) h of
      // the whole unit (slot 0), the split unit (slot 1) and the shared
      // expert (slot 2), the present ones one after the other
      const int n0 = has_w ? kI : 0, n1 = has_s ? kI : 0;
      bool ok = !dead;
      if (ok && wave < kRdWaves) {
        const uint64_t* hw = a.xw + kXHx + static_cast<size_t>(grp) * kI;
        const uint64_t* hq = a.xw + kXHq + static_cast<size_t>(grp / kQG) * kI;
        const bool r = read_tagged<(3 * kI + kRdThr - 1) / kRdThr>(
            tid, n0 + n1 + kI, kRdThr, tag, a.spin_limit,
            [&](int i) { return i < n0 ? hw + i : i < n0 + n1 ? hq + (i - n0) : shw + (i - n0 - n1); },
            [&](int i, uint32_t bits) {
              const int t = i < n0 ? 0 : i < n0 + n1 ? 1 : 2;
              const int c = i < n0 ? i : i < n0 + n1 ? i - n0 : i - n0 - n1;
              ((lds_f32*)(hs))[((t * kSegI) + c / kSegCodes) * kPad + c % kSegCodes] = __uint_as_float(bits);
            });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok(misc));
      if (tid < 3 * kSegI) {
        float v[kSegCodes];
        load_lds_seg(hs + static_cast<size_t>(tid) * kPad, 0, v);
        ((lds_f32*)(lds + S.hsum))[tid] = seg_sum(v);
      }
      __syncthreads();
    }
    if (!dead) {
      // passes of four rows: 16 of the whole unit, 4 of the split unit, 2 of
      // the shared expert (absent units take none); wave w takes passes w,
      // w + 8, w + 16.  Lane: segment lane % 16 of row lane / 16 of the pass.
      // The h segment sums were formed once in phase H.
      const int npw_ = has_w ? kDPM / kRpp : 0, nps = has_s ? kSDR / kRpp : 0;
      const int npass = npw_ + nps + kFR / kRpp;
      const int sub = lane / kSegI, seg = lane % kSegI;
      const float* hs = reinterpret_cast<const float*>(lds + S.hs);
      const lds_f32* hsum = (const lds_f32*)(lds + S.hsum);
      auto unit_of = [&](int pp) { return pp < npw_ ? 0 : pp < npw_ + nps ? 1 : 2; };   // wave-uniform
      auto row_of = [&](int pp, int t) {   // row in the unit's LDS rows
        return (pp - (t == 0 ? 0 : t == 1 ? npw_ : npw_ + nps)) * kRpp + sub;
      };
      for (int pp = wave; pp < npass; pp += kNW) {
        const int t = unit_of(pp), lr = row_of(pp, t);
        const int nrow = t == 0 ? kDPM : t == 1 ? kSDR : kFR;
        const int u = t == 0 ? grp : t == 1 ? ur_s : k;
        const int row = t == 0 ? mem * kDPM + lr
                        : t == 1 ? (grp % kQG) * (kH / kQG) + mem * kSDR + lr
                                 : grp * (kH / kNG) + mem * kFR + lr;
        bool valid = true;
        if (t < 2) (void)unit_blob(a, misc, u, l, valid);
        const uint8_t* Dq = lds + (t == 0 ? S.d[0] : t == 1 ? S.d[1] : S.d[2]);
        const lds_w16* sbw = (const lds_w16*)(Dq + nrow * kDRowQ);
        float hv[1][kSegCodes];
        load_lds_seg(hs + (static_cast<size_t>(t) * kSegI + seg) * kPad, 0, hv[0]);
        const float hsv = hsum[t * kSegI + seg];
        Seg<4> code;
        code.w[0] = *(const lds_u32x4*)((const lds_u8*)(Dq) + lr * kDRowQ + 16 * seg);
        const int gi = lr * (kI / 64) + seg / 2;
        const float sc = bf16_to_f32(sbw[gi]), bi = bf16_to_f32(sbw[nrow * (kI / 64) + gi]);
        float qv[1];
        seg_qdot_nt<4, 1>(code, hv, qv);
        float acc = 0.f;
        acc += seg_value(sc, bi, qv[0], hsv);
        const float v = group_sum(acc, kSegI);
        if (seg == 0) store_tag(part + static_cast<size_t>(u) * kH + row, __float_as_uint(valid ? v : 0.f), tag);
      }
    }
    if (b == 0 && tid == 0) store_tag(part + kSigW, misc[kMSig], tag);

    // ------------------------------------------------------------------ chained: the next input
    if (a.x_chain) {
      __syncthreads();               // every row-sum store is issued
      lds_f32* fin = (lds_f32*)(lds + S.fin);
      bool ok = !dead;
      const int nf = (k + 1) * kDPM + 1;   // the rows [64 m, 64 m + 64) of every unit, then sigma
      if (ok && wave < kRdWaves) {
        const bool r = read_tagged<((kMaxK + 1) * kDPM + 1 + kRdThr - 1) / kRdThr>(
            tid, nf, kRdThr, tag, a.spin_limit,
            [&](int i) {
              return i < nf - 1 ? part + static_cast<size_t>(i / kDPM) * kH + mem * kDPM + i % kDPM : part + kSigW;
            },
            [&](int i, uint32_t bits) { fin[i] = __uint_as_float(bits); });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok(misc));
      if (tid < kDPM) {
        // ordered combine: ranks ascending, then the gated shared expert; the
        // stack step x + y in fp32, rounded to nearest even bf16
        const int n = mem * kDPM + tid;
        const lds_f32* vals = (const lds_f32*)(misc + kMVals + p * kMaxK);
        float acc = 0.f;
        for (int i = 0; i < k; ++i) acc = fmaf(vals[i], fin[i * kDPM + tid], acc);
        acc = fmaf(fin[nf - 1], fin[k * kDPM + tid], acc);
        const float xv = bf16_to_f32(((const lds_w16*)(xl))[n]);
        const uint16_t xn = f32_to_bf16(xv + acc);
        if (grp == 0) {
          uint8_t* o = a.out + l * a.out_stride;
          if constexpr (OUT == kF32) reinterpret_cast<float*>(o)[n] = acc;
          else reinterpret_cast<uint16_t*>(o)[n] = f32_to_bf16(acc);
          reinterpret_cast<uint16_t*>(a.x_chain + l * a.xc_stride)[n] = xn;
        }
        ((lds_w16*)(lds + S.xn))[tid] = xn;
      }
      if (l + 1 < a.L) {
        __syncthreads();
        const uint32_t ntag = tag + 1u;    // the next layer's tag marks its input
        uint64_t* xg = a.xx + static_cast<size_t>(grp) * (kH / 2);
        if (tid < kDPM / 2) {
          const lds_w16* xs16 = (const lds_w16*)(lds + S.xn);
          const uint32_t bits = static_cast<uint32_t>(xs16[2 * tid]) | (static_cast<uint32_t>(xs16[2 * tid + 1]) << 16);
          store_tag(xg + mem * (kDPM / 2) + tid, bits, ntag);
        }
        __syncthreads();               // every x store is issued
        lds_w32* xd = (lds_w32*)(lds + (p ^ 1) * S.p_bytes + S.p_x);
        bool ok2 = !dead;
        if (ok2 && wave < kRdWaves) {
          const bool r = read_tagged<(kH / 2 + kRdThr - 1) / kRdThr>(
              tid, kH / 2, kRdThr, ntag, a.spin_limit, [&](int i) { return xg + i; },
              [&](int i, uint32_t bits) { xd[i] = bits; });
          if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
        }
        __syncthreads();
        dead = dead || !(ok2 && reads_ok(misc));
      }
    }
    if (wave == kWaveStatic) wait_vm0();
    __syncthreads();
  }

  // unchained: the last layer's rows, once every group's row sums are out
  if (!a.x_chain && a.L > 0) {
    const uint32_t tl = epoch + static_cast<uint32_t>(a.L);
    bool ok = !dead;
    if (wave == kWaveFin) {
      bool r = true;
      if (ok) r = finish_rows<OUT>(a, S, lds, a.L - 1, tl, lane);
      if (lane == 0) misc[kMFin] = r ? 1u : 0u;
    }
    __syncthreads();
    dead = dead || !ok || misc[kMFin] == 0u;
  }

  if (bad && lane == 0) raise_error(a.ctrl, kErrRange);
  if (dead && tid == 0) raise_error(a.ctrl, kErrTimeout);
  // every block read its counter at its start; advance them (the ones past
  // the grid by block 0), so that all counters stay equal
  if (tid == 0) a.epochs[b] = epoch + static_cast<uint32_t>(a.L);
  if (b == 0)
    for (int j = kNB + tid; j < kFusedMaxBlocks; j += kThr) a.epochs[j] = a.epochs[j] + static_cast<uint32_t>(a.L);
}

}  // namespace

bool stack_supported(const moe_desc& d) {
  // every block must write at least one logit word (see the exchange notes)
  return d.hidden == kH && d.inter == kI && d.shared_inter == kI && d.bits == 4 && d.act_dtype == kBF16 &&
         d.sb_dtype == kBF16 && d.n_experts <= kMaxE && d.n_experts % kNB == 0 && d.top_k <= kMaxK;
}

size_t stack_ws_lg() { return (kXWords > stack_t_ws_words() ? kXWords : stack_t_ws_words()) * 8; }
size_t stack_ws_x() { return static_cast<size_t>(kNG) * (kH / 2) * 8; }

// Grid and LDS of the stack kernel on the current device: 256 blocks, one per
// CU, all resident at once.
int stack_plan(const moe_desc& d, StackPlan* plan) {
  int dev = 0, cus = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ENODEV;
  if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return MOE_ENODEV;
  if (cus < kNB) return MOE_EINVAL;
  const int rpb = (d.n_experts + kNB - 1) / kNB;
  if (rpb > kMaxRpb || d.top_k < 1) return MOE_EINVAL;
  const SLds S = stack_lds(d.n_experts, rpb);
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
  plan->nb = kNB;
  plan->rb = kDPM;
  plan->rpb = rpb;
  plan->spb = kSpb;
  plan->gpb = kHPM;
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
  a.xw = reinterpret_cast<uint64_t*>(c.ws + c.L.s_lg);
  a.xx = reinterpret_cast<uint64_t*>(c.ws + c.L.s_x);
  a.ctrl = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  a.epochs = reinterpret_cast<uint32_t*>(c.ws + c.L.f_epoch);
  a.L = c.n_layers;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.rpb = plan.rpb;
  a.spin_limit = 1u << 21;
  if (d.out_dtype == kF32)
    launch_kernel(k_decode_stack<kF32>, dim3(plan.nb), dim3(kThr), plan.lds, c.stream, a);
  else
    launch_kernel(k_decode_stack<kBF16>, dim3(plan.nb), dim3(kThr), plan.lds, c.stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
