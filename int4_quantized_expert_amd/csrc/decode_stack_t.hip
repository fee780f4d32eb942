// Persistent decode of a stack of MoE layers, 2 to 8 tokens per layer (gfx950).
//
// One launch runs L layers in order on a grid of 256 resident 512-thread
// blocks (one per CU).  A layer's T tokens choose up to T k experts; the
// distinct ones, in ascending id, are its routed units 0..U-1, and the shared
// expert is unit U.  Every block gets the same bytes of every layer:
//   * gate/up: the U * 512 row pairs of the routed units, flattened in unit
//     order; block b takes pairs [2 U b, 2 U (b + 1)), at most two units;
//   * down: the (U + 1) * 2048 rows of all units, flattened the same way;
//     block b takes rows [8 (U + 1) b, 8 (U + 1) (b + 1)), at most two units;
//   * the router rows e = b rpb + j and two of the shared expert's gate/up
//     row pairs, from LDS (copied there while the previous layer ran).
// A row is read once per layer and used for every token that routes to its
// unit.
// Per layer:
//   R  the block's router rows and shared gate/up pairs for every token;
//      logits and shared h go out as tagged words
//   K  every block reads the T E logits; wave t takes token t's top-k and
//      renormalised weights; wave 0 then forms the unit list (a bitmap of the
//      chosen ids), each unit's tokens and their ranks, and the h rows its
//      down range needs; meanwhile waves 1..7 read the previous layer's row
//      sums of the block's 8 output rows (and on block 0 form sigma(g . x_t))
//   G  all eight waves stream the block's gate/up pairs (batches of two, of
//      one unit, in a three-deep ring) and store h per (token, rank) as
//      tagged words; wave 7 first finishes the previous layer's 8 output
//      rows of every token, and after its pairs copies the next layer's
//      static operands into the other LDS copy
//   H  every wave requests its share of the next layer's x and its first
//      two down batches, then reads its share of the down units' h rows
//      into LDS
//   D  all eight waves stream the block's down rows in passes of four, each row
//      against the h of every token of its unit; row sums go out as tagged
//      words by (token, rank)
// The combine of layer l (ranks ascending, then sigma times the shared unit)
// runs during layer l + 1 (the last layer's after the loop): block b owns
// output rows 8b..8b+7 of every token.
//
// Exchanges, tags and the parity copies follow the one-token stack kernel:
// every block writes logit words in phase R (E is a multiple of 256), so a
// block that has read layer l + 1's logits knows every block has finished
// its reads of layer l; regions written before that point and read after it
// (logits, shared h, row sums) alternate between two copies by layer parity.
// Every wait is bounded; on expiry the kernel raises kErrTimeout and skips all
// later waits, so the grid always drains.
//
// Every row sum, the top-k and the combine use the staged kernels' order of
// operations, so the results equal theirs bit for bit.
//
// Sources: routing to k of E experts plus a shared expert in every layer, the
// layer stack run per token on the GPU (Swiftlet README translation, "How it
// works" and "Status"); batched decode reads each chosen expert once for all
// tokens that route to it; int4 affine group quantization with byte-addressed
// kernels and 64-bit offsets (same page, "Relation to TurboFieldfare").
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
constexpr int kNB = 256;                   // blocks in the grid
constexpr int kMaxT = 8;
constexpr int kMaxK = 10;
constexpr int kMaxE = 512;
constexpr int kMaxRpb = kMaxE / kNB;
constexpr int kMaxU = kMaxT * kMaxK;       // routed units of a layer, at most
constexpr int kCW = 8;                     // waves that read h and compute phase D
constexpr int kWaveCopy = 7;               // copies operands, finishes the previous layer
constexpr int kSpb = kI / kNB;             // shared gate/up pairs per block (2)
constexpr int kSegI = kI / kSegCodes;      // 16 segments per down row
constexpr int kRpp = kWave / kSegI;        // 4 down rows per pass
constexpr int kPad = kSegCodes + 4;        // staged h: floats per segment (bank spread)
constexpr int64_t kQ = int64_t(kH) * kI / 2;        // code bytes of one matrix
constexpr int64_t kS = int64_t(kH) * (kI / 64) * 2; // bf16 scale bytes of one matrix
constexpr int64_t kBlob = 3 * kQ + 6 * kS;
constexpr int kRowQ = kH / 2;              // code bytes of a gate/up row
constexpr int kDRowQ = kI / 2;             // code bytes of a down row
constexpr int kLgRep = 8;                  // copies of the exchanged logits
constexpr int kMaxHL = 2 * kMaxT;          // h rows a block's down range needs, at most
constexpr int kGB = 2;                     // gate/up pairs per batch
constexpr int kDB = 3;                     // down passes per batch
constexpr int kFR = 8;                     // output rows a block finishes
// Cost model of the work split: a gate/up pair costs kCostG plus one per token
// of its unit, a down pass (four rows) kCostD plus one per token, so blocks
// whose units many tokens share take fewer rows.  Measured at T = 8 (80B
// shape, Zipf routing), the per-token work sets the time of the slowest
// blocks, so the fixed parts are zero.
constexpr int kCostG = 0;
constexpr int kCostD = 0;
constexpr int kFinW = kMaxT * (kMaxK + 1) * kFR + kMaxT;   // row sums and sigmas the finish reads
static_assert(kSpb == 2 && kH / kNB == kFR, "grid shape");

// Exchange regions (word offsets into the tagged-word buffer).
constexpr size_t kTLg = 0;                                          // [2][kLgRep][kMaxT][kMaxE] logits
constexpr size_t kTSh = kTLg + size_t(2) * kLgRep * kMaxT * kMaxE;  // [2][kMaxT][kI] shared h
constexpr size_t kTHu = kTSh + size_t(2) * kMaxT * kI;              // [kMaxT kMaxK][kI] h of row t k + r
constexpr size_t kTSigW = size_t(kMaxT) * (kMaxK + 1) * kH;         // sigma words in a row-sum copy
constexpr size_t kTPartW = kTSigW + 64;                             // row t (k + 1) + r, then sigma [T]
constexpr size_t kTPart = kTHu + size_t(kMaxT) * kMaxK * kI;        // [2][kTPartW]
constexpr size_t kTWords = kTPart + size_t(2) * kTPartW;

__host__ __device__ constexpr uint32_t r256(uint32_t n) { return (n + 255u) / 256u * 256u; }

struct TLds {
  uint32_t p_rr, p_suq, p_susb, p_slot, p_gv, p_bytes;   // static operands of a layer (two copies)
  uint32_t x;      // [kMaxT][kH] bf16 inputs of the current layer
  uint32_t xs;     // [kMaxT][kWave] f32 segment sums of x
  uint32_t lg;     // [kMaxT][kMaxE] f32 logits
  uint32_t cand;   // [kNW][kCandMax] u64 top-k candidates
  uint32_t hs;     // [kMaxHL][kSegI][kPad] f32 staged h rows
  uint32_t hsum;   // [kMaxHL][kSegI] f32 their segment sums
  uint32_t misc;
  uint32_t fin;    // [kFinW] f32 row sums being combined
  uint32_t total;
};

// misc words (32-bit each)
constexpr int kMIds = 0;                          // [kMaxT][kMaxK] chosen experts by token and rank
constexpr int kMVals = kMIds + kMaxT * kMaxK;     // [2][kMaxT][kMaxK] weights, by layer parity
constexpr int kMSig = kMVals + 2 * kMaxT * kMaxK; // [kMaxT] sigmoid(g . x_t) (block 0)
constexpr int kMBits = kMSig + kMaxT;             // [16] bitmap of the chosen experts
constexpr int kMPref = kMBits + 16;               // [16] units below each bitmap word
constexpr int kMNU = kMPref + 16;                 // U
constexpr int kMNH = kMNU + 1;                    // h rows staged for the down range
constexpr int kMRange = kMNH + 1;                 // [4] the block's pairs [g0, g1) and down passes [d0, d1)
constexpr int kMRd = kMRange + 4;                 // [kNW] results of the reading waves
constexpr int kMHSrc = kMRd + kNW;                // [kMaxHL] word offset of each staged h row
constexpr int kMHJ = kMHSrc + kMaxHL;             // [2][kMaxT] staged row of (down unit s, token t)
constexpr int kMUmask = kMHJ + 2 * kMaxT;         // [kMaxU + 1] tokens of each unit (bit t)
constexpr int kMUrank = kMUmask + kMaxU + 1;      // [kMaxU + 1][kMaxT] bytes: rank of the unit for token t
constexpr int kMUoff = (kMUrank + (kMaxU + 1) * kMaxT / 4 + 2) & ~1;   // [kMaxU] int64 blob offsets
constexpr int kMWords = kMUoff + 2 * kMaxU;

__host__ __device__ inline TLds stack_t_lds(int E, int rpb) {
  TLds s{};
  uint32_t o = 0;
  s.p_rr = o;   o += r256(static_cast<uint32_t>(rpb) * kH * 2);
  s.p_suq = o;  o += r256(kSpb * 2 * kRowQ);
  s.p_susb = o; o += r256(kSpb * 4 * (kH / 64) * 2);
  s.p_slot = o; o += r256(static_cast<uint32_t>(E) * 8);
  s.p_gv = o;   o += r256(kH * 2);
  s.p_bytes = o;
  uint32_t t = 2 * s.p_bytes;
  s.x = t;      t += kMaxT * kH * 2;
  s.xs = t;     t += kMaxT * kWave * 4;
  s.lg = t;     t += kMaxT * kMaxE * 4;
  s.cand = t;   t += kNW * kCandMax * 8;
  s.hs = t;     t += kMaxHL * kSegI * kPad * 4;
  s.hsum = t;   t += kMaxHL * kSegI * 4;
  s.misc = t;   t += r256(kMWords * 4);
  s.fin = t;    t += r256(kFinW * 4);
  s.total = t;
  return s;
}

struct StackTArgs {
  const uint8_t* x;          // layer l's input [T][H] bf16 at x + l * x_stride
  int64_t x_stride;
  const uint8_t* router;     // [E, H] bf16 per layer
  int64_t r_stride;
  const uint8_t* slots;      // int64 [E] per layer
  int64_t s_stride;
  const uint8_t* pool;
  int64_t pool_bytes;
  const uint8_t* shared;     // shared blob + gate vector per layer
  int64_t sh_stride;
  int64_t gv_off;
  uint8_t* out;              // [T][H] per layer
  int64_t out_stride;
  int32_t* ids_out;          // optional [L][T][k]
  float* wts_out;            // optional [L][T][k]
  uint64_t* xw;              // tagged words, regions at kT*
  uint32_t* ctrl;            // [0] error flags
  uint32_t* epochs;          // per-block call counters
  int L, T, E, k, rpb;
  uint32_t spin_limit;
};

__device__ __forceinline__ bool reads_ok_w(const lds_w32* misc, int w0, int w1) {
  bool ok = true;
  for (int w = w0; w < w1; ++w) ok = ok && misc[kMRd + w] != 0u;
  return ok;
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Layer l's static operands into LDS copy `p`: its slot table, this block's
// router rows and shared gate/up pairs, and the gate vector (block 0).
__device__ __forceinline__ void issue_static_t(const StackTArgs& a, const TLds& S, uint8_t* lds, int p, int l,
                                               int lane) {
  uint8_t* P = lds + p * S.p_bytes;
  const int b = blockIdx.x;
  copy_lds<16>(raw_rsrc(a.slots + l * a.s_stride, int64_t(a.E) * 8), P + S.p_slot, 0, a.E * 8, lane);
  {
    const u32x4 rs = raw_rsrc(a.router + l * a.r_stride, int64_t(a.E) * kH * 2);
    for (int j = 0; j < a.rpb; ++j)
      copy_lds<16>(rs, P + S.p_rr + j * kH * 2, static_cast<uint32_t>(b * a.rpb + j) * kH * 2, kH * 2, lane);
  }
  const uint8_t* sh = a.shared + l * a.sh_stride;
  const u32x4 rsh = raw_rsrc(sh, kBlob);
  for (int j = 0; j < kSpb; ++j) {
    const int r = b * kSpb + j;
    copy_lds<16>(rsh, P + S.p_suq + (2 * j) * kRowQ, static_cast<uint32_t>(r) * kRowQ, kRowQ, lane);
    copy_lds<16>(rsh, P + S.p_suq + (2 * j + 1) * kRowQ, static_cast<uint32_t>(kQ + r * kRowQ), kRowQ, lane);
  }
  {
    // [gate s, up s, gate b, up b][kSpb rows][32 groups] bf16
    constexpr uint32_t per = kSpb * (kH / 64) * 2;
    const uint32_t base = static_cast<uint32_t>(b * kSpb) * (kH / 64) * 2;
    for (uint32_t j = 0; j < 4 * per; j += kWave * 4) {
      const uint32_t q = j + static_cast<uint32_t>(lane) * 4;
      const uint32_t plane = q / per, within = q - plane * per;
      const uint32_t poff = static_cast<uint32_t>(3 * kQ) + (plane < 2 ? plane : plane + 1) * static_cast<uint32_t>(kS);
      lds_load<4>(rsh, P + S.p_susb + j, poff + base + within, 0);
    }
  }
  if (b == 0) copy_lds<16>(raw_rsrc(sh + a.gv_off, kH * 2), P + S.p_gv, 0, kH * 2, lane);
}

// Layer l's T inputs into LDS (one copy: requested once the current layer's
// gate/up phase no longer reads it), 1 KB rounds w0, w0 + nw, ... of them.
__device__ __forceinline__ void issue_x_t(const StackTArgs& a, const TLds& S, uint8_t* lds, int l, int w0, int nw,
                                          int lane) {
  const uint32_t bytes = static_cast<uint32_t>(a.T) * kH * 2;   // a multiple of 1 KB
  const u32x4 rs = raw_rsrc(a.x + l * a.x_stride, bytes);
  for (uint32_t j = static_cast<uint32_t>(w0) * 1024u; j < bytes; j += static_cast<uint32_t>(nw) * 1024u)
    lds_load<16>(rs, lds + S.x + j, j + static_cast<uint32_t>(lane) * 16u, 0);
}

// Blob of routed unit u and whether its offset is usable (an unusable blob
// reads zeros through an empty descriptor).
__device__ __forceinline__ const uint8_t* unit_blob_t(const StackTArgs& a, const lds_w32* misc, int u, int l,
                                                      bool& ok) {
  const int64_t off0 = ((const lds_i64*)(misc + kMUoff))[u];
  const int64_t off = (static_cast<int64_t>(uni(static_cast<int>(off0 >> 32))) << 32) |
                      static_cast<uint32_t>(uni(static_cast<int>(off0)));
  ok = slot_ok(off, kBlob, a.pool_bytes);
  return a.pool + (ok ? off : 0);
}

__device__ __forceinline__ int unit_rank(const lds_w32* misc, int u, int t) {
  return ((const __attribute__((address_space(3))) uint8_t*)(misc + kMUrank))[u * kMaxT + t];
}

// Inclusive prefix sum over the wave by DPP moves (no LDS crossbar): within
// each row of 16 lanes by shifts of 1, 2, 4 and 8, then across rows by the
// broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Wave 0: the layer's units from the chosen ids, each unit's tokens and
// ranks, the h rows the block's down range needs, and (block 0) the routing
// record.  Every step runs across the lanes (no per-lane loops over bits).
__device__ __forceinline__ void dispatch_t(const StackTArgs& a, const TLds& S, uint8_t* lds, int p, int l, int lane) {
  lds_w32* misc = (lds_w32*)(lds + S.misc);
  const lds_i64* slot = (const lds_i64*)(lds + p * S.p_bytes + S.p_slot);
  const int T = a.T, k = a.k, b = blockIdx.x;
  // units in ascending id: lane i < 16 counts the chosen ids in bitmap word i
  const uint32_t word = lane < 16 ? misc[kMBits + lane] : 0u;
  const int cw = __popc(word);
  const int incl = wave_scan_incl(cw);
  const int nu = __builtin_amdgcn_readlane(incl, 15);
  if (lane < 16) misc[kMPref + lane] = static_cast<uint32_t>(incl - cw);
  for (int u = lane; u <= nu; u += kWave) misc[kMUmask + u] = u == nu ? (1u << T) - 1u : 0u;
  if (lane < T) ((__attribute__((address_space(3))) uint8_t*)(misc + kMUrank))[nu * kMaxT + lane] = static_cast<uint8_t>(k);
  if (lane == 0) misc[kMNU] = static_cast<uint32_t>(nu);
  wave_sync_lds();
  // every choice (t, r): its unit's token mask, rank and blob offset (a unit
  // chosen by several tokens writes the same offset several times)
  for (int i = lane; i < T * k; i += kWave) {
    const int t = i / k, r = i - t * k;
    const int e = static_cast<int>(misc[kMIds + t * kMaxK + r]);
    const uint32_t w = misc[kMBits + (e >> 5)];
    const int u = static_cast<int>(misc[kMPref + (e >> 5)]) + __popc(w & ((1u << (e & 31)) - 1u));
    __hip_atomic_fetch_or(misc + kMUmask + u, 1u << t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    ((__attribute__((address_space(3))) uint8_t*)(misc + kMUrank))[u * kMaxT + t] = static_cast<uint8_t>(r);
    ((lds_i64*)(misc + kMUoff))[u] = slot[e];
    if (b == 0) {
      const size_t o = (static_cast<size_t>(l) * T + t) * k + r;
      if (a.ids_out) a.ids_out[o] = e;
      if (a.wts_out) a.wts_out[o] = __uint_as_float(misc[kMVals + (p * kMaxT + t) * kMaxK + r]);
    }
  }
  wave_sync_lds();
  // the block's share of the gate/up pairs (units 0..U-1, 512 pairs each) and
  // of the down passes (units 0..U, 512 passes each), equal in cost
  int rng[4];
  {
    // lane i: units 2i and 2i + 1, gate/up (d = 0) and down (d = 1) costs
    const int ua = 2 * lane, ub = 2 * lane + 1;
    const int ma = ua <= nu ? __popc(misc[kMUmask + ua]) : 0, mb = ub <= nu ? __popc(misc[kMUmask + ub]) : 0;
    int ca[2], cb[2], inc[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int nun = d == 0 ? nu : nu + 1;
      const int base = d == 0 ? kCostG : kCostD;
      ca[d] = ua < nun ? base + ma : 0;
      cb[d] = ub < nun ? base + mb : 0;
      inc[d] = wave_scan_incl(ca[d] + cb[d]);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int nun = d == 0 ? nu : nu + 1;
      const int total = __builtin_amdgcn_readlane(inc[d], kWave - 1);
      const int pa = (inc[d] - ca[d] - cb[d]) * 512, pb = pa + ca[d] * 512;   // cost before units ua and ub
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int bb = b + e;
        int q = nun * 512;                                          // the end, for bb = 256
        if (bb < kNB) {
          const int B = static_cast<int>((static_cast<int64_t>(total) * 512 * bb) / kNB);
          int cand = -1;
          if (ca[d] > 0 && pa <= B && B < pa + 512 * ca[d]) cand = ua * 512 + (B - pa + ca[d] - 1) / ca[d];
          if (cb[d] > 0 && pb <= B && B < pb + 512 * cb[d]) cand = ub * 512 + (B - pb + cb[d] - 1) / cb[d];
          const uint64_t hit = __ballot(cand >= 0);
          q = __builtin_amdgcn_readlane(cand, static_cast<int>(__builtin_ctzll(hit)));
        }
        rng[2 * d + e] = q;
      }
    }
  }
  if (lane < 4) misc[kMRange + lane] = static_cast<uint32_t>(lane == 0 ? rng[0] : lane == 1 ? rng[1] : lane == 2 ? rng[2] : rng[3]);
  // the h rows of the down range's units (at most two): routed rows by
  // (token, rank), the shared unit's by token; lane s 8 + t takes token t of
  // the range's unit s
  {
    const int r0 = kRpp * rng[2], r1 = kRpp * rng[3];
    const int u0 = r0 / kH, u1 = r1 > r0 ? (r1 - 1) / kH : u0;
    const bool any = r1 > r0 && u0 <= nu, two = any && u1 != u0 && u1 <= nu;
    const uint32_t m0 = any ? misc[kMUmask + u0] : 0u, m1 = two ? misc[kMUmask + u1] : 0u;
    if (lane < 2 * kMaxT) {
      const int s = lane / kMaxT, t = lane % kMaxT;
      const int u = s == 0 ? u0 : u1;
      const uint32_t ms = s == 0 ? m0 : m1;
      if ((ms >> t) & 1u) {
        const int j = (s == 1 ? __popc(m0) : 0) + __popc(ms & ((1u << t) - 1u));
        misc[kMHSrc + j] = u == nu ? static_cast<uint32_t>(kTSh + (size_t(p) * kMaxT + t) * kI)
                                   : static_cast<uint32_t>(kTHu + (size_t(t) * k + unit_rank(misc, u, t)) * kI);
        misc[kMHJ + s * kMaxT + t] = static_cast<uint32_t>(j);
      }
    }
    if (lane == 0) misc[kMNH] = static_cast<uint32_t>(__popc(m0) + __popc(m1));
  }
}

// Waves 1..7: the row sums of layer lf of the block's output rows (every
// token and rank, then the sigmas), tag tg, into fin.
__device__ __forceinline__ bool finish_read_t(const StackTArgs& a, const TLds& S, uint8_t* lds, int lf, uint32_t tg,
                                              int rt) {
  const uint64_t* part = a.xw + kTPart + static_cast<size_t>(lf & 1) * kTPartW;
  lds_f32* fin = (lds_f32*)(lds + S.fin);
  const int T = a.T, k = a.k, row0 = blockIdx.x * kFR;
  const int nrs = T * (k + 1) * kFR;
  constexpr int kRd = (kNW - 1) * kWave;
  return read_tagged<(kFinW + kRd - 1) / kRd>(
      rt, nrs + T, kRd, tg, a.spin_limit,
      [&](int i) {
        return i < nrs ? part + static_cast<size_t>(i / kFR) * kH + row0 + i % kFR : part + kTSigW + (i - nrs);
      },
      [&](int i, uint32_t bits) { fin[i] = __uint_as_float(bits); });
}

// Wave 7: the ordered combine of layer lf's rows (lane = t 8 + row).
template <int OUT>
__device__ __forceinline__ void finish_combine_t(const StackTArgs& a, const TLds& S, uint8_t* lds, int lf, int lane) {
  const lds_w32* misc = (const lds_w32*)(lds + S.misc);
  const lds_f32* fin = (const lds_f32*)(lds + S.fin);
  const int T = a.T, k = a.k;
  const int t = lane / kFR, row = lane % kFR;
  if (t < T) {
    const lds_f32* vals = (const lds_f32*)(misc + kMVals + ((lf & 1) * kMaxT + t) * kMaxK);
    const int base = t * (k + 1) * kFR + row;
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc = fmaf(vals[i], fin[base + i * kFR], acc);
    acc = fmaf(fin[T * (k + 1) * kFR + t], fin[base + k * kFR], acc);
    uint8_t* o = a.out + lf * a.out_stride;
    const int n = t * kH + blockIdx.x * kFR + row;
    if constexpr (OUT == kF32) reinterpret_cast<float*>(o)[n] = acc;
    else reinterpret_cast<uint16_t*>(o)[n] = f32_to_bf16(acc);
  }
}

// A batch of up to kGB gate/up pairs of one wave, all of one unit: pairs
// j0 .. j0 + n - 1 of the wave (a slot past n repeats pair j0, masked).
struct GBatch {
  Seg<4> cg[kGB], cu[kGB];
  uint32_t sg[kGB], su[kGB], bg[kGB], bu[kGB];
  int u, j0, n;
  bool v;
};

// A batch of up to kDB down passes of one wave, all of one unit: per lane its
// row's segment of codes, scale and bias.
struct DBatch {
  Seg<4> c[kDB];
  uint32_t sc[kDB], bi[kDB];
  int u, j0, n;
  bool v;
};

// Three batches in a ring: while batch i is computed, batches i + 1 and
// i + 2 are in flight.  load(B, j) requests the batch that starts at item j
// and returns its size; b0 (and b1 when h1) have been requested already.
template <typename BT, typename LoadF, typename CompF>
__device__ __forceinline__ void ring3(int n, int j, bool h1, BT& b0, BT& b1, BT& b2, LoadF&& load, CompF&& comp) {
  for (;;) {
    const bool h2 = h1 && j < n;
    if (h2) j += load(b2, j);
    comp(b0);
    if (!h1) break;
    const bool h0 = h2 && j < n;
    if (h0) j += load(b0, j);
    comp(b1);
    if (!h2) break;
    h1 = h0 && j < n;
    if (h1) j += load(b1, j);
    comp(b2);
    if (!h0) break;
  }
}

template <int OUT>
__global__ __launch_bounds__(kThr) void k_decode_stack_t(StackTArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const TLds S = stack_t_lds(a.E, a.rpb);
  const int tid0 = threadIdx.x;
  const int wave = uni(tid0 / kWave);
  const int b = blockIdx.x;
  int lane = tid0 & (kWave - 1);
  int tid = tid0;
  const int E = a.E, k = a.k, T = a.T;
  lds_w32* misc = (lds_w32*)(lds + S.misc);
  lds_f32* const lg = (lds_f32*)(lds + S.lg);
  lds_f32* const xs_tab = (lds_f32*)(lds + S.xs);
  const uint8_t* const X = lds + S.x;
  const uint32_t epoch = a.epochs[b];
  bool dead = false;
  bool bad = false;   // a routed blob offset was unusable (its unit contributes nothing)

  if (wave == kWaveCopy) {
    issue_static_t(a, S, lds, 0, 0, lane);
    issue_x_t(a, S, lds, 0, 0, 1, lane);
    wait_vm0();
  }
  __syncthreads();

  for (int l = 0; l < a.L; ++l) {
    // lane-derived addresses are formed again in every layer instead of being
    // held in registers across the loop (which spills them to scratch)
    asm volatile("" : "+v"(lane), "+v"(tid));
    const uint32_t tag = epoch + 1u + static_cast<uint32_t>(l);
    const int p = l & 1;
    const uint8_t* P = lds + p * S.p_bytes;
    uint64_t* const lgw = a.xw + kTLg + static_cast<size_t>(p) * kLgRep * kMaxT * kMaxE;
    uint64_t* const shw = a.xw + kTSh + static_cast<size_t>(p) * kMaxT * kI;
    uint64_t* const huw = a.xw + kTHu;
    uint64_t* const part = a.xw + kTPart + static_cast<size_t>(p) * kTPartW;

    // ------------------------------------------------------------------ R
    if (tid < 16) misc[kMBits + tid] = 0u;
    if (wave < T) {
      ActRaw<kBF16> xr;
      load_lds_act_bf16(X + wave * kH * 2, lane, xr);
      xs_tab[wave * kWave + lane] = xsum_bf16(xr);
    }
    {
      // items of two tokens each (their chains side by side); an odd last
      // item repeats its token and stores once
      const int ntp = (T + 1) / 2;
      const int nr = a.rpb * ntp, ns = kSpb * ntp;
      for (int i = wave; i < nr + ns; i += kNW) {
        {
          const bool router = i < nr;
          const int q = router ? i : i - nr;
          const int j = q / ntp, tp = q - j * ntp;
          const int t0 = 2 * tp, t1 = 2 * tp + 1 < T ? 2 * tp + 1 : 2 * tp;
          ActRaw<kBF16> xr0, xr1;
          load_lds_act_bf16(X + t0 * kH * 2, lane, xr0);
          load_lds_act_bf16(X + t1 * kH * 2, lane, xr1);
          if (router) {
            // router row j of tokens t0 and t1
            const int e = b * a.rpb + j;
            ActRaw<kBF16> rw;
            load_lds_act_bf16(P + S.p_rr + j * kH * 2, lane, rw);
            float r[kSegCodes], v0[kSegCodes], v1[kSegCodes];
            act_raw_f32<kBF16>(rw, r);
            act_raw_f32<kBF16>(xr0, v0);
            act_raw_f32<kBF16>(xr1, v1);
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int c = 0; c < kSegCodes; ++c) {
              acc0 = fmaf(v0[c], r[c], acc0);
              acc1 = fmaf(v1[c], r[c], acc1);
            }
            acc0 = group_sum(acc0, kWave);
            acc1 = group_sum(acc1, kWave);
            if (lane < kLgRep) {
              store_tag(lgw + (static_cast<size_t>(lane) * kMaxT + t0) * kMaxE + e, __float_as_uint(acc0), tag);
              if (t1 != t0) store_tag(lgw + (static_cast<size_t>(lane) * kMaxT + t1) * kMaxE + e, __float_as_uint(acc1), tag);
            }
          } else {
            // shared gate/up pair j of tokens t0 and t1
            const int r = b * kSpb + j;
            Seg<4> cg, cu;
            cg.w[0] = *(const lds_u32x4*)((const lds_u8*)(P + S.p_suq + (2 * j) * kRowQ) + 16 * lane);
            cu.w[0] = *(const lds_u32x4*)((const lds_u8*)(P + S.p_suq + (2 * j + 1) * kRowQ) + 16 * lane);
            constexpr uint32_t per = kSpb * (kH / 64);
            const lds_w16* sb = (const lds_w16*)(P + S.p_susb);
            const int gi = j * (kH / 64) + lane / 2;
            const float sg = bf16_to_f32(sb[gi]), su = bf16_to_f32(sb[per + gi]);
            const float bg = bf16_to_f32(sb[2 * per + gi]), bu = bf16_to_f32(sb[3 * per + gi]);
            const QPairs pg = qpairs_bf16(cg), pu = qpairs_bf16(cu);
            const float xs0 = xsum_bf16(xr0), xs1 = xsum_bf16(xr1);
            float ag0 = 0.f, au0 = 0.f, ag1 = 0.f, au1 = 0.f;
            ag0 += seg_value_d2(sg, bg, dot2_seg(pg, xr0), xs0);
            au0 += seg_value_d2(su, bu, dot2_seg(pu, xr0), xs0);
            ag1 += seg_value_d2(sg, bg, dot2_seg(pg, xr1), xs1);
            au1 += seg_value_d2(su, bu, dot2_seg(pu, xr1), xs1);
            float g0, u0_, g1, u1_;
            gu_sums_w<kWave>(ag0, au0, kWave, g0, u0_);
            gu_sums_w<kWave>(ag1, au1, kWave, g1, u1_);
            const float h0 = silu(g0) * u0_, h1 = silu(g1) * u1_;
            if (lane == 0) {
              store_tag(shw + static_cast<size_t>(t0) * kI + r, __float_as_uint(h0), tag);
              if (t1 != t0) store_tag(shw + static_cast<size_t>(t1) * kI + r, __float_as_uint(h1), tag);
            }
          }
        }
      }
    }

    // ------------------------------------------------------------------ K
    __syncthreads();                 // every wave's logit stores are issued
    {
      const bool ok = !dead;
      if (ok) {
        const uint64_t* src = lgw + static_cast<size_t>(b % kLgRep) * kMaxT * kMaxE;
        const bool r = read_tagged<kMaxT * kMaxE / kThr>(
            tid, T * E, kThr, tag, a.spin_limit,
            [&](int i) {
              const int t = i / E;
              return src + static_cast<size_t>(t) * kMaxE + (i - t * E);
            },
            [&](int i, uint32_t bits) {
              const int t = i / E;
              lg[t * kMaxE + (i - t * E)] = __uint_as_float(bits);
            });
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      __syncthreads();
      dead = dead || !(ok && reads_ok_w(misc, 0, kNW));
    }
    // top-k of token t on wave t, then its ids into the bitmap
    if (wave < T) {
      uint64_t* cand = reinterpret_cast<uint64_t*>(lds + S.cand) + wave * kCandMax;
      uint32_t* mg = reinterpret_cast<uint32_t*>(lds + S.misc);   // generic pointers to the LDS words
      int32_t* ids = reinterpret_cast<int32_t*>(mg + kMIds + wave * kMaxK);
      float* vals = reinterpret_cast<float*>(mg + kMVals + (p * kMaxT + wave) * kMaxK);
      topk_wave_n<kMaxE / kWave>(reinterpret_cast<float*>(lds + S.lg) + wave * kMaxE, E, k, lane, cand, ids, vals);
      wave_sync_lds();
      if (lane < k) {
        const int e = static_cast<int>(misc[kMIds + wave * kMaxK + lane]);
        __hip_atomic_fetch_or(misc + kMBits + (e >> 5), 1u << (e & 31), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    __syncthreads();
    // wave 0: the units; waves 1..7: the previous layer's row sums
    if (wave == 0) {
      dispatch_t(a, S, lds, p, l, lane);
    } else {
      bool r = true;
      if (l > 0 && !dead) r = finish_read_t(a, S, lds, l - 1, tag - 1u, tid - kWave);
      if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      // block 0: sigmoid(g . x_t) of this layer's tokens (stored with the row
      // sums at the end of the layer), here rather than in phase R so that
      // block 0's logits are not later than the others'
      if (b == 0)
        for (int t = wave - 1; t < T; t += kNW - 1) {
          ActRaw<kBF16> xr, gw;
          load_lds_act_bf16(X + t * kH * 2, lane, xr);
          load_lds_act_bf16(P + S.p_gv, lane, gw);
          float xv[kSegCodes], gv[kSegCodes];
          act_raw_f32<kBF16>(xr, xv);
          act_raw_f32<kBF16>(gw, gv);
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < kSegCodes; ++c) acc = fmaf(xv[c], gv[c], acc);
          acc = group_sum(acc, kWave);
          if (lane == 0) misc[kMSig + t] = __float_as_uint(sigmoid(acc));
        }
    }
    __syncthreads();
    dead = dead || !reads_ok_w(misc, 1, kNW);
    const int nu = uni(static_cast<int>(misc[kMNU]));

    // ------------------------------------------------------------------ G
    // every wave streams gate/up pairs; wave 7 first finishes the previous
    // layer's rows and, after its pairs, copies the next layer's static
    // operands into the other copy (free since the layer before this one
    // ended; waited for at the end of this one)
    if (wave == kWaveCopy && l > 0 && !dead) finish_combine_t<OUT>(a, S, lds, l - 1, lane);
    {
      const int q0 = uni(static_cast<int>(misc[kMRange + 0]));   // this block's pairs, flattened over the units
      const int np = uni(static_cast<int>(misc[kMRange + 1])) - q0;
      const int ug = q0 / kI;                // its unit; pairs from (ug + 1) 512 on are of the next
      const int npw = wave < np ? (np - wave + kNW - 1) / kNW : 0;   // this wave's pairs: wave + 8 j
      const int ib = (ug + 1) * kI - q0;     // first local pair of the next unit
      const int jb = ib <= wave ? 0 : (ib - wave + kNW - 1) / kNW < npw ? (ib - wave + kNW - 1) / kNW : npw;
      // every pair of a batch is requested before any is used
      auto load_g = [&](GBatch& B, int j0) {
        const int u = j0 < jb ? ug : ug + 1;
        const int end = j0 < jb ? jb : npw;
        B.u = u;
        B.j0 = j0;
        B.n = end - j0 < kGB ? end - j0 : kGB;
        bool ok;
        const uint8_t* blob = unit_blob_t(a, misc, u, l, ok);
        if (!ok) bad = true;
        B.v = ok;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), 0, ok ? static_cast<int>(kBlob) : 0, 0x00020000);
#pragma unroll
        for (int bb = 0; bb < kGB; ++bb) {
          const int j = j0 + (bb < B.n ? bb : 0);
          const int row = q0 + wave + kNW * j - u * kI;
          const int qo = row * kRowQ + 16 * lane;
          B.cg[bb].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qo, 0, 2));
          B.cu[bb].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, qo, kQ, 2));
          const int si = (row * (kH / 64) + lane / 2) * 2;
          B.sg[bb] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ, 0);
          B.su[bb] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + kS, 0);
          B.bg[bb] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 3 * kS, 0);
          B.bu[bb] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 4 * kS, 0);
        }
        return B.n;
      };
      // tokens outer, the batch's pairs inner (independent, so their chains
      // overlap); the batch is of one unit, so every pair has the same tokens
      auto compute_g = [&](const GBatch& B) {
        const int u = B.u;
        uint32_t m = static_cast<uint32_t>(uni(static_cast<int>(misc[kMUmask + u])));
        float sgv[kGB], bgv[kGB], suv[kGB], buv[kGB];
#pragma unroll
        for (int bb = 0; bb < kGB; ++bb) {
          sgv[bb] = raw_value<kBF16>(B.sg[bb]);
          bgv[bb] = raw_value<kBF16>(B.bg[bb]);
          suv[bb] = raw_value<kBF16>(B.su[bb]);
          buv[bb] = raw_value<kBF16>(B.bu[bb]);
        }
        while (m != 0u) {
          const int t = __builtin_ctz(m);
          m &= m - 1u;
          ActRaw<kBF16> xr;
          load_lds_act_bf16(X + t * kH * 2, lane, xr);
          const float xs = xs_tab[t * kWave + lane];
          const int r = uni(unit_rank(misc, u, t));
          float h[kGB];
#pragma unroll
          for (int bb = 0; bb < kGB; ++bb) {
            const QPairs pg = qpairs_bf16(B.cg[bb]), pu = qpairs_bf16(B.cu[bb]);
            float accg = 0.f, accu = 0.f;
            accg += seg_value_d2(sgv[bb], bgv[bb], dot2_seg(pg, xr), xs);
            accu += seg_value_d2(suv[bb], buv[bb], dot2_seg(pu, xr), xs);
            float g, uu;
            gu_sums_w<kWave>(accg, accu, kWave, g, uu);
            h[bb] = B.v ? silu(g) * uu : 0.f;
          }
          if (lane == 0) {
#pragma unroll
            for (int bb = 0; bb < kGB; ++bb)
              if (bb < B.n)
                store_tag(huw + (static_cast<size_t>(t) * k + r) * kI + q0 + wave + kNW * (B.j0 + bb) - u * kI,
                          __float_as_uint(h[bb]), tag);
          }
        }
      };
      if (npw > 0) {
        GBatch b0, b1, b2;
        int j = load_g(b0, 0);
        const bool h1 = j < npw;
        if (h1) j += load_g(b1, j);
        ring3(npw, j, h1, b0, b1, b2, load_g, compute_g);
      }
    }
    if (wave == kWaveCopy && l + 1 < a.L) issue_static_t(a, S, lds, p ^ 1, l + 1, lane);

    // ------------------------------------------------------------------ H
    __syncthreads();                 // every h store is issued; x is no longer read
    if (l + 1 < a.L) issue_x_t(a, S, lds, l + 1, wave, kNW, lane);
    const int pa = uni(static_cast<int>(misc[kMRange + 2]));   // this block's down passes, flattened
    const int npass = uni(static_cast<int>(misc[kMRange + 3])) - pa;
    const int r0 = kRpp * pa;                     // its first row
    const int u0 = r0 / kH;                       // its unit; rows from (u0 + 1) 2048 on are of the next
    const int npw_d = wave < kCW && wave < npass ? (npass - wave + kCW - 1) / kCW : 0;
    const int pb = ((u0 + 1) * kH - r0) / kRpp;   // first local pass of the next unit
    const int jb_d = pb <= wave ? 0 : (pb - wave + kCW - 1) / kCW < npw_d ? (pb - wave + kCW - 1) / kCW : npw_d;
    const int sub = lane / kSegI, seg = lane % kSegI;
    auto load_d = [&](DBatch& B, int j0) {
      const int u = j0 < jb_d ? u0 : u0 + 1;
      const int end = j0 < jb_d ? jb_d : npw_d;
      B.u = u;
      B.j0 = j0;
      B.n = end - j0 < kDB ? end - j0 : kDB;
      bool ok = true;
      const uint8_t* blob = u == nu ? a.shared + l * a.sh_stride : unit_blob_t(a, misc, u, l, ok);
      B.v = ok;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blob), 0, ok ? static_cast<int>(kBlob) : 0, 0x00020000);
#pragma unroll
      for (int bb = 0; bb < kDB; ++bb) {
        const int j = j0 + (bb < B.n ? bb : 0);
        const int row = r0 + kRpp * (wave + kCW * j) - u * kH + sub;
        B.c[bb].w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, row * kDRowQ + 16 * seg, 2 * kQ, 2));
        const int si = (row * (kI / 64) + seg / 2) * 2;
        B.sc[bb] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 2 * kS, 0);
        B.bi[bb] = __builtin_amdgcn_raw_buffer_load_b16(rs, si, 3 * kQ + 5 * kS, 0);
      }
      return B.n;
    };
    // the first two down batches are requested before the h wait
    DBatch d0, d1, d2;
    int jd = npw_d > 0 ? load_d(d0, 0) : 0;
    const bool hd1 = npw_d > 0 && jd < npw_d;
    if (hd1) jd += load_d(d1, jd);
    {
      // every wave reads a share of the staged h rows (the wait for them
      // also covers the wave's input copy and first down batches)
      lds_f32* hs = (lds_f32*)(lds + S.hs);
      const int nh = uni(static_cast<int>(misc[kMNH]));
      bool ok = !dead;
      if (ok && wave < kCW) {
        constexpr int kRd = kCW * kWave;
        constexpr int kPer = 12;           // up to 16 h rows in at most two rounds
        bool r = true;
        for (int c0 = 0; r && c0 < nh * kI; c0 += kPer * kRd) {
          const int n = nh * kI - c0 < kPer * kRd ? nh * kI - c0 : kPer * kRd;
          r = read_tagged<kPer>(
              tid, n, kRd, tag, a.spin_limit,
              [&](int i) {
                const int w = c0 + i;
                return a.xw + misc[kMHSrc + (w >> 9)] + (w & (kI - 1));
              },
              [&](int i, uint32_t bits) {
                const int w = c0 + i, j = w >> 9, c = w & (kI - 1);
                hs[(j * kSegI + c / kSegCodes) * kPad + c % kSegCodes] = __uint_as_float(bits);
              });
        }
        if (lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
      }
      wait_vm0();   // this wave's share of the next layer's inputs has landed
      __syncthreads();
      dead = dead || !(ok && reads_ok_w(misc, 0, kCW));
      if (tid < nh * kSegI) {
        float v[kSegCodes];
        load_lds_seg((const float*)(lds + S.hs) + static_cast<size_t>(tid) * kPad, 0, v);
        ((lds_f32*)(lds + S.hsum))[tid] = seg_sum(v);
      }
      __syncthreads();
    }

    // ------------------------------------------------------------------ D
    if (!dead && npw_d > 0) {
      const float* hs = reinterpret_cast<const float*>(lds + S.hs);
      const lds_f32* hsum = (const lds_f32*)(lds + S.hsum);
      // tokens outer (the token's h segment read once per batch), the
      // batch's passes inner; the batch is of one unit
      auto compute_d = [&](const DBatch& B) {
        const int u = B.u;
        const int s = u == u0 ? 0 : 1;
        uint32_t m = static_cast<uint32_t>(uni(static_cast<int>(misc[kMUmask + u])));
        float sc[kDB], bi[kDB];
#pragma unroll
        for (int bb = 0; bb < kDB; ++bb) {
          sc[bb] = raw_value<kBF16>(B.sc[bb]);
          bi[bb] = raw_value<kBF16>(B.bi[bb]);
        }
        while (m != 0u) {
          const int t = __builtin_ctz(m);
          m &= m - 1u;
          const int j = uni(static_cast<int>(misc[kMHJ + s * kMaxT + t]));
          float hv[1][kSegCodes];
          load_lds_seg(hs + (static_cast<size_t>(j) * kSegI + seg) * kPad, 0, hv[0]);
          const float hsv = hsum[j * kSegI + seg];
          const int r = u == nu ? k : uni(unit_rank(misc, u, t));
          float v[kDB];
#pragma unroll
          for (int bb = 0; bb < kDB; ++bb) {
            float qv[1];
            seg_qdot_nt<4, 1>(B.c[bb], hv, qv);
            float acc = 0.f;
            acc += seg_value(sc[bb], bi[bb], qv[0], hsv);
            v[bb] = group_sum(acc, kSegI);
          }
          if (seg == 0) {
#pragma unroll
            for (int bb = 0; bb < kDB; ++bb)
              if (bb < B.n)
                store_tag(part + static_cast<size_t>(t * (k + 1) + r) * kH + r0 + kRpp * (wave + kCW * (B.j0 + bb)) -
                              u * kH + sub,
                          __float_as_uint(B.v ? v[bb] : 0.f), tag);
          }
        }
      };
      ring3(npw_d, jd, hd1, d0, d1, d2, load_d, compute_d);
    }
    if (b == 0 && tid < T) store_tag(part + kTSigW + tid, misc[kMSig + tid], tag);

    // ------------------------------------------------------------------ end of layer
    if (wave == kWaveCopy) wait_vm0();
    __syncthreads();
  }

  // the last layer's rows, once every block's row sums are out
  if (a.L > 0) {
    const uint32_t tl = epoch + static_cast<uint32_t>(a.L);
    bool r = true;
    if (wave >= 1 && !dead) r = finish_read_t(a, S, lds, a.L - 1, tl, tid - kWave);
    if (wave >= 1 && lane == 0) misc[kMRd + wave] = r ? 1u : 0u;
    __syncthreads();
    dead = dead || !reads_ok_w(misc, 1, kNW);
    if (wave == kWaveCopy && !dead) finish_combine_t<OUT>(a, S, lds, a.L - 1, lane);
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

bool stack_t_supported(const moe_desc& d, int T) {
  // every block must write at least one logit word (see the exchange notes)
  return T >= 2 && T <= kMaxT && d.hidden == kH && d.inter == kI && d.shared_inter == kI && d.bits == 4 &&
         d.act_dtype == kBF16 && d.sb_dtype == kBF16 && d.n_experts <= kMaxE && d.n_experts % kNB == 0 &&
         d.top_k >= 1 && d.top_k <= kMaxK;
}

size_t stack_t_ws_words() { return kTWords; }

// Grid and LDS of the kernel on the current device: 256 blocks, one per CU,
// all resident at once.
int stack_t_plan(const moe_desc& d, StackPlan* plan) {
  int dev = 0, cus = 0, lds_max = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ENODEV;
  if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return MOE_ENODEV;
  if (cus < kNB) return MOE_EINVAL;
  const int rpb = d.n_experts / kNB;
  if (rpb < 1 || rpb > kMaxRpb) return MOE_EINVAL;
  const TLds S = stack_t_lds(d.n_experts, rpb);
  if (S.total > static_cast<uint32_t>(lds_max)) return MOE_EINVAL;
  const void* fn = d.out_dtype == kF32 ? reinterpret_cast<const void*>(k_decode_stack_t<kF32>)
                                       : reinterpret_cast<const void*>(k_decode_stack_t<kBF16>);
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(S.total)) != hipSuccess)
    return MOE_EHIP;
  int fit = 0;
  const hipError_t e = d.out_dtype == kF32
                           ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, k_decode_stack_t<kF32>, kThr, S.total)
                           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, k_decode_stack_t<kBF16>, kThr, S.total);
  if (e != hipSuccess) return MOE_EHIP;
  if (fit < 1) return MOE_EINVAL;
  plan->nb = kNB;
  plan->rb = kFR;
  plan->rpb = rpb;
  plan->spb = kSpb;
  plan->gpb = 0;
  plan->lds = S.total;
  return MOE_OK;
}

int launch_decode_stack_t(const StackCall& c, const StackPlan& plan) {
  const moe_desc& d = c.d;
  StackTArgs a;
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
  a.ids_out = c.ids_out;
  a.wts_out = c.wts_out;
  a.xw = reinterpret_cast<uint64_t*>(c.ws + c.L.s_lg);
  a.ctrl = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  a.epochs = reinterpret_cast<uint32_t*>(c.ws + c.L.f_epoch);
  a.L = c.n_layers;
  a.T = c.T;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.rpb = plan.rpb;
  a.spin_limit = 1u << 21;
  if (d.out_dtype == kF32)
    launch_kernel(k_decode_stack_t<kF32>, dim3(plan.nb), dim3(kThr), plan.lds, c.stream, a);
  else
    launch_kernel(k_decode_stack_t<kBF16>, dim3(plan.nb), dim3(kThr), plan.lds, c.stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
