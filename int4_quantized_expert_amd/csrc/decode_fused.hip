// Decode of one MoE layer (T <= 8 tokens) in two launches, gfx950.
//
// The staged path needs six dependent launches per layer, and each of them
// starts with a chain of dependent loads; at decode sizes that costs far more
// than streaming the 21.6 MB of the 80B-shaped layer.  Here:
//
// Launch A (persistent grid, every block resident):
//   R  router rows (one logit per wave and token), shared-expert gate/up rows,
//      sigmoid(g . x) -- everything that does not depend on the routing
//   K  every block gathers all logits and computes top-k, the renormalised
//      weights and the expert -> token dispatch itself (no further exchange)
//   G  routed gate/up rows + SwiGLU, flattened over (expert, row) across all
//      waves; h goes to the workspace with plain stores
// Launch B (one block per slice of output rows):
//   D  down rows of every chosen expert and the shared one for the slice,
//      then the ordered combine; h is read through the caches, which the
//      launch boundary makes coherent
//
// Inside launch A only the logits cross blocks.  They travel as 64-bit words
// holding the float bits and a per-call tag, written and read with relaxed
// device-scope atomics; each router block raises a flag word once its phase-R
// stores are acknowledged, and every block waits for those flags before
// reading the logits.  Logits and flags are written in kFusedReplicas copies
// and each block reads the copy of its index modulo kFusedReplicas: hundreds of
// blocks polling the same few cache lines otherwise queue up behind each other.  A word is valid when its tag matches, so no fence is needed (an
// agent-scope release on this chip writes back the L2 and costs microseconds).
// The tag is the workspace epoch + 1; block 0 retires it at its end, after it
// has seen every block's flag.  Every wait is bounded: on expiry the kernel
// raises kErrTimeout and finishes.
//
// Per-row arithmetic uses the same helpers and orders as the staged kernels,
// so both paths give bitwise identical results.
//
// Sources: routing to k of E experts per layer plus the shared expert
// (Swiftlet README translation, "How it works"); int4/int8 affine group
// quantization, byte-addressed kernels with 64-bit offsets, explicit hazard
// management (same page, "Relation to TurboFieldfare").
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fused_common.h"
#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {

namespace {

constexpr int kThreads = 512;             // launch B blocks
constexpr int kWaves = kThreads / kWave;
constexpr int kThreadsA = 512;            // launch A blocks: one per CU (fewer blocks start sooner)
constexpr int kWavesA = kThreadsA / kWave;
constexpr int kMaxDownPerWave = 4;    // down tasks per wave per round in launch B
constexpr int kRouterRowsPerWave = 1; // router row groups per wave in phase R
constexpr int kRowCost = 2;           // phase-G cost of a row's loads, in per-token dots

template <int V>
struct IntC {
  static constexpr int value = V;
};

__device__ __forceinline__ void store_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The logits area also holds, after top-k, one float per (wave, token, lane)
// for phase G.
__host__ __device__ inline size_t lg_floats(int T, int E) {
  const size_t lg = static_cast<size_t>(T) * E, xs = static_cast<size_t>(kWavesA) * T * kWave;
  return lg > xs ? lg : xs;
}

struct LdsA {
  uint8_t* x;        // [T][H] activations, storage dtype
  float* lg;         // [T][E] logits
  int32_t* ids;      // [T][k]
  float* vals;       // [T][k] chosen logits, then weights
  int64_t* slot;     // [E]
  int32_t* umap;     // [E] expert -> distinct index
  int32_t* uniq;     // [umax]
  int32_t* pidx;     // [umax][T] rank i of the expert for token t, or -1
  int32_t* ucost;    // [umax + 1] phase-G work before distinct expert u (T > 1)
  uint64_t* uranks;  // [umax] byte t: 1 + rank of expert u for token t, 0 if unused
  uint64_t* cand;    // [kWavesA][kCandMax] packed candidates
  int32_t* misc;     // [0] U, [1] tag
};

__device__ inline LdsA carve_a(uint8_t* base, const FusedArgs& a) {
  LdsA s;
  size_t o = 0;
  auto take = [&](size_t n) { uint8_t* p = base + o; o += (n + 15) / 16 * 16; return p; };
  s.x = take(static_cast<size_t>(a.T) * a.H * a.act_sz);
  s.lg = reinterpret_cast<float*>(take(lg_floats(a.T, a.E) * 4));
  s.ids = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.T) * a.k * 4));
  s.vals = reinterpret_cast<float*>(take(static_cast<size_t>(a.T) * a.k * 4));
  s.slot = reinterpret_cast<int64_t*>(take(static_cast<size_t>(a.E) * 8));
  s.umap = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.E) * 4));
  s.uniq = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.umax) * 4));
  s.pidx = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.umax) * a.T * 4));
  s.ucost = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.umax + 1) * 4));
  s.uranks = reinterpret_cast<uint64_t*>(take(static_cast<size_t>(a.umax) * 8));
  s.cand = reinterpret_cast<uint64_t*>(take(kWavesA * kCandMax * 8));
  s.misc = reinterpret_cast<int32_t*>(take(16 * 4));
  return s;
}

// ---------------------------------------------------------------------------
// Launch B: one block per (slice of rb output rows, token): the slice's down
// rows of the token's k experts and of the shared expert, then the ordered
// combine.  A block's partial sums are all its own, and the token's k + 1 h
// rows (a few tens of KB) are staged in LDS once, so the work does not grow
// per block with T.  Blocks are numbered so that the tokens of one slice run
// on one XCD and share the slice's weight rows through its L2.
// One task = `rpp` rows of one expert's Wd (lane: one segment of one row).
template <int BITS>
struct DownTask {
  Seg<BITS> code;
  uint32_t sc, bi;   // raw scale and bias bits (see load_raw)
  int i;        // pair rank of the expert for the token (k = shared), -1 if none
  int rloc;     // this lane's row within the block, -1 if outside
  bool valid;   // blob offset usable
};

struct LdsB {
  int64_t* poff;     // [k] blob offsets of the token's experts, by rank
  float* wts;        // [k] the token's combine weights
  float* sig;        // [1] its shared-expert gate
  float* part;       // [k + 1][rb]
  float* h;          // [k + 1][hs / 32][kSegPad] staged activations, or nullptr when they do not fit
  float* hsum;       // [k + 1][hs / 32] segment sums of the staged rows
};

// h rows are staged in LDS when they take at most this many bytes.  Each
// 32-float segment sits at a stride of kSegPad floats, so the 16 lanes that
// read the 16 segments of one row hit different LDS banks.
constexpr size_t kHStageMax = 56 * 1024;
constexpr int kSegPad = kSegCodes + 4;
constexpr int kXcds = 8;

__host__ __device__ inline size_t h_stage_floats(int k, int hs) {
  return static_cast<size_t>(k + 1) * (hs / kSegCodes) * kSegPad;
}

__host__ __device__ inline bool h_staged(int k, int hs) { return h_stage_floats(k, hs) * 4 <= kHStageMax; }

__device__ inline LdsB carve_b(uint8_t* base, const FusedArgs& a) {
  LdsB s;
  size_t o = 0;
  auto take = [&](size_t n) { uint8_t* p = base + o; o += (n + 15) / 16 * 16; return p; };
  s.poff = reinterpret_cast<int64_t*>(take(static_cast<size_t>(a.k) * 8));
  s.wts = reinterpret_cast<float*>(take(static_cast<size_t>(a.k) * 4));
  s.sig = reinterpret_cast<float*>(take(4));
  s.part = reinterpret_cast<float*>(take(static_cast<size_t>(a.k + 1) * a.rb * 4));
  const bool st = h_staged(a.k, a.hs);
  s.h = st ? reinterpret_cast<float*>(take(h_stage_floats(a.k, a.hs) * 4)) : nullptr;
  s.hsum = st ? reinterpret_cast<float*>(take(static_cast<size_t>(a.k + 1) * (a.hs / kSegCodes) * 4)) : nullptr;
  return s;
}

// Per-launch constants of the down tasks, computed once per wave: plane
// offsets and row sizes of the routed and the shared blobs, and this lane's
// byte offsets within a row.
struct DownCtx {
  int64_t q_r, s_r, q_s, s_s;       // code / scale plane bytes (routed, shared)
  int64_t blob_r;                   // routed blob bytes
  int64_t rowb_r, rowb_s;           // code bytes per row
  int gpr_r, gpr_s;                 // scale groups per row
  int np;                           // row passes per expert
};

template <int BITS, int SB>
__device__ __forceinline__ DownCtx down_ctx(const FusedArgs& a, const RowLanes& rli, const RowLanes& rls) {
  DownCtx c;
  const Planes pr = planes_of(a.H, a.I, BITS, SB), ps = planes_of(a.H, a.SI, BITS, SB);
  c.q_r = pr.q;
  c.s_r = pr.s;
  c.q_s = ps.q;
  c.s_s = ps.s;
  c.blob_r = pr.blob;
  c.rowb_r = static_cast<int64_t>(a.I) * BITS / 8;
  c.rowb_s = static_cast<int64_t>(a.SI) * BITS / 8;
  c.gpr_r = a.I / 64;
  c.gpr_s = a.SI / 64;
  const int rpp_min = rli.rpp < rls.rpp ? rli.rpp : rls.rpp;
  c.np = (a.rb + rpp_min - 1) / rpp_min;
  return c;
}

// Requests one task's codes, scale and bias.  Straight-line code with
// selects only: a dead task (past ntask) or a row past the end reads a valid
// row of the shared blob or of blob 0, and an unusable blob reads blob 0;
// all are masked at use.  Without branches the compiler keeps every task's
// loads of a wave in flight together instead of draining them in between.
template <int BITS, int SB>
__device__ __forceinline__ void load_down_task(DownTask<BITS>& d, int task, int ntask, const DownCtx& c, int row_lo,
                                               const FusedArgs& a, const LdsB& s, const RowLanes& rli,
                                               const RowLanes& rls) {
  const int k = a.k;
  const bool live = task < ntask;
  const int tk = live ? task : 0;
  const int i = c.np == 1 ? tk : tk / c.np;
  const int p = c.np == 1 ? 0 : tk - i * c.np;
  const bool is_sh = i == k;
  const int rpp = is_sh ? rls.rpp : rli.rpp;
  const int sub_row = is_sh ? rls.sub_row : rli.sub_row;
  const int seg0 = is_sh ? rls.seg0 : rli.seg0;
  const int64_t off = s.poff[is_sh ? 0 : i];
  const bool valid = is_sh || slot_ok(off, c.blob_r, a.pool_bytes);
  const uint8_t* blob = is_sh ? a.shared : a.pool + (valid ? off : 0);
  const int64_t q = is_sh ? c.q_s : c.q_r;
  const int64_t sp = is_sh ? c.s_s : c.s_r;
  const int rloc = p * rpp + sub_row;
  const int r0 = row_lo + rloc;
  const bool in = rloc < a.rb && r0 < a.H;
  const int r = in ? r0 : row_lo;
  d.code = load_codes<BITS>(blob + 2 * q + r * (is_sh ? c.rowb_s : c.rowb_r) + seg0 * (kSegCodes * BITS / 8));
  const int si = r * (is_sh ? c.gpr_s : c.gpr_r) + seg0 / 2;
  d.sc = load_raw<SB>(blob + 3 * q + 2 * sp, si);
  d.bi = load_raw<SB>(blob + 3 * q + 5 * sp, si);
  d.i = live ? i : -1;
  d.rloc = live && in ? rloc : -1;
  d.valid = valid;
}

// This lane's byte offsets inside a routed and inside the shared blob for the
// single-pass layout (every task = rpp rows of one expert, np == 1): the code
// word, the scale and the bias of its segment of its row.
struct LaneOffsets {
  int64_t code_r, sc_r, bi_r, code_s, sc_s, bi_s;
  int rloc_r, rloc_s;   // row within the block, -1 if past the block or H
};

template <int BITS, int SB>
__device__ __forceinline__ LaneOffsets lane_offsets(const FusedArgs& a, const DownCtx& c, const RowLanes& rli,
                                                    const RowLanes& rls, int row_lo) {
  LaneOffsets o;
  const int sbsz = SB == kF32 ? 4 : 2;
  const int r0r = row_lo + rli.sub_row, r0s = row_lo + rls.sub_row;
  const bool inr = rli.sub_row < a.rb && r0r < a.H, ins = rls.sub_row < a.rb && r0s < a.H;
  const int rr = inr ? r0r : row_lo, rs = ins ? r0s : row_lo;
  o.code_r = 2 * c.q_r + rr * c.rowb_r + rli.seg0 * (kSegCodes * BITS / 8);
  o.sc_r = 3 * c.q_r + 2 * c.s_r + static_cast<int64_t>(rr * c.gpr_r + rli.seg0 / 2) * sbsz;
  o.bi_r = o.sc_r + 3 * c.s_r;
  o.code_s = 2 * c.q_s + rs * c.rowb_s + rls.seg0 * (kSegCodes * BITS / 8);
  o.sc_s = 3 * c.q_s + 2 * c.s_s + static_cast<int64_t>(rs * c.gpr_s + rls.seg0 / 2) * sbsz;
  o.bi_s = o.sc_s + 3 * c.s_s;
  o.rloc_r = inr ? rli.sub_row : -1;
  o.rloc_s = ins ? rls.sub_row : -1;
  return o;
}

// load_down_task for np == 1: the pair rank is the task index, the blob base
// is wave-uniform (scalar), the lane offsets are precomputed and the blob
// offset `off` (s.poff[i], read by the caller before any task's loads) is
// given.
template <int BITS, int SB>
__device__ __forceinline__ void load_down_task_1(DownTask<BITS>& d, int task, int ntask, const DownCtx& c,
                                                 const FusedArgs& a, int64_t off, const LaneOffsets& o) {
  const int k = a.k;
  const bool live = task < ntask;
  const int i = live ? task : k;            // a dead task re-reads the shared blob
  const bool is_sh = i == k;
  const bool valid = is_sh || slot_ok(off, c.blob_r, a.pool_bytes);
  const uint64_t bits = reinterpret_cast<uint64_t>(is_sh ? a.shared : a.pool + (valid ? off : 0));
  const uint64_t blob = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bits >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bits)));
  d.code = load_codes_g<BITS>(blob + (is_sh ? o.code_s : o.code_r));
  d.sc = load_raw_g<SB>(blob + (is_sh ? o.sc_s : o.sc_r));
  d.bi = load_raw_g<SB>(blob + (is_sh ? o.bi_s : o.bi_r));
  d.i = live ? i : -1;
  d.rloc = live ? (is_sh ? o.rloc_s : o.rloc_r) : -1;
  d.valid = valid;
}

// (slice, token) unit of this block: XCD x (blocks x, x + 8, ...) runs a
// contiguous range of units, token-minor, so the tokens of one slice read
// the slice's weight rows through one L2.  False for a block without a unit.
__device__ __forceinline__ bool unit_of(int nunits, int T, int* slice, int* t) {
  const int per = (nunits + kXcds - 1) / kXcds;
  const int idx = blockIdx.x / kXcds;
  if (idx >= per) return false;
  const int logical = (blockIdx.x % kXcds) * per + idx;
  if (logical >= nunits) return false;
  *slice = logical / T;
  *t = logical - *slice * T;
  return true;
}

// Per-unit constants of a block's down tasks (kept as separate locals by the
// callers: bundled in one struct, selects between its fields become loads
// through a selected address and the struct lands in scratch memory).
#define DOWN_SETUP(BITS, SB, a, slice, lane)                                  \
  const RowLanes rli = row_lanes((a).I, lane);                                \
  const RowLanes rls = row_lanes((a).SI, lane);                               \
  const int row_lo = (slice) * (a).rb;                                        \
  const DownCtx dc = down_ctx<BITS, SB>(a, rli, rls);                         \
  const int ntask = ((a).k + 1) * dc.np;                                      \
  const LaneOffsets lo = lane_offsets<BITS, SB>(a, dc, rli, rls, row_lo)

// Requests the loads of the round of tasks starting at `base` (this wave's
// kMaxDownPerWave of them); every blob offset is read before any load.
template <int BITS, int SB>
__device__ __forceinline__ void issue_down_round(DownTask<BITS> (&dt)[kMaxDownPerWave], int base, int ntask,
                                                 const DownCtx& dc, const LaneOffsets& lo, const RowLanes& rli,
                                                 const RowLanes& rls, int row_lo, const FusedArgs& a, const LdsB& s,
                                                 int wave) {
  if (dc.np == 1) {
    int64_t offs[kMaxDownPerWave];
#pragma unroll
    for (int q = 0; q < kMaxDownPerWave; ++q) {
      const int i = base + wave + q * kWaves;
      offs[q] = s.poff[i < a.k ? i : 0];
    }
#pragma unroll
    for (int q = 0; q < kMaxDownPerWave; ++q)
      load_down_task_1<BITS, SB>(dt[q], base + wave + q * kWaves, ntask, dc, a, offs[q], lo);
  } else {
#pragma unroll
    for (int q = 0; q < kMaxDownPerWave; ++q)
      load_down_task<BITS, SB>(dt[q], base + wave + q * kWaves, ntask, dc, row_lo, a, s, rli, rls);
  }
}

// Single launch: a block's down operands are copied into LDS by direct loads
// issued right after the block raises its flag, so that they arrive while it
// waits for every other block's.  Per wave, d_slots slots of
// [64 lanes x 16 code bytes][64 scale words][64 bias words]; lane l's code
// chunk sits at 16 l and its scale and bias words at 4 l.
constexpr int kDownSlotBytes = kWave * 16 + 2 * kWave * 4;

__device__ __forceinline__ uint8_t* down_slot(uint8_t* lds_raw, const FusedArgs& a, int wave, int q) {
  return lds_raw + a.lds_d_off + static_cast<size_t>(wave * a.d_slots + q) * kDownSlotBytes;
}

// Issues the direct loads of this wave's tasks and fills their rank, row and
// validity as load_down_task does; sc and bi hold, until read_down, the shift
// that selects a 2-byte value within its aligned word.  The blob of pair
// rank i < k is at slot[ids[i]] (the token's experts and the slot table, in
// LDS); a dead task (past ntask or past d_slots) gets rank -1 and no loads.
template <int BITS, int SB>
__device__ __forceinline__ void prefetch_down(DownTask<BITS> (&dt)[kMaxDownPerWave], uint8_t* lds_raw, int ntask,
                                              const DownCtx& c, int row_lo, const FusedArgs& a, const int64_t* slot,
                                              const int32_t* ids, const RowLanes& rli, const RowLanes& rls, int wave) {
  static_assert(BITS == 4, "one 16-byte code chunk per lane");
  const int k = a.k;
  const int sbsz = SB == kF32 ? 4 : 2;
#pragma unroll
  for (int q = 0; q < kMaxDownPerWave; ++q) {
    const int task = wave + q * kWaves;
    dt[q].i = -1;
    if (q >= a.d_slots || task >= ntask) continue;
    const int i = c.np == 1 ? task : task / c.np;
    const int p = c.np == 1 ? 0 : task - i * c.np;
    const bool is_sh = i == k;
    const int rpp = is_sh ? rls.rpp : rli.rpp;
    const int sub_row = is_sh ? rls.sub_row : rli.sub_row;
    const int seg0 = is_sh ? rls.seg0 : rli.seg0;
    const int64_t q_b = is_sh ? c.q_s : c.q_r;
    const int64_t s_b = is_sh ? c.s_s : c.s_r;
    const int64_t off = is_sh ? 0 : slot[ids[i]];
    const bool valid = is_sh || slot_ok(off, c.blob_r, a.pool_bytes);
    const uint8_t* blob = is_sh ? a.shared : a.pool + (valid ? off : 0);
    const int rloc = p * rpp + sub_row;
    const int r0 = row_lo + rloc;
    const bool in = rloc < a.rb && r0 < a.H;
    const int r = in ? r0 : row_lo;
    const uint32_t code = static_cast<uint32_t>(2 * q_b + r * (is_sh ? c.rowb_s : c.rowb_r) + seg0 * (kSegCodes * BITS / 8));
    const int64_t si = static_cast<int64_t>(r) * (is_sh ? c.gpr_s : c.gpr_r) + seg0 / 2;
    const uint32_t sc = static_cast<uint32_t>(3 * q_b + 2 * s_b + si * sbsz);
    const uint32_t bi = static_cast<uint32_t>(3 * q_b + 5 * s_b + si * sbsz);
    // the blob's data; an unusable blob reads zeros
    const u32x4 rs = raw_rsrc(blob, valid ? 3 * q_b + 6 * s_b : 0);
    uint8_t* sl = down_slot(lds_raw, a, wave, q);
    lds_load<16>(rs, sl, code, 0);
    lds_load<4>(rs, sl + kWave * 16, sc & ~3u, 0);
    lds_load<4>(rs, sl + kWave * 20, bi & ~3u, 0);
    dt[q].i = i;
    dt[q].rloc = in ? rloc : -1;
    dt[q].valid = valid;
    dt[q].sc = 8 * (sc & 2u);
    dt[q].bi = 8 * (bi & 2u);
  }
}

// The operands of prefetch_down's tasks, read back from LDS once the wave
// has waited for its direct loads.
template <int BITS, int SB>
__device__ __forceinline__ void read_down(DownTask<BITS> (&dt)[kMaxDownPerWave], uint8_t* lds_raw,
                                          const FusedArgs& a, int wave, int lane) {
  typedef __attribute__((address_space(3))) const uint32_t lds_w;
#pragma unroll
  for (int q = 0; q < kMaxDownPerWave; ++q) {
    if (dt[q].i < 0) continue;
    const lds_u8* sl = (const lds_u8*)(down_slot(lds_raw, a, wave, q));
    dt[q].code.w[0] = *(const lds_u32x4*)(sl + 16 * lane);
    const uint32_t sw = *(lds_w*)(sl + kWave * 16 + 4 * lane);
    const uint32_t bw = *(lds_w*)(sl + kWave * 20 + 4 * lane);
    dt[q].sc = SB == kF32 ? sw : sw >> dt[q].sc;
    dt[q].bi = SB == kF32 ? bw : bw >> dt[q].bi;
  }
}

__device__ __forceinline__ size_t h_row_of(int T, int k, int t, int i) {
  return i < k ? static_cast<size_t>(t) * k + i : static_cast<size_t>(T) * k + t;
}

// One round: each task's row segment dot with the token's h row, reduced over
// the row's lanes, into s.part.
template <int BITS, int SB>
__device__ __forceinline__ void compute_down_round(const DownTask<BITS> (&dt)[kMaxDownPerWave], const RowLanes& rli,
                                                   const RowLanes& rls, const FusedArgs& a, const LdsB& s, int T, int t,
                                                   int lane) {
  const int k = a.k, nseg = a.hs / kSegCodes;
#pragma unroll
  for (int q = 0; q < kMaxDownPerWave; ++q) {
    if (dt[q].i < 0) continue;
    const int i = dt[q].i;
    const bool is_sh = i == k;
    const int seg0 = is_sh ? rls.seg0 : rli.seg0;
    const int width = is_sh ? rls.width : rli.width;
    float hv[1][kSegCodes];
    float hs;
    if (s.h) {
      load_lds_seg(s.h + (static_cast<size_t>(i) * nseg + seg0) * kSegPad, 0, hv[0]);
      hs = ((const lds_f32*)(s.hsum))[i * nseg + seg0];
    } else {
      load_f32_seg(a.h + h_row_of(T, k, t, i) * a.hs, seg0, hv[0]);
      hs = seg_sum(hv[0]);
    }
    float qv[1];
    seg_qdot_nt<BITS, 1>(dt[q].code, hv, qv);
    float acc = 0.f;
    acc += seg_value(raw_value<SB>(dt[q].sc), raw_value<SB>(dt[q].bi), qv[0], hs);
    const float v = group_sum(acc, width);
    if ((lane % width) == 0 && dt[q].rloc >= 0) s.part[i * a.rb + dt[q].rloc] = dt[q].valid ? v : 0.f;
  }
}

// Segment sums of the staged h rows, in the order seg_sum uses.
__device__ __forceinline__ void h_segment_sums(const FusedArgs& a, const LdsB& s, int tid) {
  for (int j = tid; j < (a.k + 1) * (a.hs / kSegCodes); j += kThreads) {
    float v[kSegCodes];
    load_lds_seg(s.h + static_cast<size_t>(j) * kSegPad, 0, v);
    ((lds_f32*)(s.hsum))[j] = seg_sum(v);
  }
}

// The token's k + 1 h rows from the plain h buffer into s.h.
__device__ __forceinline__ void stage_h_plain(const FusedArgs& a, const LdsB& s, int T, int t, int tid) {
  const int k = a.k;
  const int r4 = a.hs / 4;                            // float4 per row
  const int n4 = (k + 1) * r4;
  lds_u32x4* dst = (lds_u32x4*)(s.h);
  // each thread's loads of a pass are all requested before any is stored
  constexpr int kPer = 4;
  for (int j0 = 0; j0 < n4; j0 += kPer * kThreads) {
    u32x4 v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int j = j0 + q * kThreads + tid;
      const int jc = j < n4 ? j : 0;
      const int i = jc / r4;
      v[q] = reinterpret_cast<const u32x4*>(a.h + h_row_of(T, k, t, i) * a.hs)[jc - i * r4];
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int j = j0 + q * kThreads + tid;
      if (j < n4) dst[(j >> 3) * (kSegPad / 4) + (j & 7)] = v[q];
    }
  }
  __syncthreads();
  h_segment_sums(a, s, tid);
  __syncthreads();
}

// Single launch (T = 1): the token's k + 1 h rows into s.h with loads that
// bypass this XCD's L2 (scope-of-device, the level the writers' stores were
// acknowledged at), and the shared-expert gate likewise.
__device__ __forceinline__ void stage_h_device(const FusedArgs& a, const LdsB& s, int tid) {
  const int k = a.k;
  const int r4 = a.hs / 4;
  const int n4 = (k + 1) * r4;
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(a.h, 0, (k + 1) * a.hs * 4, 0x00020000);
  constexpr int kScDevice = 16;   // cache policy: scope device (sc1)
  lds_u32x4* dst = (lds_u32x4*)(s.h);
  constexpr int kPer = 4;
  for (int j0 = 0; j0 < n4; j0 += kPer * kThreads) {
    u32x4 v[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int j = j0 + q * kThreads + tid;
      v[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hr, (j < n4 ? j : 0) * 16, 0, kScDevice));
    }
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int j = j0 + q * kThreads + tid;
      if (j < n4) dst[(j >> 3) * (kSegPad / 4) + (j & 7)] = v[q];
    }
  }
  if (tid == 0) s.sig[0] = __hip_atomic_load(a.sig, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  h_segment_sums(a, s, tid);
  __syncthreads();
}

// Ordered combine of the unit's rows: sum over ranks of weight * partial,
// then the gated shared expert.
template <int OUT>
__device__ __forceinline__ void combine_unit(const FusedArgs& a, const LdsB& s, int row_lo, int t, int tid) {
  const int k = a.k;
  for (int rloc = tid; rloc < a.rb; rloc += kThreads) {
    const int n = row_lo + rloc;
    if (n >= a.H) continue;
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc = fmaf(s.wts[i], s.part[i * a.rb + rloc], acc);
    acc = fmaf(s.sig[0], s.part[k * a.rb + rloc], acc);
    if constexpr (OUT == kF32) {
      const size_t j = static_cast<size_t>(t) * a.H + n;
      static_cast<float*>(a.out)[j] = acc;
      if (a.x_next) {
        // the stack step, as moe_residual_add takes it: fp32 sum, nearest-even bf16
        if (a.act_sz == 2) {
          const float xv = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.x)[j]) << 16);
          static_cast<uint16_t*>(a.x_next)[j] = f32_to_bf16(xv + acc);
        } else {
          static_cast<float*>(a.x_next)[j] = static_cast<const float*>(a.x)[j] + acc;
        }
      }
    } else {
      static_cast<uint16_t*>(a.out)[static_cast<size_t>(t) * a.H + n] = f32_to_bf16(acc);
    }
  }
}

// sigmoid(g . x) for one token on one wave (lane covers segments L, L + 64,
// ... as in the staged path).
template <int ACT>
__device__ __forceinline__ float shared_gate(const uint8_t* xrow, const uint8_t* gvec, int H, int lane) {
  const int nseg = H / kSegCodes;
  float acc = 0.f;
  if (lane < nseg) {
    float xv[kSegCodes], gv[kSegCodes];
    load_act_seg<ACT>(xrow, lane, xv);
    load_act_seg<ACT>(gvec, lane, gv);
#pragma unroll
    for (int c = 0; c < kSegCodes; ++c) acc = fmaf(xv[c], gv[c], acc);
  }
  acc = group_sum(acc, kWave);
  return sigmoid(acc);
}

// ---------------------------------------------------------------------------
// Launch A: phases R, K, G.  With ONE (T = 1 only) the same blocks then run
// launch B's work as well, with no second launch: h and the shared-expert
// gate are written with scope-of-device stores, every block raises a tagged
// completion flag once its stores are acknowledged, and after every block's
// flag is seen a block requests the codes of its down unit, stages h with
// scope-of-device loads, finishes its down rows and the ordered combine, and
// advances the epoch counters itself.  (Requesting the down codes before
// phase G instead made the waves wait for them there, about 2 us, and was no
// faster overall.)
template <int BITS, int SB, int ACT, int OUT = kF32, bool ONE = false>
__global__ __launch_bounds__(kThreadsA) void k_decode_a(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const LdsA s = carve_a(lds_raw, a);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: lets the compiler use scalar math
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  // bf16 activations with int4 codes take the v_dot2 segment dot
  constexpr bool kDot2 = ACT == kBF16 && BITS == 4;
  uint32_t spins = 0;
  bool timed_out = false;

  // This call's tag: this block's epoch counter plus one.  Every block's
  // counter holds the same value at the start of a call; launch B advances
  // them all, after every block of this launch has read its own.
  if (tid == 0) s.misc[1] = static_cast<int32_t>(a.epochs[blockIdx.x] + 1u);
  // ---- phase R setup: router rows on the first blocks (block-major,
  // kRouterRowsPerWave row groups per wave, so only a few blocks produce
  // logits); shared gate/up rows on the waves of the other blocks (wave-major,
  // spread over the machine).  The first task's weights are requested before
  // the x / slot-table copy below, so the two memory round trips overlap.
  const size_t xrow = static_cast<size_t>(H) * a.act_sz;
  const int nwaves = a.nb * kWavesA;
  const RowLanes rlh = row_lanes(H, lane);
  const int router_tasks = (E + rlh.rpp - 1) / rlh.rpp;
  const int router_waves = (router_tasks + kRouterRowsPerWave - 1) / kRouterRowsPerWave;
  const int router_blocks = min(a.nb, (router_waves + kWavesA - 1) / kWavesA);
  const int sh_tasks = (a.SI + rlh.rpp - 1) / rlh.rpp;
  const int bwave = blockIdx.x * kWavesA + wave;
  const int r_task0 = bwave * kRouterRowsPerWave;
  ActRaw<ACT> rw[kRouterRowsPerWave];
  int ee[kRouterRowsPerWave];
  auto load_router_rows = [&](int task) {
#pragma unroll
    for (int j = 0; j < kRouterRowsPerWave; ++j) {
      const int e = (task + j) * rlh.rpp + rlh.sub_row;
      ee[j] = task + j < router_tasks && e < E ? e : -1;
      load_act_raw<ACT>(static_cast<const uint8_t*>(a.router) + static_cast<size_t>(ee[j] < 0 ? 0 : e) * xrow,
                        rlh.seg0, rw[j]);
    }
  };
  if (r_task0 < router_tasks) load_router_rows(r_task0);
  const Planes pls = planes_of(H, a.SI, BITS, SB);
  const int64_t sh_row_bytes = static_cast<int64_t>(H) * BITS / 8;
  const int gpr = H / 64;
  const int sh_blocks = a.nb > router_blocks ? a.nb - router_blocks : a.nb;
  const int sh_b = a.nb > router_blocks ? static_cast<int>(blockIdx.x) - router_blocks : static_cast<int>(blockIdx.x);
  const int s_task0 = sh_b >= 0 ? wave * sh_blocks + sh_b : sh_tasks;
  Seg<BITS> scg, scu;
  uint32_t ssg = 0, ssu = 0, sbg = 0, sbu = 0;
  auto load_shared_row = [&](int task) {
    const int rr0 = task * rlh.rpp + rlh.sub_row;
    const int rr = rr0 < a.SI ? rr0 : 0;   // loads stay unconditional; the store is masked
    const int64_t qo = rr * sh_row_bytes + static_cast<int64_t>(rlh.seg0) * (kSegCodes * BITS / 8);
    scg = load_codes<BITS>(a.shared + qo);
    scu = load_codes<BITS>(a.shared + pls.q + qo);
    const size_t si = static_cast<size_t>(rr) * gpr + rlh.seg0 / 2;
    ssg = load_raw<SB>(a.shared + 3 * pls.q, si);
    ssu = load_raw<SB>(a.shared + 3 * pls.q + pls.s, si);
    sbg = load_raw<SB>(a.shared + 3 * pls.q + 3 * pls.s, si);
    sbu = load_raw<SB>(a.shared + 3 * pls.q + 4 * pls.s, si);
  };
  if (s_task0 < sh_tasks) load_shared_row(s_task0);
  {
    // x and the slot table into LDS; each round requests its elements of both
    // before storing any, so the copy costs one memory round trip per round
    const int n16 = T * H * a.act_sz / 16;
    const u32x4* src = static_cast<const u32x4*>(a.x);
    u32x4* dst = reinterpret_cast<u32x4*>(s.x);
    const int n = n16 > E ? n16 : E;
    for (int i0 = 0; i0 < n; i0 += 2 * kThreadsA) {
      u32x4 xv[2];
      int64_t sv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * kThreadsA + tid;
        xv[u] = src[i < n16 ? i : 0];
        sv[u] = a.slot_table[i < E ? i : 0];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * kThreadsA + tid;
        if (i < n16) dst[i] = xv[u];
        if (i < E) s.slot[i] = sv[u];
      }
    }
  }
  __syncthreads();
  const uint32_t tag = static_cast<uint32_t>(s.misc[1]);
  const int gwave = wave * a.nb + blockIdx.x;
  auto put_h = [&](size_t row, int r, float v) {
    if constexpr (ONE) __hip_atomic_store(a.h + row * a.hs + r, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else a.h[row * a.hs + r] = v;
  };

  // ---- phase R
  for (int task = r_task0; task < router_tasks; task += nwaves * kRouterRowsPerWave) {
    if (task != r_task0) load_router_rows(task);
#pragma unroll
    for (int j = 0; j < kRouterRowsPerWave; ++j) {
      if (task + j >= router_tasks) break;
      const bool active = ee[j] >= 0;
      float r[kSegCodes];
      act_raw_f32<ACT>(rw[j], r);
      for (int t = 0; t < T; ++t) {
        float acc = 0.f;
        if (active) {
          float v[kSegCodes];
          load_act_seg<ACT>(s.x + t * xrow, rlh.seg0, v);
#pragma unroll
          for (int c = 0; c < kSegCodes; ++c) acc = fmaf(v[c], r[c], acc);
        }
        acc = group_sum(acc, rlh.width);
        if (active)   // every lane of the row holds the sum: each stores some of the copies
          for (int rep = lane % rlh.width; rep < kFusedReplicas; rep += rlh.width)
            store_tagged(a.lg + (static_cast<size_t>(rep) * T + t) * E + ee[j], acc, tag);
      }
    }
  }
  for (int task = s_task0; task < sh_tasks; task += sh_blocks * kWavesA) {
    if (task != s_task0) load_shared_row(task);
    const int rr = task * rlh.rpp + rlh.sub_row;
    const bool ok = rr < a.SI;
    if constexpr (kDot2) {
      const QPairs pg = qpairs_bf16(scg), pu = qpairs_bf16(scu);
      for (int t = 0; t < T; ++t) {
        ActRaw<kBF16> xr;
        load_lds_act_bf16(s.x + t * xrow, rlh.seg0, xr);
        const float xs = xsum_bf16(xr);
        float accg = 0.f, accu = 0.f;
        accg += seg_value_d2(raw_value<SB>(ssg), raw_value<SB>(sbg), dot2_seg(pg, xr), xs);
        accu += seg_value_d2(raw_value<SB>(ssu), raw_value<SB>(sbu), dot2_seg(pu, xr), xs);
        float g, u;
        gu_sums(accg, accu, rlh.width, g, u);
        if (ok && (lane % rlh.width) == 0) put_h(static_cast<size_t>(T) * k + t, rr, silu(g) * u);
      }
    } else {
      for (int t = 0; t < T; ++t) {
        float v[1][kSegCodes];
        load_act_seg<ACT>(s.x + t * xrow, rlh.seg0, v[0]);
        const float xs = seg_sum(v[0]);
        float qg[1], qu[1];
        seg_qdot_nt<BITS, 1>(scg, v, qg);
        seg_qdot_nt<BITS, 1>(scu, v, qu);
        float accg = 0.f, accu = 0.f;
        accg += seg_value(raw_value<SB>(ssg), raw_value<SB>(sbg), qg[0], xs);
        accu += seg_value(raw_value<SB>(ssu), raw_value<SB>(sbu), qu[0], xs);
        float g, u;
        gu_sums(accg, accu, rlh.width, g, u);
        if (ok && (lane % rlh.width) == 0) put_h(static_cast<size_t>(T) * k + t, rr, silu(g) * u);
      }
    }
  }
  // sigmoid(g . x_t) for launch B on block 0
  if (blockIdx.x == 0 && wave == kWavesA - 1) {
    for (int t = 0; t < T; ++t) {
      const float g = shared_gate<ACT>(s.x + t * xrow, a.shared + a.shared_stride, H, lane);
      if (lane == 0) {
        if constexpr (ONE) __hip_atomic_store(a.sig + t, g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else a.sig[t] = g;
      }
    }
  }

  // ---- phase K: gather all logits (each word checked against this call's
  // tag, re-read until every one has arrived), top-k, dispatch
  const int rep = blockIdx.x % kFusedReplicas;
  for (;;) {
    int missing = 0;
    for (int i = tid; i < T * E; i += kThreadsA) {
      const uint64_t w = load_tagged(a.lg + static_cast<size_t>(rep) * T * E + i);
      if (static_cast<uint32_t>(w >> 32) != tag) missing = 1;
      else s.lg[i] = __uint_as_float(static_cast<uint32_t>(w));
    }
    if (!__syncthreads_or(missing)) break;
    if (++spins > a.spin_limit) { timed_out = true; break; }
    __builtin_amdgcn_s_sleep(2);
  }
  for (int t = wave; t < T; t += kWavesA)
    topk_wave(s.lg + static_cast<size_t>(t) * E, E, k, lane, s.cand + wave * kCandMax, s.ids + t * k,
              s.vals + t * k);
  if (T == 1) {
    // one token: its k experts are distinct; order them by id with a rank count
    if (wave == 0) {
      int e = lane < k ? s.ids[lane] : 0x7fffffff;
      e = e >= 0 && e < E ? e : 0;
      int r = 0;
      for (int j = 0; j < k; ++j) r += s.ids[j] < e ? 1 : 0;
      if (lane < k) {
        s.uniq[r] = e;
        s.pidx[r] = lane;
        s.uranks[r] = static_cast<uint64_t>(lane + 1);
      }
      if (lane == 0) s.misc[0] = k;
    }
    __syncthreads();
  } else {
    for (int e = tid; e < E; e += kThreadsA) s.umap[e] = -1;
    __syncthreads();
    for (int p = tid; p < T * k; p += kThreadsA) {
      const int e = s.ids[p];
      s.ids[p] = e >= 0 && e < E ? e : 0;           // ids come from [0, E) by construction
      s.umap[s.ids[p]] = 0;                         // mark
    }
    __syncthreads();
    if (wave == 0) {
      int base = 0;
      for (int c0 = 0; c0 < E; c0 += kWave) {
        const int e = c0 + lane;
        const bool used = e < E && s.umap[e] == 0;
        const uint64_t m = __ballot(used);
        const int pos = base + __popcll(m & lane_mask_lt(lane));
        if (used) { s.uniq[pos] = e; s.umap[e] = pos; }
        base += __popcll(m);
      }
      if (lane == 0) s.misc[0] = base;
    }
    __syncthreads();
    const int Ud = s.misc[0];
    for (int i = tid; i < Ud * T; i += kThreadsA) s.pidx[i] = -1;
    __syncthreads();
    for (int p = tid; p < T * k; p += kThreadsA) s.pidx[s.umap[s.ids[p]] * T + p / k] = p % k;
    __syncthreads();
    // phase-G work per distinct expert: a row's loads plus one dot per token
    // that uses it; prefix sums so that every wave takes an equal share
    if (wave == 0) {
      int carry = 0;
      for (int u0 = 0; u0 < Ud; u0 += kWave) {
        const int u = u0 + lane;
        int c = 0;
        if (u < Ud) {
          c = kRowCost;
          uint64_t rk = 0;
          for (int t = 0; t < T; ++t) {
            const int i = s.pidx[u * T + t];
            c += i >= 0 ? 1 : 0;
            rk |= static_cast<uint64_t>(i + 1) << (8 * t);
          }
          s.uranks[u] = rk;
        }
        int incl = c;
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) {
          const int o = __shfl_up(incl, m, kWave);
          if (lane >= m) incl += o;
        }
        if (u < Ud) s.ucost[u + 1] = carry + incl;
        carry += __shfl(incl, kWave - 1, kWave);
      }
      if (lane == 0) s.ucost[0] = 0;
    }
    __syncthreads();
  }
  const int U = s.misc[0];
  if (blockIdx.x == 0) {
    // routing record for launch B (and the optional outputs)
    for (int p = tid; p < T * k; p += kThreadsA) {
      a.wts[p] = s.vals[p];
      if (a.ids_out) a.ids_out[p] = s.ids[p];
      if (a.wts_out) a.wts_out[p] = s.vals[p];
    }
    for (int i = tid; i < U * T; i += kThreadsA) a.pidx[i] = s.pidx[i];
    for (int i = tid; i < U; i += kThreadsA) {
      a.uniq[i] = s.uniq[i];
      a.uoff[i] = s.slot[s.uniq[i]];
    }
    if (tid == 0) *a.ucount = U;
  }
  // ---- single launch: the routing of this block's down unit
  int slice = 0, ut = 0;
  bool has_unit = false;
  LdsB sb{};
  if constexpr (ONE) {
    sb = carve_b(lds_raw + a.lds_b_off, a);
    if (tid < k) {
      sb.poff[tid] = s.slot[s.ids[tid]];
      sb.wts[tid] = s.vals[tid];
    }
    has_unit = unit_of(a.nslice, 1, &slice, &ut);
  }
  // ---- phase G: routed gate/up rows, flattened over (expert, row group)
  {
    const Planes pl = planes_of(H, a.I, BITS, SB);
    const int64_t row_bytes = static_cast<int64_t>(H) * BITS / 8;
    const int seg_bytes = kSegCodes * BITS / 8;
    const int gpr = H / 64;
    const int groups_per_expert = a.I / rlh.rpp;
    const int total = U * groups_per_expert;
    int g_lo, g_hi;
    if (T == 1) {
      // every unit costs the same
      const int per_wave = (total + nwaves - 1) / nwaves;
      g_lo = min(total, gwave * per_wave);
      g_hi = min(total, g_lo + per_wave);
    } else {
      // equal shares of the work: unit (u, group) costs ucost[u + 1] - ucost[u]
      // over groups_per_expert; a share starts at the first unit that starts
      // at or after its cost position
      const int64_t W = static_cast<int64_t>(s.ucost[U]) * groups_per_expert;
      auto unit_at = [&](int64_t x) {
        if (x >= W) return total;
        int lo = 0, hi = U - 1;   // last u with ucost[u] * gpe <= x
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (static_cast<int64_t>(s.ucost[mid]) * groups_per_expert <= x) lo = mid;
          else hi = mid - 1;
        }
        const int64_t c = s.ucost[lo + 1] - s.ucost[lo];   // cost of one unit of expert lo
        const int64_t i = (x - static_cast<int64_t>(s.ucost[lo]) * groups_per_expert + c - 1) / c;
        return lo * groups_per_expert + static_cast<int>(i);
      };
      g_lo = unit_at(W * gwave / nwaves);
      g_hi = unit_at(W * (gwave + 1) / nwaves);
    }
    // per-token segment sums of x (the lane's segment is the same in every
    // row), once per wave, in a wave-private table in the logits area, which
    // nothing reads after top-k
    lds_f32* const xs_tab = (lds_f32*)(s.lg) + wave * T * kWave;
    if constexpr (kDot2) {
      for (int t = 0; t < T; ++t) {
        ActRaw<kBF16> xr;
        load_lds_act_bf16(s.x + t * xrow, rlh.seg0, xr);
        xs_tab[t * kWave + lane] = xsum_bf16(xr);
      }
    }
    // Rows go in batches of kBatch; the next batch's loads are requested
    // before the current batch is computed (two register sets, alternating).
    constexpr int kBatch = 4;
    struct Batch {
      Seg<BITS> cg[kBatch], cu[kBatch];
      uint32_t sg[kBatch], su[kBatch], bg[kBatch], bu[kBatch];
      int uu[kBatch], rr[kBatch];
      bool vv[kBatch];
    };
    // every row of a batch is requested before any is used: no branches on
    // the loads (a row past the end repeats the first one, an unusable blob
    // reads blob 0; both are masked at the store) and raw scale bits
    auto load_batch = [&](Batch& B, int g0) {
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int g = g0 + b;
        const bool live = g < g_hi;
        const int gc = live ? g : g_lo;
        const int u = gc / groups_per_expert;
        const int r = (gc % groups_per_expert) * rlh.rpp + rlh.sub_row;
        const int64_t off = s.slot[s.uniq[u]];
        const bool valid = slot_ok(off, pl.blob, a.pool_bytes);
        B.uu[b] = live ? u : -1;
        B.rr[b] = r;
        B.vv[b] = valid;
        if (live && !valid && lane == 0) raise_error(a.ctrl, kErrRange);
        const uint8_t* blob = a.pool + (valid ? off : 0);
        const int64_t qo = r * row_bytes + static_cast<int64_t>(rlh.seg0) * seg_bytes;
        B.cg[b] = load_codes<BITS>(blob + qo);
        B.cu[b] = load_codes<BITS>(blob + pl.q + qo);
        const size_t si = static_cast<size_t>(r) * gpr + rlh.seg0 / 2;
        B.sg[b] = load_raw<SB>(blob + 3 * pl.q, si);
        B.su[b] = load_raw<SB>(blob + 3 * pl.q + pl.s, si);
        B.bg[b] = load_raw<SB>(blob + 3 * pl.q + 3 * pl.s, si);
        B.bu[b] = load_raw<SB>(blob + 3 * pl.q + 4 * pl.s, si);
      }
    };
    auto compute_batch = [&](const Batch& B, auto wtag) {
      // row sums: width known at compile time for full-wave rows
      constexpr int W = decltype(wtag)::value;
      if constexpr (kDot2) {
        // rows outer: each row's codes become bf16 pairs once for all its
        // tokens; the tokens that use the row come from its packed ranks
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          if (B.uu[b] < 0) continue;
          const uint64_t rkv = s.uranks[B.uu[b]];
          uint64_t rk = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(rkv >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(rkv)));
          const QPairs pg = qpairs_bf16(B.cg[b]), pu = qpairs_bf16(B.cu[b]);
          const float sgv = raw_value<SB>(B.sg[b]), bgv = raw_value<SB>(B.bg[b]);
          const float suv = raw_value<SB>(B.su[b]), buv = raw_value<SB>(B.bu[b]);
          while (rk != 0) {
            const int sh = __builtin_ctzll(rk) & ~7;
            const int t = sh >> 3;
            const int i = static_cast<int>((rk >> sh) & 0xffu) - 1;
            rk &= ~(0xffull << sh);
            ActRaw<kBF16> xr;
            load_lds_act_bf16(s.x + t * xrow, rlh.seg0, xr);
            const float xs = xs_tab[t * kWave + lane];
            float accg = 0.f, accu = 0.f;
            accg += seg_value_d2(sgv, bgv, dot2_seg(pg, xr), xs);
            accu += seg_value_d2(suv, buv, dot2_seg(pu, xr), xs);
            float g, u;
            gu_sums_w<W>(accg, accu, rlh.width, g, u);
            if ((lane % rlh.width) == 0)
              put_h(static_cast<size_t>(t) * k + i, B.rr[b], B.vv[b] ? silu(g) * u : 0.f);
          }
        }
      } else {
        for (int t = 0; t < T; ++t) {
          float v[1][kSegCodes];
          load_act_seg<ACT>(s.x + t * xrow, rlh.seg0, v[0]);
          const float xs = seg_sum(v[0]);
#pragma unroll
          for (int b = 0; b < kBatch; ++b) {
            if (B.uu[b] < 0) continue;
            const int i = s.pidx[B.uu[b] * T + t];
            if (i < 0) continue;                      // token t does not use this expert
            float qg[1], qu[1];
            seg_qdot_nt<BITS, 1>(B.cg[b], v, qg);
            seg_qdot_nt<BITS, 1>(B.cu[b], v, qu);
            float accg = 0.f, accu = 0.f;
            accg += seg_value(raw_value<SB>(B.sg[b]), raw_value<SB>(B.bg[b]), qg[0], xs);
            accu += seg_value(raw_value<SB>(B.su[b]), raw_value<SB>(B.bu[b]), qu[0], xs);
            float g, u;
            gu_sums_w<W>(accg, accu, rlh.width, g, u);
            if ((lane % rlh.width) == 0)
              put_h(static_cast<size_t>(t) * k + i, B.rr[b], B.vv[b] ? silu(g) * u : 0.f);
          }
        }
      }
    };
    auto run = [&](auto wtag) {
      Batch b0, b1;
      load_batch(b0, g_lo);
      for (int g0 = g_lo; g0 < g_hi; g0 += 2 * kBatch) {
        if (g0 + kBatch < g_hi) load_batch(b1, g0 + kBatch);
        compute_batch(b0, wtag);
        if (g0 + kBatch >= g_hi) break;
        if (g0 + 2 * kBatch < g_hi) load_batch(b0, g0 + 2 * kBatch);
        compute_batch(b1, wtag);
      }
    };
    if (g_lo < g_hi) {
      if (rlh.width == kWave) run(IntC<kWave>{});
      else run(IntC<0>{});
    }
  }
  if constexpr (ONE) {
    // this block's h and gate stores are acknowledged (scope device), then its
    // flag goes out in every replica; wait for every block's flag
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid < kFusedReplicas)
      __hip_atomic_store(a.gflags + tid * kFusedMaxBlocks + blockIdx.x, tag, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    // this block's down operands travel to LDS during the wait
    DownTask<BITS> dt[kMaxDownPerWave];
    if (has_unit) {
      DOWN_SETUP(BITS, SB, a, slice, lane);
      (void)lo;
      prefetch_down<BITS, SB>(dt, lds_raw, ntask, dc, row_lo, a, s.slot, s.ids, rli, rls, wave);
    }
    const uint32_t* fl = a.gflags + (blockIdx.x % kFusedReplicas) * kFusedMaxBlocks;
    uint32_t fspins = 0;
    bool flags_out = false;
    for (;;) {
      int missing = 0;
      for (int j = tid; j < a.nb; j += kThreadsA)
        if (__hip_atomic_load(fl + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) missing = 1;
      if (!__syncthreads_or(missing)) break;
      if (++fspins > a.spin_limit) { flags_out = true; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    if (flags_out) {
      timed_out = true;
      __builtin_amdgcn_s_waitcnt(0);   // no direct load outlives the block
    }
    if (has_unit && !flags_out) {
      // stage h (its loads wait for the direct ones too: one counter, in
      // order), then the down rows from LDS
      const RowLanes rli = row_lanes(a.I, lane);
      const RowLanes rls = row_lanes(a.SI, lane);
      const int row_lo = slice * a.rb;
      stage_h_device(a, sb, tid);
      __builtin_amdgcn_s_waitcnt(0);
      read_down<BITS, SB>(dt, lds_raw, a, wave, lane);
      compute_down_round<BITS, SB>(dt, rli, rls, a, sb, 1, 0, lane);
      __syncthreads();
      combine_unit<OUT>(a, sb, row_lo, 0, tid);
    }
    // every block has read its epoch counter (at its start, before its flag):
    // advance them, the ones past the grid by block 0
    if (tid == 0) a.epochs[blockIdx.x] = a.epochs[blockIdx.x] + 1u;
    if (blockIdx.x == 0)
      for (int j = a.nb + tid; j < kFusedMaxBlocks; j += kThreadsA) a.epochs[j] = a.epochs[j] + 1u;
  }
  if (timed_out && lane == 0) raise_error(a.ctrl, kErrTimeout);
}

// ---------------------------------------------------------------------------
// Launch B: one block per (slice of rb output rows, token): the slice's down
// rows of the token's k experts and of the shared expert, then the ordered
// combine.  A block's partial sums are all its own, and the token's k + 1 h
// rows are staged in LDS once.
template <int BITS, int SB, int OUT>
__global__ __launch_bounds__(kThreads) void k_decode_b(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const LdsB s = carve_b(lds_raw, a);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: lets the compiler use scalar math
  const int T = a.T, k = a.k;
  // Retire launch A's tag: every block of A has finished, so none can still
  // read its epoch counter; each thread advances its own counters.
  if (blockIdx.x == 0)
    for (int j = tid; j < kFusedMaxBlocks; j += kThreads) a.epochs[j] = a.epochs[j] + 1u;
  int slice, t;
  if (!unit_of(a.nslice * T, T, &slice, &t)) return;
  // the token's routing: blob offsets by rank, weights, gate; every element
  // requested before any is stored (a rank that no distinct expert claims
  // keeps offset -1, which slot_ok rejects)
  if (tid < k) s.poff[tid] = -1;
  __syncthreads();
  {
    const int U = *a.ucount;
    const int n = a.umax > k ? a.umax : k;
    for (int u0 = 0; u0 < n; u0 += kThreads) {
      const int u = u0 + tid;
      const int uc = u < a.umax ? u : 0;
      const int32_t i = __builtin_nontemporal_load(a.pidx + uc * T + t);
      const int64_t off = __builtin_nontemporal_load(a.uoff + uc);
      const float wt = __builtin_nontemporal_load(a.wts + t * k + (u < k ? u : 0));
      const float sg = __builtin_nontemporal_load(a.sig + t);
      const bool claim = u < a.umax && u < U && i >= 0 && i < k;
      if (claim) s.poff[i] = off;
      if (u < k) s.wts[u] = wt;
      if (u == 0) s.sig[0] = sg;
    }
  }
  __syncthreads();
  DOWN_SETUP(BITS, SB, a, slice, lane);
  DownTask<BITS> dt[kMaxDownPerWave];
  for (int base = 0; base < ntask; base += kWaves * kMaxDownPerWave) {
    // codes of this round's tasks, all requested before any compute
    issue_down_round<BITS, SB>(dt, base, ntask, dc, lo, rli, rls, row_lo, a, s, wave);
    // the token's h rows into LDS once, while the codes above are in flight
    if (s.h && base == 0) stage_h_plain(a, s, T, t, tid);
    compute_down_round<BITS, SB>(dt, rli, rls, a, s, T, t, lane);
  }
  __syncthreads();
  combine_unit<OUT>(a, s, row_lo, t, tid);
}

size_t lds_bytes_a(int T, int H, int E, int k, int umax, int act_sz) {
  size_t o = 0;
  auto take = [&](size_t n) { o += (n + 15) / 16 * 16; };
  take(static_cast<size_t>(T) * H * act_sz);
  take(lg_floats(T, E) * 4);
  take(static_cast<size_t>(T) * k * 4);
  take(static_cast<size_t>(T) * k * 4);
  take(static_cast<size_t>(E) * 8);
  take(static_cast<size_t>(E) * 4);
  take(static_cast<size_t>(umax) * 4);
  take(static_cast<size_t>(umax) * T * 4);
  take(static_cast<size_t>(umax + 1) * 4);
  take(static_cast<size_t>(umax) * 8);
  take(kWavesA * kCandMax * 8);
  take(16 * 4);
  return o;
}

size_t lds_bytes_b(int k, int rb, int hs) {
  size_t o = 0;
  auto take = [&](size_t n) { o += (n + 15) / 16 * 16; };
  take(static_cast<size_t>(k) * 8);
  take(static_cast<size_t>(k) * 4);
  take(4);
  take(static_cast<size_t>(k + 1) * rb * 4);
  if (h_staged(k, hs)) {
    take(h_stage_floats(k, hs) * 4);
    take(static_cast<size_t>(k + 1) * (hs / kSegCodes) * 4);
  }
  return o;
}

}  // namespace

template <int BITS, int SB, int ACT, int OUT>
static int launch_variant(const FusedArgs& a, const FusedPlan& p, hipStream_t stream) {
  if (BITS == 4 && p.one) {
    // int4 only (the int8 variant would not fit its registers)
    if constexpr (BITS == 4)
      launch_kernel(k_decode_a<BITS, SB, ACT, OUT, true>, dim3(p.nb), dim3(kThreadsA), p.lds_one, stream, a);
  } else {
    launch_kernel(k_decode_a<BITS, SB, ACT>, dim3(p.nb), dim3(kThreadsA), p.lds, stream, a);
    launch_kernel(k_decode_b<BITS, SB, OUT>, dim3(p.nb_b), dim3(kThreads), p.lds_b, stream, a);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <int BITS, int SB, int ACT, int OUT>
static int occupancy_variant(size_t lds, int* blocks, bool one) {
  hipError_t e = hipErrorInvalidValue;
  if constexpr (BITS == 4) {
    if (one) {
      // the single launch may take more than the default 64 KB of dynamic LDS
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_decode_a<BITS, SB, ACT, OUT, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_decode_a<BITS, SB, ACT, OUT, true>, kThreadsA, lds);
    }
  }
  if (!one) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_decode_a<BITS, SB, ACT>, kThreadsA, lds);
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

#define FUSED_DISPATCH(FN, ...)                                                            \
  do {                                                                                     \
    const int b_ = d.bits, s_ = d.sb_dtype, a_ = d.act_dtype, o_ = d.out_dtype;            \
    if (b_ == 4 && s_ == kBF16 && a_ == kBF16 && o_ == kF32) return FN<4, kBF16, kBF16, kF32>(__VA_ARGS__);   \
    if (b_ == 4 && s_ == kBF16 && a_ == kBF16 && o_ == kBF16) return FN<4, kBF16, kBF16, kBF16>(__VA_ARGS__); \
    if (b_ == 8 && s_ == kBF16 && a_ == kBF16 && o_ == kF32) return FN<8, kBF16, kBF16, kF32>(__VA_ARGS__);   \
    if (b_ == 8 && s_ == kBF16 && a_ == kBF16 && o_ == kBF16) return FN<8, kBF16, kBF16, kBF16>(__VA_ARGS__); \
    if (b_ == 4 && s_ == kF32 && a_ == kF32 && o_ == kF32) return FN<4, kF32, kF32, kF32>(__VA_ARGS__);       \
    if (b_ == 8 && s_ == kF32 && a_ == kF32 && o_ == kF32) return FN<8, kF32, kF32, kF32>(__VA_ARGS__);       \
    return MOE_EINVAL;                                                                     \
  } while (0)

static int fused_occupancy(const moe_desc& d, size_t lds, int* blocks, bool one) {
  FUSED_DISPATCH(occupancy_variant, lds, blocks, one);
}

static int fused_launch(const moe_desc& d, const FusedArgs& a, const FusedPlan& p, hipStream_t s) {
  FUSED_DISPATCH(launch_variant, a, p, s);
}

bool fused_supported(const moe_desc& d, int T) {
  if (T < 1 || T > kFusedMaxT) return false;
  const int s = d.sb_dtype, a = d.act_dtype;
  return (s == kBF16 && a == kBF16) || (s == kF32 && a == kF32 && d.out_dtype == kF32);
}

// Rows per wave pass of row_lanes (host side).
static int row_lanes_rpp(int cols) {
  const int spr = cols / kSegCodes;
  return spr >= kWave ? 1 : kWave / spr;
}

int fused_plan(const moe_desc& d, int T, FusedPlan* plan) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ENODEV;
  const int act_sz = d.act_dtype == kF32 ? 4 : 2;
  const int umax = T * d.top_k < d.n_experts ? T * d.top_k : d.n_experts;
  const int hs = d.inter > d.shared_inter ? d.inter : d.shared_inter;
  const size_t lds = lds_bytes_a(T, d.hidden, d.n_experts, d.top_k, umax, act_sz);
  if (lds > 64 * 1024) return MOE_EINVAL;
  // launch A: one resident block per CU
  for (int per_cu = 1; per_cu >= 1; --per_cu) {
    const int nb = cus * per_cu;
    if (nb > kFusedMaxBlocks) continue;
    int fit = 0;
    if (fused_occupancy(d, lds, &fit, false) != MOE_OK) return MOE_EHIP;
    if (fit >= per_cu) {
      plan->nb = nb;
      plan->lds = lds;
      plan->umax = umax;
      // launch B: one block per (slice, token); slices of a few output rows,
      // wider as T grows, so that the grid stays at one to two blocks per CU
      const int rb1 = (d.hidden + cus - 1) / cus;
      plan->rb_b = rb1 * ((T + 1) / 2);
      plan->nslice = (d.hidden + plan->rb_b - 1) / plan->rb_b;
      plan->nb_b = (plan->nslice * T + kXcds - 1) / kXcds * kXcds;
      plan->lds_b = lds_bytes_b(d.top_k, plan->rb_b, hs);
      // T = 1 in one launch: every down unit on its own block of launch A, the
      // h rows staged in LDS, one round of down tasks per wave, and a resident
      // block per CU with both phases' LDS
      // (plus the prefetched down operands; blob offsets fit 32 bits)
      plan->one = false;
      const int rpp_i = row_lanes_rpp(d.inter), rpp_s = row_lanes_rpp(d.shared_inter);
      const int rpp_min = rpp_i < rpp_s ? rpp_i : rpp_s;
      const int ntask = (d.top_k + 1) * ((plan->rb_b + rpp_min - 1) / rpp_min);
      plan->d_slots = (ntask + kWaves - 1) / kWaves;
      plan->lds_one = (lds + 15) / 16 * 16 + (plan->lds_b + 15) / 16 * 16 +
                      static_cast<size_t>(kWaves) * plan->d_slots * kDownSlotBytes;
      int lds_max = 0;
      if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return MOE_ENODEV;
      const int64_t ext = planes_of(d.hidden, hs, d.bits, d.sb_dtype).blob;
      if (T == 1 && d.bits == 4 && plan->nslice <= nb && h_staged(d.top_k, hs) &&
          plan->lds_one <= static_cast<size_t>(lds_max) && ntask <= kWaves * kMaxDownPerWave && ext < (1ll << 31)) {
        int fit1 = 0;
        if (fused_occupancy(d, plan->lds_one, &fit1, true) == MOE_OK && fit1 >= 1) plan->one = true;
      }
      return MOE_OK;
    }
  }
  return MOE_EINVAL;
}

int launch_decode_fused(const Call& c, const FusedPlan& plan) {
  const moe_desc& d = c.d;
  FusedArgs a;
  a.x = c.x;
  a.router = c.router_w;
  a.slot_table = c.slot_table;
  a.pool = c.pool;
  a.shared = c.shared;
  a.out = c.out;
  a.x_next = c.x_next;
  a.ids_out = c.ids_out;
  a.wts_out = c.wts_out;
  a.lg = reinterpret_cast<uint64_t*>(c.ws + c.L.f_lg);
  a.h = reinterpret_cast<float*>(c.ws + c.L.h);
  a.wts = reinterpret_cast<float*>(c.ws + c.L.wts);
  a.sig = reinterpret_cast<float*>(c.ws + c.L.gate);
  a.ucount = reinterpret_cast<int32_t*>(c.ws + c.L.ucount);
  a.uniq = reinterpret_cast<int32_t*>(c.ws + c.L.uniq);
  a.uoff = reinterpret_cast<int64_t*>(c.ws + c.L.f_uoff);
  a.pidx = reinterpret_cast<int32_t*>(c.ws + c.L.f_pidx);
  a.ctrl = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  a.pool_bytes = d.pool_bytes;
  a.shared_stride = d.shared_stride;
  a.T = c.T;
  a.H = d.hidden;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.I = d.inter;
  a.SI = d.shared_inter;
  a.hs = c.L.hstride;
  a.nb = plan.nb;
  a.rb = plan.rb_b;
  a.nslice = plan.nslice;
  a.epochs = reinterpret_cast<uint32_t*>(c.ws + c.L.f_epoch);
  a.gflags = reinterpret_cast<uint32_t*>(c.ws + c.L.f_gflag);
  a.lds_b_off = (plan.lds + 15) / 16 * 16;
  a.lds_d_off = a.lds_b_off + (plan.lds_b + 15) / 16 * 16;
  a.d_slots = plan.d_slots;
  a.umax = plan.umax;
  a.act_sz = d.act_dtype == kF32 ? 4 : 2;
  a.spin_limit = 1u << 20;
  return fused_launch(d, a, plan, c.stream);
}

}  // namespace moe
