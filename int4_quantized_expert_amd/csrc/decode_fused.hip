// Fused single-launch decode of one MoE layer (T <= 8 tokens), gfx950.
//
// The staged path needs six dependent launches per layer; at decode sizes the
// launch gaps and the dependent-load chains between them cost more than the
// 21.6 MB the 80B-shaped layer has to stream.  Here one persistent grid whose
// blocks are all resident at once runs the whole layer:
//
//   R  router rows (logits), shared-expert gate/up rows, sigmoid(g . x)
//   K  every block gathers all logits and computes top-k, the renormalised
//      weights and the expert -> token dispatch itself (no extra exchange)
//   G  routed gate/up rows + SwiGLU, spread over all waves; the down-projection
//      codes each block will need are requested before this compute starts
//   D  each block owns a slice of output rows: down rows of every chosen
//      expert + the shared one, then the ordered combine, written to out
//
// Data crossing blocks (logits, h) travels as 64-bit words holding the float
// bits and a per-call tag, written and read with relaxed device-scope atomics.
// A word is valid when its tag matches, so no fence is needed (an agent-scope
// release on this chip writes back the L2 and costs microseconds).  The tag is
// the workspace epoch + 1; block 0 advances the epoch at its end, after it has
// seen every block's arrival word, so the next call gets a fresh tag.  Every
// wait is bounded: on expiry the kernel raises kErrTimeout and finishes.
//
// Per-row arithmetic uses the same helpers and the same orders as the staged
// kernels, so the two paths give bitwise identical results.
//
// Sources: routing to k of E experts per layer plus the shared expert
// (Swiftlet README translation, "How it works"); int4/int8 affine group
// quantization, byte-addressed kernels with 64-bit offsets, explicit hazard
// management (same page, "Relation to TurboFieldfare").
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fused_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCandMax = 64;
constexpr int kMaxDownPerWave = 8;    // down tasks per wave per round in phase D

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) == 0) return 0x80000000u;          // +0 and -0 rank equal
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
  return (static_cast<uint64_t>(tag) << 32) | __float_as_uint(v);
}

__device__ __forceinline__ void store_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, tagged(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_tagged(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave waits until flags[0..n) all equal `tag` (bounded, with backoff).
__device__ bool wait_block_flags(const uint32_t* f, int n, uint32_t tag, int lane, uint32_t& spins, uint32_t limit) {
  for (;;) {
    bool mine = true;
    for (int b = lane; b < n; b += kWave)
      mine &= __hip_atomic_load(const_cast<uint32_t*>(f) + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
    if (__all(mine)) return true;
    if (++spins > limit) return false;
    __builtin_amdgcn_s_sleep(8);
  }
}

// All stores of this block are acknowledged, then thread 0 raises the block's
// flag.  The flag is only a hint that the tagged words are there: readers
// still check every word's tag.
__device__ __forceinline__ void publish_block_flag(uint32_t* f, uint32_t tag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(f + blockIdx.x, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t lane_mask_lt(int lane) { return lane == 0 ? 0ull : (~0ull >> (64 - lane)); }

// Activation segment from LDS in its storage dtype.
template <int ACT>
__device__ __forceinline__ void lds_act_seg(const uint8_t* row, int seg, float (&v)[kSegCodes]) {
  load_act_seg<ACT>(row, seg, v);   // plain loads; `row` points into LDS
}

struct Lds {
  uint8_t* x;        // [T][H] activations, storage dtype
  float* lg;         // [T][E] logits
  int32_t* ids;      // [T][k]
  float* wts;        // [T][k]
  float* sig;        // [T]
  int64_t* slot;     // [E]
  int32_t* umap;     // [E] expert -> distinct index (or mark)
  int32_t* uniq;     // [umax]
  int32_t* pidx;     // [umax][T] rank i of the expert for token t, or -1
  float* part;       // [(T k + T)][rb]
  uint32_t* cand_k;  // [kWaves][kCandMax]
  int32_t* cand_i;   // [kWaves][kCandMax]
  int32_t* misc;     // [0] U, [1] tag, [2] timeout seen
};

__device__ inline Lds carve(uint8_t* base, const FusedArgs& a) {
  Lds s;
  size_t o = 0;
  auto take = [&](size_t n) { uint8_t* p = base + o; o += (n + 15) / 16 * 16; return p; };
  s.x = take(static_cast<size_t>(a.T) * a.H * a.act_sz);
  s.lg = reinterpret_cast<float*>(take(static_cast<size_t>(a.T) * a.E * 4));
  s.ids = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.T) * a.k * 4));
  s.wts = reinterpret_cast<float*>(take(static_cast<size_t>(a.T) * a.k * 4));
  s.sig = reinterpret_cast<float*>(take(static_cast<size_t>(a.T) * 4));
  s.slot = reinterpret_cast<int64_t*>(take(static_cast<size_t>(a.E) * 8));
  s.umap = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.E) * 4));
  s.uniq = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.umax) * 4));
  s.pidx = reinterpret_cast<int32_t*>(take(static_cast<size_t>(a.umax) * a.T * 4));
  s.part = reinterpret_cast<float*>(take(static_cast<size_t>(a.T) * (a.k + 1) * a.rb * 4));
  s.cand_k = reinterpret_cast<uint32_t*>(take(kWaves * kCandMax * 4));
  s.cand_i = reinterpret_cast<int32_t*>(take(kWaves * kCandMax * 4));
  s.misc = reinterpret_cast<int32_t*>(take(16 * 4));
  return s;
}

// One down-projection task of a wave: `rpp` rows of one expert's Wd for this
// block's output rows (lane: one segment of one row).
template <int BITS>
struct DownTask {
  Seg<BITS> code;
  float sc, bi;
  int j;        // distinct-expert index (U = shared), -1 if none
  int rloc;     // this lane's row within the block, -1 if outside
  bool valid;   // blob offset usable
};

template <int BITS, int SB>
__device__ __forceinline__ void load_down_task(DownTask<BITS>& d, int task, int ntask, int np, int U, int row_lo,
                                               const FusedArgs& a, const Lds& s, const RowLanes& rli,
                                               const RowLanes& rls, int lane, uint32_t* flags) {
  d.j = -1;
  d.rloc = -1;
  d.valid = false;
  d.sc = 0.f;
  d.bi = 0.f;
#pragma unroll
  for (int i = 0; i < BITS / 4; ++i) d.code.w[i] = u32x4{0, 0, 0, 0};
  if (task >= ntask) return;
  const int j = task / np, p = task % np;
  const bool is_sh = j == U;
  const RowLanes& rl = is_sh ? rls : rli;
  const int inter = is_sh ? a.SI : a.I;
  const Planes pl = planes_of(a.H, inter, BITS, SB);
  const uint8_t* blob = a.shared;
  bool valid = true;
  if (!is_sh) {
    const int64_t off = s.slot[s.uniq[j]];
    valid = slot_ok(off, pl.blob, a.pool_bytes);
    blob = a.pool + (valid ? off : 0);
    if (!valid && lane == 0) raise_error(flags, kErrRange);
  }
  d.j = j;
  d.valid = valid;
  const int rloc = p * rl.rpp + rl.sub_row;
  const int r = row_lo + rloc;
  if (rloc < a.rb && r < a.H) {
    d.rloc = rloc;
    if (valid) {
      const int64_t row_bytes = static_cast<int64_t>(inter) * BITS / 8;
      d.code = load_codes<BITS>(blob + 2 * pl.q + r * row_bytes + static_cast<int64_t>(rl.seg0) * (kSegCodes * BITS / 8));
      const size_t si = static_cast<size_t>(r) * (inter / 64) + rl.seg0 / 2;
      d.sc = load_scalar<SB>(blob + 3 * pl.q + 2 * pl.s, si);
      d.bi = load_scalar<SB>(blob + 3 * pl.q + 5 * pl.s, si);
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k of one token on one wave.  The k-th largest per-lane maximum is a
// lower bound of the k-th largest logit, so every top-k logit is at least it;
// the (few) candidates above the bound are ranked exactly by (logit desc, id
// asc).  If more than kCandMax candidates tie above the bound, k rounds of a
// wave arg-max finish the job.
__device__ void topk_wave(const float* lg, int E, int k, int lane, uint32_t* ck, int32_t* ci, int32_t* ids_out,
                          float* wts_out) {
  uint32_t key[16];
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int e = lane + j * kWave;
    const uint32_t kv = order_key(lg[e < E ? e : 0]);
    key[j] = e < E ? (kv > 1u ? kv : 1u) : 0u;   // every real entry ranks above "no entry"
    lm = key[j] > lm ? key[j] : lm;
  }
  uint32_t theta = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = theta | (1u << b);
    if (__popcll(__ballot(lm >= c)) >= static_cast<unsigned>(k)) theta = c;
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool in = key[j] != 0u && key[j] >= theta;
    const uint64_t m = __ballot(in);
    const int pos = cnt + __popcll(m & lane_mask_lt(lane));
    if (in && pos < kCandMax) { ck[pos] = key[j]; ci[pos] = lane + j * kWave; }
    cnt += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int my_id = -1;
  float my_v = 0.f;
  if (cnt <= kCandMax) {
    if (lane < cnt) {
      const uint32_t kc = ck[lane];
      const int ic = ci[lane];
      int rank = 0;
      for (int d = 0; d < cnt; ++d) {
        const uint32_t kd = ck[d];
        rank += (kd > kc || (kd == kc && ci[d] < ic)) ? 1 : 0;
      }
      if (rank < k) { ids_out[rank] = ic; wts_out[rank] = lg[ic]; }
    }
  } else {
    // rare: too many candidates tie above the bound
    uint64_t taken_lo = 0;
    uint32_t taken = 0;
    (void)taken_lo;
    for (int i = 0; i < k; ++i) {
      uint32_t bk = 0;
      int bid = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = lane + j * kWave;
        if (!((taken >> j) & 1u) && e < E && (key[j] > bk || (key[j] == bk && e < bid))) { bk = key[j]; bid = e; }
      }
#pragma unroll
      for (int m = kWave / 2; m > 0; m >>= 1) {
        const uint32_t ok = __shfl_xor(bk, m, kWave);
        const int oid = __shfl_xor(bid, m, kWave);
        if (ok > bk || (ok == bk && oid < bid)) { bk = ok; bid = oid; }
      }
      if ((bid & (kWave - 1)) == lane) taken |= 1u << (bid / kWave);
      if (lane == 0) { ids_out[i] = bid; wts_out[i] = lg[bid]; }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // renormalised weights, summed in rank order (same operations as the staged path)
  if (lane < k) { my_v = wts_out[lane]; my_id = ids_out[lane]; }
  const float top = wts_out[0];
  const float ex = lane < k ? expf(my_v - top) : 0.f;
  float sum = 0.f;
  for (int i = 0; i < k; ++i) sum += __shfl(ex, i, kWave);
  __builtin_amdgcn_wave_barrier();
  if (lane < k) wts_out[lane] = ex / sum;
  (void)my_id;
}

template <int BITS, int SB, int ACT, int OUT>
__global__ __launch_bounds__(kThreads) void k_decode_fused(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  const Lds s = carve(lds_raw, a);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  uint32_t* flags = a.ctrl;
  uint32_t spins = 0;
  bool timed_out = false;

  // ---- start: tag, arrival, x and slot table into LDS
  if (tid == 0) {
    const uint32_t ep = __hip_atomic_load(a.ctrl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t tag = ep + 1u;
    s.misc[1] = static_cast<int32_t>(tag);
    s.misc[2] = 0;
  }
  {
    const int n16 = T * H * a.act_sz / 16;
    const u32x4* src = static_cast<const u32x4*>(a.x);
    u32x4* dst = reinterpret_cast<u32x4*>(s.x);
    for (int i = tid; i < n16; i += kThreads) dst[i] = src[i];
    for (int e = tid; e < E; e += kThreads) s.slot[e] = a.slot_table[e];
  }
  __syncthreads();
  const uint32_t tag = static_cast<uint32_t>(s.misc[1]);
  const size_t xrow = static_cast<size_t>(H) * a.act_sz;

  // ---- phase R: router rows, shared gate/up rows (wave-major task order)
  const int gwave = wave * a.nb + blockIdx.x;          // spreads tasks over blocks first
  const int nwaves = a.nb * kWaves;
  const RowLanes rlh = row_lanes(H, lane);
  const int router_tasks = (E + rlh.rpp - 1) / rlh.rpp;
  const int npass_h = rlh.rpp >= kMaxPass ? 1 : kMaxPass / rlh.rpp;
  const int sh_rows_per_task = npass_h * rlh.rpp;
  const int sh_tasks = (a.SI + sh_rows_per_task - 1) / sh_rows_per_task;
  for (int task = gwave; task < router_tasks + sh_tasks; task += nwaves) {
    if (task < router_tasks) {
      const int e = task * rlh.rpp + rlh.sub_row;
      const bool active = e < E;
      float r[kSegCodes];
      if (active) load_act_seg<ACT>(static_cast<const uint8_t*>(a.router) + static_cast<size_t>(e) * xrow, rlh.seg0, r);
      for (int t = 0; t < T; ++t) {
        float acc = 0.f;
        if (active) {
          float v[kSegCodes];
          lds_act_seg<ACT>(s.x + t * xrow, rlh.seg0, v);
#pragma unroll
          for (int c = 0; c < kSegCodes; ++c) acc = fmaf(v[c], r[c], acc);
        }
        acc = group_sum(acc, rlh.width);
        if (active && (lane % rlh.width) == 0) store_tagged(a.lg + static_cast<size_t>(t) * E + e, acc, tag);
      }
    } else {
      // shared expert gate/up rows for every token
      const int row0 = (task - router_tasks) * sh_rows_per_task;
      const Planes pl = planes_of(H, a.SI, BITS, SB);
      const int64_t row_bytes = static_cast<int64_t>(H) * BITS / 8;
      const int seg_bytes = kSegCodes * BITS / 8;
      const int gpr = H / 64;
      for (int p = 0; p < npass_h; ++p) {
        const int rr = row0 + p * rlh.rpp + rlh.sub_row;
        const bool ok = rr < a.SI;
        Seg<BITS> cg, cu;
        float sg = 0.f, su = 0.f, bg = 0.f, bu = 0.f;
        if (ok) {
          const int64_t qo = rr * row_bytes + static_cast<int64_t>(rlh.seg0) * seg_bytes;
          cg = load_codes<BITS>(a.shared + qo);
          cu = load_codes<BITS>(a.shared + pl.q + qo);
          const size_t si = static_cast<size_t>(rr) * gpr + rlh.seg0 / 2;
          sg = load_scalar<SB>(a.shared + 3 * pl.q, si);
          su = load_scalar<SB>(a.shared + 3 * pl.q + pl.s, si);
          bg = load_scalar<SB>(a.shared + 3 * pl.q + 3 * pl.s, si);
          bu = load_scalar<SB>(a.shared + 3 * pl.q + 4 * pl.s, si);
        } else {
#pragma unroll
          for (int i = 0; i < BITS / 4; ++i) { cg.w[i] = u32x4{0, 0, 0, 0}; cu.w[i] = u32x4{0, 0, 0, 0}; }
        }
        for (int t = 0; t < T; ++t) {
          float v[1][kSegCodes];
          lds_act_seg<ACT>(s.x + t * xrow, rlh.seg0, v[0]);
          const float xs = seg_sum(v[0]);
          float qg[1], qu[1];
          seg_qdot_nt<BITS, 1>(cg, v, qg);
          seg_qdot_nt<BITS, 1>(cu, v, qu);
          float accg = 0.f, accu = 0.f;
          accg += seg_value(sg, bg, qg[0], xs);
          accu += seg_value(su, bu, qu[0], xs);
          const float g = group_sum(accg, rlh.width);
          const float u = group_sum(accu, rlh.width);
          if (ok && (lane % rlh.width) == 0)
            store_tagged(a.hx + (static_cast<size_t>(T) * k + t) * a.hs + rr, silu(g) * u, tag);
        }
      }
    }
  }
  // sigmoid(g . x_t), same lane order as the staged path (lane covers segments L, L+64, ...)
  if (wave == kWaves - 1) {
    const uint8_t* gvec = a.shared + a.shared_stride;
    const int nseg = H / kSegCodes;
    for (int t = 0; t < T; ++t) {
      float acc = 0.f;
      if (lane < nseg) {
        float xv[kSegCodes], gv[kSegCodes];
        lds_act_seg<ACT>(s.x + t * xrow, lane, xv);
        load_act_seg<ACT>(gvec, lane, gv);
#pragma unroll
        for (int c = 0; c < kSegCodes; ++c) acc = fmaf(xv[c], gv[c], acc);
      }
      acc = group_sum(acc, kWave);
      if (lane == 0) s.sig[t] = sigmoid(acc);
    }
  }

  // ---- phase K: gather all logits (tag-checked), top-k, dispatch
  publish_block_flag(a.flag_r, tag);
  if (wave == 0 && !wait_block_flags(a.flag_r, a.nb, tag, lane, spins, a.spin_limit)) timed_out = true;
  __syncthreads();
  for (;;) {
    int missing = 0;
    for (int i = tid; i < T * E; i += kThreads) {
      const uint64_t w = load_tagged(a.lg + i);
      if (static_cast<uint32_t>(w >> 32) != tag) missing = 1;
      else s.lg[i] = __uint_as_float(static_cast<uint32_t>(w));
    }
    if (!__syncthreads_or(missing)) break;
    if (++spins > a.spin_limit) { timed_out = true; break; }
    __builtin_amdgcn_s_sleep(8);
  }
  for (int t = wave; t < T; t += kWaves)
    topk_wave(s.lg + static_cast<size_t>(t) * E, E, k, lane, s.cand_k + wave * kCandMax, s.cand_i + wave * kCandMax,
              s.ids + t * k, s.wts + t * k);
  for (int e = tid; e < E; e += kThreads) s.umap[e] = -1;
  __syncthreads();
  for (int p = tid; p < T * k; p += kThreads) {
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
  const int U = s.misc[0];
  for (int i = tid; i < U * T; i += kThreads) s.pidx[i] = -1;
  __syncthreads();
  for (int p = tid; p < T * k; p += kThreads) {
    const int t = p / k, i = p % k;
    s.pidx[s.umap[s.ids[p]] * T + t] = i;
  }
  if (blockIdx.x == 0) {
    for (int p = tid; p < T * k; p += kThreads) {
      if (a.ids_out) a.ids_out[p] = s.ids[p];
      if (a.wts_out) a.wts_out[p] = s.wts[p];
    }
  }
  __syncthreads();

  // ---- phase D prefetch: this block's output rows.  Down tasks are (expert j, pass p)
  // for j < U (routed, distinct) and j == U (shared), passes of rpp rows each;
  // wave w takes tasks w, w + 4, ... in rounds of kMaxDownPerWave.
  const RowLanes rli = row_lanes(a.I, lane);
  const RowLanes rls = row_lanes(a.SI, lane);
  const int row_lo = blockIdx.x * a.rb;
  const int nd = U + 1;
  const int rpp_min = rli.rpp < rls.rpp ? rli.rpp : rls.rpp;
  const int np = (a.rb + rpp_min - 1) / rpp_min;
  const int ntask = nd * np;
  DownTask<BITS> dt[kMaxDownPerWave];
#pragma unroll
  for (int q = 0; q < kMaxDownPerWave; ++q)
    load_down_task<BITS, SB>(dt[q], wave + q * kWaves, ntask, np, U, row_lo, a, s, rli, rls, lane, flags);

  // ---- phase G: routed gate/up rows, flattened over (expert, row group)
  {
    const Planes pl = planes_of(H, a.I, BITS, SB);
    const int64_t row_bytes = static_cast<int64_t>(H) * BITS / 8;
    const int seg_bytes = kSegCodes * BITS / 8;
    const int gpr = H / 64;
    const int groups_per_expert = a.I / rlh.rpp;
    const int total = U * groups_per_expert;
    const int per_wave = (total + nwaves - 1) / nwaves;
    const int g_lo = gwave * per_wave;
    const int g_hi = min(total, g_lo + per_wave);
    constexpr int kBatch = 4;
    for (int g0 = g_lo; g0 < g_hi; g0 += kBatch) {
      Seg<BITS> cg[kBatch], cu[kBatch];
      float sg[kBatch], su[kBatch], bg[kBatch], bu[kBatch];
      int uu[kBatch], rr[kBatch];
      bool vv[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int g = g0 + b;
        uu[b] = -1;
        vv[b] = false;
        if (g < g_hi) {
          const int u = g / groups_per_expert;
          const int r = (g % groups_per_expert) * rlh.rpp + rlh.sub_row;
          const int64_t off = s.slot[s.uniq[u]];
          const bool valid = slot_ok(off, pl.blob, a.pool_bytes);
          uu[b] = u;
          rr[b] = r;
          vv[b] = valid;
          if (valid) {
            const uint8_t* blob = a.pool + off;
            const int64_t qo = r * row_bytes + static_cast<int64_t>(rlh.seg0) * seg_bytes;
            cg[b] = load_codes<BITS>(blob + qo);
            cu[b] = load_codes<BITS>(blob + pl.q + qo);
            const size_t si = static_cast<size_t>(r) * gpr + rlh.seg0 / 2;
            sg[b] = load_scalar<SB>(blob + 3 * pl.q, si);
            su[b] = load_scalar<SB>(blob + 3 * pl.q + pl.s, si);
            bg[b] = load_scalar<SB>(blob + 3 * pl.q + 3 * pl.s, si);
            bu[b] = load_scalar<SB>(blob + 3 * pl.q + 4 * pl.s, si);
          } else if (lane == 0) {
            raise_error(flags, kErrRange);
          }
        }
        if (!vv[b]) {
#pragma unroll
          for (int i = 0; i < BITS / 4; ++i) { cg[b].w[i] = u32x4{0, 0, 0, 0}; cu[b].w[i] = u32x4{0, 0, 0, 0}; }
          sg[b] = su[b] = bg[b] = bu[b] = 0.f;
        }
      }
      for (int t = 0; t < T; ++t) {
        float v[1][kSegCodes];
        lds_act_seg<ACT>(s.x + t * xrow, rlh.seg0, v[0]);
        const float xs = seg_sum(v[0]);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
          if (uu[b] < 0) continue;
          const int i = s.pidx[uu[b] * T + t];
          if (i < 0) continue;                      // token t does not use this expert
          float qg[1], qu[1];
          seg_qdot_nt<BITS, 1>(cg[b], v, qg);
          seg_qdot_nt<BITS, 1>(cu[b], v, qu);
          float accg = 0.f, accu = 0.f;
          accg += seg_value(sg[b], bg[b], qg[0], xs);
          accu += seg_value(su[b], bu[b], qu[0], xs);
          const float g = group_sum(accg, rlh.width);
          const float u = group_sum(accu, rlh.width);
          if ((lane % rlh.width) == 0)
            store_tagged(a.hx + (static_cast<size_t>(t) * k + i) * a.hs + rr[b], vv[b] ? silu(g) * u : 0.f, tag);
        }
      }
    }
  }

  // ---- phase D: down rows of this block for every (token, expert) pair
  publish_block_flag(a.flag_g, tag);
  if (wave == 0 && !wait_block_flags(a.flag_g, a.nb, tag, lane, spins, a.spin_limit)) timed_out = true;
  __syncthreads();
  for (int base = 0; base < ntask; base += kWaves * kMaxDownPerWave) {
    if (base > 0) {
#pragma unroll
      for (int q = 0; q < kMaxDownPerWave; ++q)
        load_down_task<BITS, SB>(dt[q], base + wave + q * kWaves, ntask, np, U, row_lo, a, s, rli, rls, lane, flags);
    }
#pragma unroll
    for (int q = 0; q < kMaxDownPerWave; ++q) {
      if (dt[q].j < 0) continue;
      const bool is_sh = dt[q].j == U;
      const RowLanes& rl = is_sh ? rls : rli;
      for (int t = 0; t < T; ++t) {
        const int i = is_sh ? k : s.pidx[dt[q].j * T + t];
        if (i < 0) continue;
        const size_t pair = is_sh ? static_cast<size_t>(T) * k + t : static_cast<size_t>(t) * k + i;
        const uint64_t* hp = a.hx + pair * a.hs + rl.seg0 * kSegCodes;
        float hv[1][kSegCodes];
        for (;;) {
          bool ready = true;
#pragma unroll
          for (int c = 0; c < kSegCodes; ++c) {
            const uint64_t w = load_tagged(hp + c);
            ready &= static_cast<uint32_t>(w >> 32) == tag;
            hv[0][c] = __uint_as_float(static_cast<uint32_t>(w));
          }
          if (__all(ready)) break;
          if (++spins > a.spin_limit) { timed_out = true; break; }
          __builtin_amdgcn_s_sleep(8);
        }
        const float hs = seg_sum(hv[0]);
        float qv[1];
        seg_qdot_nt<BITS, 1>(dt[q].code, hv, qv);
        float acc = 0.f;
        acc += seg_value(dt[q].sc, dt[q].bi, qv[0], hs);
        const float v = group_sum(acc, rl.width);
        if ((lane % rl.width) == 0 && dt[q].rloc >= 0) s.part[pair * a.rb + dt[q].rloc] = dt[q].valid ? v : 0.f;
      }
    }
  }
  if (timed_out) s.misc[2] = 1;
  __syncthreads();
  // ordered combine for this block's rows
  for (int idx = tid; idx < T * a.rb; idx += kThreads) {
    const int t = idx / a.rb, rloc = idx % a.rb;
    const int n = row_lo + rloc;
    if (n >= H) continue;
    float acc = 0.f;
    for (int i = 0; i < k; ++i) acc = fmaf(s.wts[t * k + i], s.part[(static_cast<size_t>(t) * k + i) * a.rb + rloc], acc);
    acc = fmaf(s.sig[t], s.part[(static_cast<size_t>(T) * k + t) * a.rb + rloc], acc);
    if constexpr (OUT == kF32) {
      static_cast<float*>(a.out)[static_cast<size_t>(t) * H + n] = acc;
    } else {
      static_cast<uint16_t*>(a.out)[static_cast<size_t>(t) * H + n] = f32_to_bf16(acc);
    }
  }
  if (tid == 0 && s.misc[2]) raise_error(flags, kErrTimeout);
  // Every block read the epoch before raising its phase-R flag, and block 0
  // saw all those flags in phase K, so it can retire the tag now.
  if (blockIdx.x == 0 && tid == 0) __hip_atomic_store(a.ctrl + 1, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t fused_lds_bytes(int T, int H, int E, int k, int umax, int rb, int act_sz) {
  size_t o = 0;
  auto take = [&](size_t n) { o += (n + 15) / 16 * 16; };
  take(static_cast<size_t>(T) * H * act_sz);
  take(static_cast<size_t>(T) * E * 4);
  take(static_cast<size_t>(T) * k * 4);
  take(static_cast<size_t>(T) * k * 4);
  take(static_cast<size_t>(T) * 4);
  take(static_cast<size_t>(E) * 8);
  take(static_cast<size_t>(E) * 4);
  take(static_cast<size_t>(umax) * 4);
  take(static_cast<size_t>(umax) * T * 4);
  take(static_cast<size_t>(T) * (k + 1) * rb * 4);
  take(kWaves * kCandMax * 4);
  take(kWaves * kCandMax * 4);
  take(16 * 4);
  return o;
}

template <int BITS, int SB, int ACT, int OUT>
static int launch_variant(const FusedArgs& a, size_t lds, hipStream_t stream) {
  auto kern = k_decode_fused<BITS, SB, ACT, OUT>;
  hipLaunchKernelGGL(kern, dim3(a.nb), dim3(kThreads), lds, stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

template <int BITS, int SB, int ACT, int OUT>
static int occupancy_variant(size_t lds, int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, k_decode_fused<BITS, SB, ACT, OUT>, kThreads, lds) ==
                 hipSuccess
             ? MOE_OK
             : MOE_EHIP;
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

static int fused_occupancy(const moe_desc& d, size_t lds, int* blocks) { FUSED_DISPATCH(occupancy_variant, lds, blocks); }

static int fused_launch(const moe_desc& d, const FusedArgs& a, size_t lds, hipStream_t s) {
  FUSED_DISPATCH(launch_variant, a, lds, s);
}

bool fused_supported(const moe_desc& d, int T) {
  if (T < 1 || T > kFusedMaxT) return false;
  const int b = d.bits, s = d.sb_dtype, a = d.act_dtype;
  const bool combo = (s == kBF16 && a == kBF16) || (s == kF32 && a == kF32 && d.out_dtype == kF32);
  (void)b;
  return combo;
}

int fused_plan(const moe_desc& d, int T, FusedPlan* plan) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEV;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ENODEV;
  const int act_sz = d.act_dtype == kF32 ? 4 : 2;
  const int umax = T * d.top_k < d.n_experts ? T * d.top_k : d.n_experts;
  // blocks: two per CU when they fit, else one; each block owns rb output rows
  for (int per_cu = 2; per_cu >= 1; --per_cu) {
    const int nb = cus * per_cu;
    if (nb > kFusedMaxBlocks) continue;
    const int rb = (d.hidden + nb - 1) / nb;
    const size_t lds = fused_lds_bytes(T, d.hidden, d.n_experts, d.top_k, umax, rb, act_sz);
    int fit = 0;
    if (lds > 160 * 1024) continue;
    if (fused_occupancy(d, lds, &fit) != MOE_OK) return MOE_EHIP;
    if (fit >= per_cu) {
      plan->nb = nb;
      plan->rb = rb;
      plan->lds = lds;
      plan->umax = umax;
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
  a.ids_out = c.ids_out;
  a.wts_out = c.wts_out;
  a.lg = reinterpret_cast<uint64_t*>(c.ws + c.L.f_lg);
  a.hx = reinterpret_cast<uint64_t*>(c.ws + c.L.f_hx);
  a.ctrl = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  a.flag_r = reinterpret_cast<uint32_t*>(c.ws + c.L.f_arrive);
  a.flag_g = a.flag_r + kFusedMaxBlocks;
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
  a.rb = plan.rb;
  a.umax = plan.umax;
  a.act_sz = d.act_dtype == kF32 ? 4 : 2;
  a.spin_limit = 1u << 20;
  return fused_launch(d, a, plan.lds, c.stream);
}

}  // namespace moe
