// Decode-path kernels of the MoE layer (gfx950, wave64).
//
// One call runs, on the caller's stream:
//   router_logits -> topk -> dispatch -> gateup -> down -> combine
// Routing follows the Swiftlet README translation ("How it works": each token
// goes to k of E experts per layer, plus the always-on shared expert); the
// expert weights are read from fixed-stride blobs through 64-bit slot offsets
// ("Relation to TurboFieldfare": byte-addressed kernels, 64-bit offsets).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"
#include "topk_wave.h"

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// Router logits: l[t, e] = sum_h x[t, h] R[e, h] in float32 (FMA chain over
// the lane's codes in order, then the lane butterfly).  Rows 0..E-1.
template <int ACT, int NSL>
__global__ __launch_bounds__(256) void k_router_logits(const void* __restrict__ x, const void* __restrict__ router,
                                                      float* __restrict__ logits, int T, int H, int E) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const RowLanes rl = row_lanes(H, lane);
  const int e = wave * rl.rpp + rl.sub_row;
  const bool active = e < E;
  const size_t act_sz = ACT == kF32 ? 4 : 2;
  float r[NSL][kSegCodes];
  if (active) {
    const uint8_t* row = static_cast<const uint8_t*>(router) + static_cast<size_t>(e) * H * act_sz;
#pragma unroll
    for (int n = 0; n < NSL; ++n) load_act_seg<ACT>(row, rl.seg0 + n * kWave, r[n]);
  }
  for (int t = 0; t < T; ++t) {
    float acc = 0.f;
    if (active) {
      const uint8_t* xr = static_cast<const uint8_t*>(x) + static_cast<size_t>(t) * H * act_sz;
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
        float v[kSegCodes];
        load_act_seg<ACT>(xr, rl.seg0 + n * kWave, v);
#pragma unroll
        for (int c = 0; c < kSegCodes; ++c) acc = fmaf(v[c], r[n][c], acc);
      }
    }
    acc = group_sum(acc, rl.width);
    if (active && (lane % rl.width) == 0) logits[static_cast<size_t>(t) * E + e] = acc;
  }
}

// ---------------------------------------------------------------------------
// Top-k per token, one wave per token (topk_wave: a threshold from the lane
// maxima, then the candidates above it ranked exactly by (logit descending,
// id ascending)), then p_i = exp(l_i - l_0) / sum_j exp(l_j - l_0) with the
// sum taken in rank order.  The token's logits row is copied to LDS first,
// all loads of a lane issued together.
constexpr int kTopkWaves = 4;
constexpr int kTopkMaxE = 1024;

__global__ __launch_bounds__(kTopkWaves * kWave) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                                           int32_t* __restrict__ ids, float* __restrict__ wts,
                                                           int32_t* __restrict__ ids2, float* __restrict__ wts2) {
  __shared__ float s_lg[kTopkWaves][kTopkMaxE];
  __shared__ uint64_t s_cand[kTopkWaves][kCandMax];
  __shared__ int32_t s_ids[kTopkWaves][kWave];
  __shared__ float s_vals[kTopkWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int t = blockIdx.x * kTopkWaves + wv;
  if (t >= T) return;   // the waves of a block never synchronise with each other
  const float* row = logits + static_cast<size_t>(t) * E;
  float v[kTopkMaxE / kWave];
#pragma unroll
  for (int j = 0; j < kTopkMaxE / kWave; ++j) {
    const int e = lane + j * kWave;
    v[j] = row[e < E ? e : 0];
  }
#pragma unroll
  for (int j = 0; j < kTopkMaxE / kWave; ++j) {
    const int e = lane + j * kWave;
    if (e < E) s_lg[wv][e] = v[j];
  }
  wave_sync_lds();
  topk_wave(s_lg[wv], E, k, lane, s_cand[wv], s_ids[wv], s_vals[wv]);
  wave_sync_lds();
  if (lane < k) {
    const size_t o = static_cast<size_t>(t) * k + lane;
    const int id = s_ids[wv][lane];
    const float p = s_vals[wv][lane];
    ids[o] = id;
    wts[o] = p;
    if (ids2) ids2[o] = id;
    if (wts2) wts2[o] = p;
  }
}

// ---------------------------------------------------------------------------
// Dispatch (one block of 1024 threads): group the T*k (token, rank) pairs by
// expert.  Distinct experts are listed in ascending id; within an expert the
// pair order is unspecified (every pair writes its own output rows, so the
// order does not change any value).  Also forms sigmoid(g . x_t) per token.
constexpr int kDispatchThreads = 1024;

template <int ACT, int NSL>
__global__ __launch_bounds__(kDispatchThreads) void k_dispatch(const int32_t* __restrict__ ids, int T, int k, int E,
                                                               int H, const void* __restrict__ x,
                                                               const void* __restrict__ gvec, float* __restrict__ gate,
                                                               int32_t* __restrict__ ucount, int32_t* __restrict__ uniq,
                                                               int32_t* __restrict__ ustart, int32_t* __restrict__ plist,
                                                               uint32_t* __restrict__ flags) {
  __shared__ int hist[kDispatchThreads];
  __shared__ int cursor[kDispatchThreads];
  __shared__ int wsum_c[kDispatchThreads / kWave];
  __shared__ int wsum_u[kDispatchThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int npairs = T * k;
  hist[tid] = 0;
  __syncthreads();
  for (int p = tid; p < npairs; p += kDispatchThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    else raise_error(flags, kErrRange);
  }
  __syncthreads();
  // exclusive scans of counts and of "expert used"
  const int c = hist[tid];
  const int u = c > 0 ? 1 : 0;
  int ic = c, iu = u;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int oc = __shfl_up(ic, m, kWave);
    const int ou = __shfl_up(iu, m, kWave);
    if (lane >= m) { ic += oc; iu += ou; }
  }
  if (lane == kWave - 1) { wsum_c[wid] = ic; wsum_u[wid] = iu; }
  __syncthreads();
  if (wid == 0) {
    int vc = lane < kDispatchThreads / kWave ? wsum_c[lane] : 0;
    int vu = lane < kDispatchThreads / kWave ? wsum_u[lane] : 0;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int oc = __shfl_up(vc, m, kWave);
      const int ou = __shfl_up(vu, m, kWave);
      if (lane >= m) { vc += oc; vu += ou; }
    }
    if (lane < kDispatchThreads / kWave) { wsum_c[lane] = vc; wsum_u[lane] = vu; }
  }
  __syncthreads();
  const int base_c = wid > 0 ? wsum_c[wid - 1] : 0;
  const int base_u = wid > 0 ? wsum_u[wid - 1] : 0;
  const int start = base_c + ic - c;
  const int rank = base_u + iu - u;
  if (u) {
    uniq[rank] = tid;
    ustart[rank] = start;
  }
  cursor[tid] = start;
  if (tid == kDispatchThreads - 1) {
    const int U = base_u + iu;
    *ucount = U;
    ustart[U] = base_c + ic;
  }
  __syncthreads();
  for (int p = tid; p < npairs; p += kDispatchThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&cursor[e], 1);
      plist[pos] = p;
    }
  }
  // gate: sigmoid(g . x_t), lane L covers segments L, L + 64, ...
  const size_t act_sz = ACT == kF32 ? 4 : 2;
  const int nseg = H / kSegCodes;
  for (int t = wid; t < T; t += kDispatchThreads / kWave) {
    float acc = 0.f;
    const uint8_t* xr = static_cast<const uint8_t*>(x) + static_cast<size_t>(t) * H * act_sz;
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
      const int sg = lane + n * kWave;
      if (sg < nseg) {
        float a[kSegCodes], g[kSegCodes];
        load_act_seg<ACT>(xr, sg, a);
        load_act_seg<ACT>(gvec, sg, g);
#pragma unroll
        for (int cc = 0; cc < kSegCodes; ++cc) acc = fmaf(a[cc], g[cc], acc);
      }
    }
    acc = group_sum(acc, kWave);
    if (lane == 0) gate[t] = sigmoid(acc);
  }
}

// ---------------------------------------------------------------------------
// Gate/up GEMV + SwiGLU.  Block = 4 waves; a wave owns `npass` passes of
// row_lanes rows of one expert and processes every token routed to it in
// chunks of TOKC, writing h[pair, r] = silu(Wg x)_r * (Wu x)_r.
// Blocks [0, umax * bpe_r) take routed experts (expert slot u = block / bpe_r,
// idle if u >= U); the rest take the shared expert for all T tokens.
struct GateUpArgs {
  const void* x;
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  const int32_t* ucount;
  const int32_t* uniq;
  const int32_t* ustart;
  const int32_t* plist;
  float* h;
  uint32_t* flags;
  int64_t pool_bytes;
  int T, k, H, I, SI, umax, bpe_r, bpe_s, hstride;
};

template <int BITS, int SB, int ACT, int NSL, int TOKC>
__global__ __launch_bounds__(256) void k_gateup(GateUpArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const bool shared = blockIdx.x >= a.umax * a.bpe_r;
  int rb, u = 0, e = -1;
  if (!shared) {
    u = blockIdx.x / a.bpe_r;
    rb = blockIdx.x % a.bpe_r;
    if (u >= *a.ucount) return;
    e = a.uniq[u];
  } else {
    rb = blockIdx.x - a.umax * a.bpe_r;
  }
  const int rows = shared ? a.SI : a.I;
  const Planes pl = planes_of(a.H, rows, BITS, SB);
  const uint8_t* blob;
  bool valid = true;
  if (shared) {
    blob = a.shared;
  } else {
    const int64_t off = a.slot_table[e];
    valid = slot_ok(off, pl.blob, a.pool_bytes);
    blob = a.pool + (valid ? off : 0);
    if (!valid && threadIdx.x == 0) raise_error(a.flags, kErrRange);
  }
  const RowLanes rl = row_lanes(a.H, lane);
  const int npass = rl.rpp >= kMaxPass ? 1 : kMaxPass / rl.rpp;
  const int rows_per_wave = npass * rl.rpp;
  const int row0 = (rb * 4 + wave) * rows_per_wave;
  const int64_t row_bytes = static_cast<int64_t>(a.H) * BITS / 8;
  const int seg_bytes = kSegCodes * BITS / 8;
  const int gpr = a.H / 64;   // groups per row

  Seg<BITS> cg[kMaxPass][NSL], cu[kMaxPass][NSL];
  float sg[kMaxPass][NSL], bg[kMaxPass][NSL], su[kMaxPass][NSL], bu[kMaxPass][NSL];
#pragma unroll
  for (int p = 0; p < kMaxPass; ++p) {
    const int r = row0 + p * rl.rpp + rl.sub_row;
    if (p < npass && r < rows && valid) {
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
        const int seg = rl.seg0 + n * kWave;
        const int64_t qo = r * row_bytes + static_cast<int64_t>(seg) * seg_bytes;
        cg[p][n] = load_codes<BITS>(blob + qo);
        cu[p][n] = load_codes<BITS>(blob + pl.q + qo);
        const size_t si = static_cast<size_t>(r) * gpr + seg / 2;
        sg[p][n] = load_scalar<SB>(blob + 3 * pl.q, si);
        su[p][n] = load_scalar<SB>(blob + 3 * pl.q + pl.s, si);
        bg[p][n] = load_scalar<SB>(blob + 3 * pl.q + 3 * pl.s, si);
        bu[p][n] = load_scalar<SB>(blob + 3 * pl.q + 4 * pl.s, si);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) { cg[p][n].w[i] = u32x4{0, 0, 0, 0}; cu[p][n].w[i] = u32x4{0, 0, 0, 0}; }
        sg[p][n] = su[p][n] = bg[p][n] = bu[p][n] = 0.f;
      }
    }
  }
  // token list
  int n_tok, first = 0;
  if (shared) {
    n_tok = a.T;
  } else {
    first = a.ustart[u];
    n_tok = a.ustart[u + 1] - first;
  }
  const size_t act_sz = ACT == kF32 ? 4 : 2;
  if constexpr (ACT == kBF16 && BITS == 4) {
    // v_dot2 segment dots (same arithmetic as the two-launch decode kernel)
    for (int c = 0; c < n_tok; ++c) {
      int tok, hrow;
      if (shared) {
        tok = c;
        hrow = a.T * a.k + c;
      } else {
        const int pair = a.plist[first + c];
        tok = pair / a.k;
        hrow = pair;
      }
      float accg[kMaxPass], accu[kMaxPass];
#pragma unroll
      for (int p = 0; p < kMaxPass; ++p) { accg[p] = 0.f; accu[p] = 0.f; }
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
        const int seg = rl.seg0 + n * kWave;
        ActRaw<kBF16> xr;
        load_act_raw<kBF16>(static_cast<const uint8_t*>(a.x) + static_cast<size_t>(tok) * a.H * act_sz, seg, xr);
        const float xs = xsum_bf16(xr);
#pragma unroll
        for (int p = 0; p < kMaxPass; ++p) {
          if (p < npass) {
            accg[p] += seg_value_d2(sg[p][n], bg[p][n], dot2_seg(qpairs_bf16(cg[p][n]), xr), xs);
            accu[p] += seg_value_d2(su[p][n], bu[p][n], dot2_seg(qpairs_bf16(cu[p][n]), xr), xs);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < kMaxPass; ++p) {
        if (p < npass) {
          const int r = row0 + p * rl.rpp + rl.sub_row;
          float g, v;
          gu_sums(accg[p], accu[p], rl.width, g, v);
          if (r < rows && (lane % rl.width) == 0)
            a.h[static_cast<size_t>(hrow) * a.hstride + r] = valid ? silu(g) * v : 0.f;
        }
      }
    }
    return;
  }
  for (int c0 = 0; c0 < n_tok; c0 += TOKC) {
    float xv[TOKC][kSegCodes];
    float xs[TOKC][NSL];
    int hrow[TOKC];
    float accg[kMaxPass][TOKC], accu[kMaxPass][TOKC];
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p)
#pragma unroll
      for (int t = 0; t < TOKC; ++t) { accg[p][t] = 0.f; accu[p][t] = 0.f; }
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
      const int seg = rl.seg0 + n * kWave;
#pragma unroll
      for (int t = 0; t < TOKC; ++t) {
        const int ci = c0 + t < n_tok ? c0 + t : n_tok - 1;
        int tok;
        if (shared) {
          tok = ci;
          hrow[t] = a.T * a.k + ci;
        } else {
          const int pair = a.plist[first + ci];
          tok = pair / a.k;
          hrow[t] = pair;
        }
        load_act_seg<ACT>(static_cast<const uint8_t*>(a.x) + static_cast<size_t>(tok) * a.H * act_sz, seg, xv[t]);
        xs[t][n] = seg_sum(xv[t]);
      }
#pragma unroll
      for (int p = 0; p < kMaxPass; ++p) {
        if (p < npass) {
          float qg[TOKC], qu[TOKC];
          seg_qdot_nt<BITS, TOKC>(cg[p][n], xv, qg);
          seg_qdot_nt<BITS, TOKC>(cu[p][n], xv, qu);
#pragma unroll
          for (int t = 0; t < TOKC; ++t) {
            accg[p][t] += seg_value(sg[p][n], bg[p][n], qg[t], xs[t][n]);
            accu[p][t] += seg_value(su[p][n], bu[p][n], qu[t], xs[t][n]);
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
      if (p < npass) {
        const int r = row0 + p * rl.rpp + rl.sub_row;
#pragma unroll
        for (int t = 0; t < TOKC; ++t) {
          float g, v;
          gu_sums(accg[p][t], accu[p][t], rl.width, g, v);
          if (c0 + t < n_tok && r < rows && (lane % rl.width) == 0) {
            a.h[static_cast<size_t>(hrow[t]) * a.hstride + r] = valid ? silu(g) * v : 0.f;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection per (expert, row block): partial[pair, n] = Wd[n, :] . h[pair, :].
// Same lane layout over rows of `inter` codes.
struct DownArgs {
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  const int32_t* ucount;
  const int32_t* uniq;
  const int32_t* ustart;
  const int32_t* plist;
  const float* h;
  float* partial;
  uint32_t* flags;
  int64_t pool_bytes;
  int T, k, H, I, SI, umax, bpe, hstride;
};

template <int BITS, int SB, int NSL>
__global__ __launch_bounds__(256) void k_down(DownArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const bool shared = blockIdx.x >= a.umax * a.bpe;
  int rb, u = 0, e = -1;
  if (!shared) {
    u = blockIdx.x / a.bpe;
    rb = blockIdx.x % a.bpe;
    if (u >= *a.ucount) return;
    e = a.uniq[u];
  } else {
    rb = blockIdx.x - a.umax * a.bpe;
  }
  const int inter = shared ? a.SI : a.I;
  const Planes pl = planes_of(a.H, inter, BITS, SB);
  const uint8_t* blob;
  bool valid = true;
  if (shared) {
    blob = a.shared;
  } else {
    const int64_t off = a.slot_table[e];
    valid = slot_ok(off, pl.blob, a.pool_bytes);
    blob = a.pool + (valid ? off : 0);
  }
  const RowLanes rl = row_lanes(inter, lane);
  const int npass = rl.rpp >= kMaxPass ? 1 : kMaxPass / rl.rpp;
  const int rows_per_wave = npass * rl.rpp;
  const int row0 = (rb * 4 + wave) * rows_per_wave;
  const int64_t row_bytes = static_cast<int64_t>(inter) * BITS / 8;
  const int seg_bytes = kSegCodes * BITS / 8;
  const int gpr = inter / 64;
  const uint8_t* dq = blob + 2 * pl.q;
  const uint8_t* ds = blob + 3 * pl.q + 2 * pl.s;
  const uint8_t* db = blob + 3 * pl.q + 5 * pl.s;

  Seg<BITS> cd[kMaxPass][NSL];
  float sd[kMaxPass][NSL], bd[kMaxPass][NSL];
#pragma unroll
  for (int p = 0; p < kMaxPass; ++p) {
    const int r = row0 + p * rl.rpp + rl.sub_row;
    if (p < npass && r < a.H && valid) {
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
        const int seg = rl.seg0 + n * kWave;
        cd[p][n] = load_codes<BITS>(dq + r * row_bytes + static_cast<int64_t>(seg) * seg_bytes);
        const size_t si = static_cast<size_t>(r) * gpr + seg / 2;
        sd[p][n] = load_scalar<SB>(ds, si);
        bd[p][n] = load_scalar<SB>(db, si);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NSL; ++n) {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) cd[p][n].w[i] = u32x4{0, 0, 0, 0};
        sd[p][n] = bd[p][n] = 0.f;
      }
    }
  }
  int n_pair, first = 0;
  if (shared) {
    n_pair = a.T;
  } else {
    first = a.ustart[u];
    n_pair = a.ustart[u + 1] - first;
  }
  for (int ci = 0; ci < n_pair; ++ci) {
    const int hrow = shared ? a.T * a.k + ci : a.plist[first + ci];
    const float* hr = a.h + static_cast<size_t>(hrow) * a.hstride;
    float acc[kMaxPass];
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) acc[p] = 0.f;
#pragma unroll
    for (int n = 0; n < NSL; ++n) {
      float hv[1][kSegCodes];
      load_f32_seg(hr, rl.seg0 + n * kWave, hv[0]);
      const float hs = seg_sum(hv[0]);
#pragma unroll
      for (int p = 0; p < kMaxPass; ++p) {
        if (p < npass) {
          float q[1];
          seg_qdot_nt<BITS, 1>(cd[p][n], hv, q);
          acc[p] += seg_value(sd[p][n], bd[p][n], q[0], hs);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kMaxPass; ++p) {
      if (p < npass) {
        const int r = row0 + p * rl.rpp + rl.sub_row;
        const float v = group_sum(acc[p], rl.width);
        if (r < a.H && (lane % rl.width) == 0) {
          a.partial[static_cast<size_t>(hrow) * a.H + r] = valid ? v : 0.f;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t, n] = sum_{i<k} p[t,i] partial[t k + i, n] (i ascending, FMA
// chain) then + sigmoid(g.x_t) partial_shared[t, n].  Pairs whose id is out of
// range contribute nothing.
// Four consecutive partial values as floats: fp32 rows (staged path) or
// float16 rows (prefill path).
__device__ __forceinline__ float4 load_part4(const float* p, size_t row, int H, int n4) {
  return reinterpret_cast<const float4*>(p + row * H)[n4];
}

__device__ __forceinline__ float4 load_part4(const _Float16* p, size_t row, int H, int n4) {
  const uint2 v = reinterpret_cast<const uint2*>(p + row * H)[n4];
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 a = __builtin_bit_cast(h2, v.x), b = __builtin_bit_cast(h2, v.y);
  return make_float4(static_cast<float>(a[0]), static_cast<float>(a[1]), static_cast<float>(b[0]),
                     static_cast<float>(b[1]));
}

template <int OUT, typename PT>
__global__ __launch_bounds__(256) void k_combine(const PT* __restrict__ partial, const int32_t* __restrict__ ids,
                                                 const float* __restrict__ wts, const float* __restrict__ gate,
                                                 void* __restrict__ out, int T, int k, int H, int E) {
  // one thread per 4 consecutive outputs of one token; the partial rows of a
  // group of pairs are all requested before any is used, and an unusable
  // expert id only masks its term (same order of operations as before)
  constexpr int kGroup = 4;
  const int h4 = H / 4;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(T) * h4) return;
  const int t = static_cast<int>(idx / h4);
  const int n4 = static_cast<int>(idx % h4);
  const float4 sh = load_part4(partial, static_cast<size_t>(T) * k + t, H, n4);
  const float g = gate[t];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < k; i0 += kGroup) {
    float4 p[kGroup];
    float w[kGroup];
    bool ok[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const int i = i0 + j < k ? i0 + j : i0;
      const int e = ids[t * k + i];
      ok[j] = i0 + j < k && e >= 0 && e < E;
      w[j] = wts[t * k + i];
      p[j] = load_part4(partial, static_cast<size_t>(t) * k + i, H, n4);
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (ok[j]) {
        acc.x = fmaf(w[j], p[j].x, acc.x);
        acc.y = fmaf(w[j], p[j].y, acc.y);
        acc.z = fmaf(w[j], p[j].z, acc.z);
        acc.w = fmaf(w[j], p[j].w, acc.w);
      }
    }
  }
  acc.x = fmaf(g, sh.x, acc.x);
  acc.y = fmaf(g, sh.y, acc.y);
  acc.z = fmaf(g, sh.z, acc.z);
  acc.w = fmaf(g, sh.w, acc.w);
  if constexpr (OUT == kF32) {
    reinterpret_cast<float4*>(out)[idx] = acc;
  } else {
    const uint32_t lo = f32_to_bf16(acc.x) | (static_cast<uint32_t>(f32_to_bf16(acc.y)) << 16);
    const uint32_t hi = f32_to_bf16(acc.z) | (static_cast<uint32_t>(f32_to_bf16(acc.w)) << 16);
    reinterpret_cast<uint2*>(out)[idx] = make_uint2(lo, hi);
  }
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// The device error flags into *status, then cleared (one thread).
__global__ void k_take_flags(uint32_t* flags, uint32_t* status) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    *status = *flags;
    *flags = 0u;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers.

static int last_launch_error() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

// x_next = x + y per element: the sum in fp32, rounded to nearest even when
// the activations are bf16.  Each element is read and written by one thread,
// so x_next may be x.
template <int ACT>
// x_next may be x (the in-place step): no pointer here is restrict-qualified,
// and each element is read before it is written by the same thread.
__global__ __launch_bounds__(256) void k_residual(const void* x, const float* y, void* x_next, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  if constexpr (ACT == kBF16) {
    const float xv = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(x)[i]) << 16);
    static_cast<uint16_t*>(x_next)[i] = f32_to_bf16(xv + y[i]);
  } else {
    static_cast<float*>(x_next)[i] = static_cast<const float*>(x)[i] + y[i];
  }
}

int launch_residual(int act_dtype, const void* x, const float* y, void* x_next, int64_t n, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  if (act_dtype == kBF16)
    hipLaunchKernelGGL(k_residual<kBF16>, dim3(blocks), dim3(256), 0, stream, x, y, x_next, n);
  else
    hipLaunchKernelGGL(k_residual<kF32>, dim3(blocks), dim3(256), 0, stream, x, y, x_next, n);
  return last_launch_error();
}

int launch_take_flags(uint32_t* flags, uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(k_take_flags, dim3(1), dim3(64), 0, stream, flags, status);
  return last_launch_error();
}

int launch_ws_init(uint8_t* ws, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 4;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(ws), n, 0u);
  return last_launch_error();
}

int launch_router_topk(const Call& c, int32_t* ids2, float* wts2) {
  const moe_desc& d = c.d;
  float* logits = reinterpret_cast<float*>(c.ws + c.L.logits);
  int32_t* ids = reinterpret_cast<int32_t*>(c.ws + c.L.ids);
  float* wts = reinterpret_cast<float*>(c.ws + c.L.wts);
  const int spr = d.hidden / kSegCodes;
  const int rpp = spr >= kWave ? 1 : kWave / spr;
  const int nsl = spr > kWave ? spr / kWave : 1;
  const int waves = (d.n_experts + rpp - 1) / rpp;
  const dim3 grid((waves + 3) / 4), block(256);
#define ROUTER(ACT, NSL) \
  launch_kernel(k_router_logits<ACT, NSL>, grid, block, 0, c.stream, c.x, c.router_w, logits, c.T, d.hidden, d.n_experts)
  (void)nsl;
  if (d.act_dtype == kF32) ROUTER(kF32, 1); else ROUTER(kBF16, 1);
#undef ROUTER
  return launch_topk(c, logits, ids, wts, ids2, wts2);
}

int launch_topk(const Call& c, const float* logits, int32_t* ids, float* wts, int32_t* ids2, float* wts2) {
  launch_kernel(k_topk, dim3((c.T + kTopkWaves - 1) / kTopkWaves), dim3(kTopkWaves * kWave), 0, c.stream, logits,
                c.T, c.d.n_experts, c.d.top_k, ids, wts, ids2, wts2);
  return last_launch_error();
}

int launch_experts(const Call& c) {
  const moe_desc& d = c.d;
  uint32_t* flags = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  float* gate = reinterpret_cast<float*>(c.ws + c.L.gate);
  int32_t* ucount = reinterpret_cast<int32_t*>(c.ws + c.L.ucount);
  int32_t* uniq = reinterpret_cast<int32_t*>(c.ws + c.L.uniq);
  int32_t* ustart = reinterpret_cast<int32_t*>(c.ws + c.L.ustart);
  int32_t* plist = reinterpret_cast<int32_t*>(c.ws + c.L.plist);
  float* h = reinterpret_cast<float*>(c.ws + c.L.h);
  float* partial = reinterpret_cast<float*>(c.ws + c.L.partial);
  const void* gvec = c.shared + d.shared_stride;

  // dispatch + gate
#define DISPATCH(ACT, NSL)                                                                                      \
  launch_kernel(k_dispatch<ACT, NSL>, dim3(1), dim3(kDispatchThreads), 0, c.stream, c.ids, c.T, d.top_k, \
                     d.n_experts, d.hidden, c.x, gvec, gate, ucount, uniq, ustart, plist, flags)
  if (d.act_dtype == kF32) DISPATCH(kF32, 1); else DISPATCH(kBF16, 1);
#undef DISPATCH

  // gate/up
  {
    const int spr = d.hidden / kSegCodes;
    const int rpp = spr >= kWave ? 1 : kWave / spr;
    const int npass = rpp >= kMaxPass ? 1 : kMaxPass / rpp;
    const int rpb = 4 * npass * rpp;
    GateUpArgs a;
    a.x = c.x;
    a.slot_table = c.slot_table;
    a.pool = c.pool;
    a.shared = c.shared;
    a.ucount = ucount;
    a.uniq = uniq;
    a.ustart = ustart;
    a.plist = plist;
    a.h = h;
    a.flags = flags;
    a.pool_bytes = d.pool_bytes;
    a.T = c.T;
    a.k = d.top_k;
    a.H = d.hidden;
    a.I = d.inter;
    a.SI = d.shared_inter;
    a.umax = c.L.umax;
    a.bpe_r = (d.inter + rpb - 1) / rpb;
    a.bpe_s = (d.shared_inter + rpb - 1) / rpb;
    a.hstride = c.L.hstride;
    const dim3 grid(a.umax * a.bpe_r + a.bpe_s), block(256);
#define GATEUP(BITS, SB, ACT, NSL, TOKC) launch_kernel(k_gateup<BITS, SB, ACT, NSL, TOKC>, grid, block, 0, c.stream, a)
#define GATEUP_T(BITS, SB, ACT, NSL) \
  do { if (c.T == 1) GATEUP(BITS, SB, ACT, NSL, 1); else GATEUP(BITS, SB, ACT, NSL, 2); } while (0)
#define GATEUP_N(BITS, SB, ACT) GATEUP_T(BITS, SB, ACT, 1)
#define GATEUP_A(BITS, SB) \
  do { if (d.act_dtype == kF32) GATEUP_N(BITS, SB, kF32); else GATEUP_N(BITS, SB, kBF16); } while (0)
#define GATEUP_S(BITS) \
  do { if (d.sb_dtype == kF32) GATEUP_A(BITS, kF32); else GATEUP_A(BITS, kBF16); } while (0)
    if (d.bits == 4) GATEUP_S(4); else GATEUP_S(8);
#undef GATEUP_S
#undef GATEUP_A
#undef GATEUP_N
#undef GATEUP_T
#undef GATEUP
  }
  // down
  {
    const int rpp_r = (d.inter / kSegCodes) >= kWave ? 1 : kWave / (d.inter / kSegCodes);
    const int rpp_s = (d.shared_inter / kSegCodes) >= kWave ? 1 : kWave / (d.shared_inter / kSegCodes);
    const int np_r = rpp_r >= kMaxPass ? 1 : kMaxPass / rpp_r;
    const int np_s = rpp_s >= kMaxPass ? 1 : kMaxPass / rpp_s;
    const int rpb_r = 4 * np_r * rpp_r, rpb_s = 4 * np_s * rpp_s;
    DownArgs a;
    a.slot_table = c.slot_table;
    a.pool = c.pool;
    a.shared = c.shared;
    a.ucount = ucount;
    a.uniq = uniq;
    a.ustart = ustart;
    a.plist = plist;
    a.h = h;
    a.partial = partial;
    a.flags = flags;
    a.pool_bytes = d.pool_bytes;
    a.T = c.T;
    a.k = d.top_k;
    a.H = d.hidden;
    a.I = d.inter;
    a.SI = d.shared_inter;
    a.umax = c.L.umax;
    a.bpe = (d.hidden + rpb_r - 1) / rpb_r;
    a.hstride = c.L.hstride;
    const int bpe_s = (d.hidden + rpb_s - 1) / rpb_s;
    const dim3 grid(a.umax * a.bpe + bpe_s), block(256);
#define DOWN(BITS, SB) launch_kernel(k_down<BITS, SB, 1>, grid, block, 0, c.stream, a)
#define DOWN_S(BITS) do { if (d.sb_dtype == kF32) DOWN(BITS, kF32); else DOWN(BITS, kBF16); } while (0)
    if (d.bits == 4) DOWN_S(4); else DOWN_S(8);
#undef DOWN_S
#undef DOWN
  }
  return launch_combine(c, partial, gate);
}

template <typename PT>
static int launch_combine_t(const Call& c, const PT* partial, const float* gate) {
  const moe_desc& d = c.d;
  const size_t n = static_cast<size_t>(c.T) * d.hidden / 4;   // one thread per 4 outputs (H % 64 == 0)
  const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
  if (d.out_dtype == kF32)
    launch_kernel(k_combine<kF32, PT>, grid, block, 0, c.stream, partial, c.ids, c.wts, gate, c.out, c.T, d.top_k,
                  d.hidden, d.n_experts);
  else
    launch_kernel(k_combine<kBF16, PT>, grid, block, 0, c.stream, partial, c.ids, c.wts, gate, c.out, c.T,
                  d.top_k, d.hidden, d.n_experts);
  return last_launch_error();
}

int launch_combine(const Call& c, const float* partial, const float* gate) { return launch_combine_t(c, partial, gate); }

int launch_combine(const Call& c, const _Float16* partial, const float* gate) {
  return launch_combine_t(c, partial, gate);
}

}  // namespace moe
