// Gated delta rule at decode time (gfx950): B sequences advanced by T tokens.
//
// Rule (Gated DeltaNet as its authors publish it; the pages name it in the
// linlog.top article, design 4, without an equation), per value head with
// state S [d_v, d_k]:
//   S <- alpha S (I - beta k k^T) + beta v k^T = alpha S + u k^T,
//   u = beta (v - alpha S k),   out = S q      (q, k L2-normalised, q scaled)
// Each row of S evolves on its own: row r needs only k, q, v[r], alpha, beta.
//
// Organisation.  The work is bound by HBM: every token reads and writes the
// whole state (64 KB per 128 x 128 head) and does 4 flops per element.  So:
//   - a block owns 16 rows of one head's state (P = 1 pass; the kernel takes
//     more passes as a template argument, measured slower) and holds them in
//     registers for all T tokens of the call (one read and one write of the
//     state per call, whatever T), read and written with non-temporal
//     accesses (the state is streamed once per call and should not displace
//     the caches' other lines);
//   - 16 lanes share a row, each with 4-column chunks at 64 m + 4 j
//     (m < d_k / 64), so that a wave's 16-byte loads cover 256 contiguous
//     bytes of each of its 4 rows;
//   - a row's dot products (S k and S q) are 16-lane sums on DPP row
//     permutations that give every lane the same bits;
//   - the next token's q, k, v, alpha and beta are requested before the
//     current token's arithmetic, so their latency hides behind it;
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>

#include "device_common.h"
#include "gdn_recurrence.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGThr = 256;                        // 4 waves
constexpr int kRowLanes = 16;                     // lanes per state row
constexpr int kRowsPerPass = kGThr / kRowLanes;   // 16 rows per block pass

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GdnArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  float* state;
  void* out;
  int T, nk, nv, dv;
  float scale, eps;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row; every lane ends with the same bits
// (each step adds a value to its mirror partner's, and the partner adds the
// same two values in the other order).
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp<0x140>(v);   // mirror within 16
  v = v + dpp<0x141>(v);   // mirror within 8
  v = v + dpp<0x1B>(v);    // reverse within 4
  v = v + dpp<0xB1>(v);    // swap pairs
  return v;
}

// One token's inputs for this lane: its q and k columns, the v entries of
// its rows, alpha and beta.
template <int NC, int P, int ACT>
struct TokIn {
  uint32_t q[NC][ACT == kF32 ? 4 : 2];
  uint32_t k[NC][ACT == kF32 ? 4 : 2];
  float v[P];
  float alpha, beta;
};

template <int NC, int ACT>
__device__ __forceinline__ void load_cols(const void* base, int64_t off, int j, uint32_t (&dst)[NC][ACT == kF32 ? 4 : 2]) {
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    const int64_t c = off + 64 * m + 4 * j;
    if constexpr (ACT == kF32) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + c);
      dst[m][0] = w.x; dst[m][1] = w.y; dst[m][2] = w.z; dst[m][3] = w.w;
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + c);
      dst[m][0] = w.x; dst[m][1] = w.y;
    }
  }
}

template <int NC, int ACT>
__device__ __forceinline__ void cols_f32(const uint32_t (&src)[NC][ACT == kF32 ? 4 : 2], float (&dst)[NC][4]) {
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    if constexpr (ACT == kF32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[m][i] = __uint_as_float(src[m][i]);
    } else {
      dst[m][0] = bf16_to_f32(static_cast<uint16_t>(src[m][0] & 0xffffu));
      dst[m][1] = bf16_to_f32(static_cast<uint16_t>(src[m][0] >> 16));
      dst[m][2] = bf16_to_f32(static_cast<uint16_t>(src[m][1] & 0xffffu));
      dst[m][3] = bf16_to_f32(static_cast<uint16_t>(src[m][1] >> 16));
    }
  }
}

template <int DK, int P, int ACT>
__device__ __forceinline__ void load_token(const GdnArgs& a, int64_t tok, int h, int kh, int row_lane0, int j,
                                           TokIn<DK / 64, P, ACT>& in) {
  constexpr int NC = DK / 64;
  const int64_t qk = (tok * a.nk + kh) * DK;
  load_cols<NC, ACT>(a.q, qk, j, in.q);
  load_cols<NC, ACT>(a.k, qk, j, in.k);
  const int64_t vb = (tok * a.nv + h) * static_cast<int64_t>(a.dv) + row_lane0;
#pragma unroll
  for (int p = 0; p < P; ++p) in.v[p] = load_scalar<ACT>(a.v, static_cast<size_t>(vb + p * kRowsPerPass));
  in.alpha = a.alpha[tok * a.nv + h];
  in.beta = a.beta[tok * a.nv + h];
}

template <int DK, int P, int ACT, int OUT>
__global__ __launch_bounds__(kGThr) void k_gdn_recurrence(GdnArgs a) {
  constexpr int NC = DK / 64;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int j = lane & (kRowLanes - 1);
  const int sub = lane / kRowLanes;
  const int nz = a.dv / (kRowsPerPass * P);
  const int64_t blk = blockIdx.x;
  const int z = static_cast<int>(blk % nz);
  const int64_t bh = blk / nz;
  const int h = static_cast<int>(bh % a.nv);
  const int64_t b = bh / a.nv;
  const int kh = h / (a.nv / a.nk);
  // this lane's rows: r_p = row_lane0 + 16 p
  const int row_lane0 = z * kRowsPerPass * P + wave * 4 + sub;

  float* st = a.state + (b * a.nv + h) * static_cast<int64_t>(a.dv) * DK;
  float S[P][NC][4];
#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      const f32x4 w = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(st + static_cast<int64_t>(row_lane0 + p * kRowsPerPass) * DK + 64 * m + 4 * j));
      S[p][m][0] = w[0]; S[p][m][1] = w[1]; S[p][m][2] = w[2]; S[p][m][3] = w[3];
    }
  }

  TokIn<NC, P, ACT> cur;
  load_token<DK, P, ACT>(a, b * a.T, h, kh, row_lane0, j, cur);
  for (int t = 0; t < a.T; ++t) {
    const int64_t tok = b * a.T + t;
    TokIn<NC, P, ACT> nxt;
    if (t + 1 < a.T) load_token<DK, P, ACT>(a, tok + 1, h, kh, row_lane0, j, nxt);

    float qv[NC][4], kv[NC][4];
    cols_f32<NC, ACT>(cur.q, qv);
    cols_f32<NC, ACT>(cur.k, kv);
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int m = 0; m < NC; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sq = fmaf(qv[m][i], qv[m][i], sq);
        sk = fmaf(kv[m][i], kv[m][i], sk);
      }
    }
    sq = row16_sum(sq);
    sk = row16_sum(sk);
    const float rq = a.scale / sqrtf(sq + a.eps);
    const float rk = 1.0f / sqrtf(sk + a.eps);
#pragma unroll
    for (int m = 0; m < NC; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[m][i] *= rq;
        kv[m][i] *= rk;
      }
    }
    const float al = cur.alpha, be = cur.beta;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float w = 0.f;
#pragma unroll
      for (int m = 0; m < NC; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w = fmaf(S[p][m][i], kv[m][i], w);
      }
      w = row16_sum(w);
      const float u = be * (cur.v[p] - al * w);
      float o = 0.f;
#pragma unroll
      for (int m = 0; m < NC; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          S[p][m][i] = fmaf(u, kv[m][i], al * S[p][m][i]);
          o = fmaf(S[p][m][i], qv[m][i], o);
        }
      }
      o = row16_sum(o);
      if (j == 0) {
        const int64_t oi = (tok * a.nv + h) * static_cast<int64_t>(a.dv) + row_lane0 + p * kRowsPerPass;
        if constexpr (OUT == kF32) static_cast<float*>(a.out)[oi] = o;
        else static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(o);
      }
    }
    if (t + 1 < a.T) cur = nxt;
  }

#pragma unroll
  for (int p = 0; p < P; ++p) {
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      const f32x4 w = {S[p][m][0], S[p][m][1], S[p][m][2], S[p][m][3]};
      __builtin_nontemporal_store(
          w, reinterpret_cast<f32x4*>(st + static_cast<int64_t>(row_lane0 + p * kRowsPerPass) * DK + 64 * m + 4 * j));
    }
  }
}

template <int DK, int P, int ACT, int OUT>
hipError_t launch_p(const GdnArgs& a, int64_t blocks, hipStream_t s) {
  hipLaunchKernelGGL((k_gdn_recurrence<DK, P, ACT, OUT>), dim3(static_cast<uint32_t>(blocks)), dim3(kGThr), 0, s, a);
  return hipGetLastError();
}

template <int DK, int ACT, int OUT>
hipError_t launch_dk(const GdnArgs& a, int P, int64_t blocks, hipStream_t s) {
  (void)P;
  return launch_p<DK, 1, ACT, OUT>(a, blocks, s);
}

template <int ACT, int OUT>
hipError_t launch_act(const GdnArgs& a, int dk, int P, int64_t blocks, hipStream_t s) {
  return dk == 128 ? launch_dk<128, ACT, OUT>(a, P, blocks, s) : launch_dk<64, ACT, OUT>(a, P, blocks, s);
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int bad(const char* fmt, long long x = 0, long long y = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, x, y);
  return api_fail(MOE_EINVAL, buf);
}

}  // namespace
}  // namespace moe

extern "C" int gdn_recurrence_forward(const gdn_desc* d, int32_t B, int32_t T, const void* q, const void* k,
                                      const void* v, const float* alpha, const float* beta, float* state, void* out,
                                      void* stream) {
  using namespace moe;
  if (!d) return bad("descriptor is NULL");
  if (d->n_k_heads < 1 || d->n_v_heads < 1 || d->n_v_heads > 1024 || d->n_v_heads % d->n_k_heads != 0)
    return bad("n_v_heads=%lld must be in [1, 1024] and a multiple of n_k_heads=%lld", d->n_v_heads, d->n_k_heads);
  if (d->d_k != 64 && d->d_k != 128) return bad("d_k=%lld must be 64 or 128", d->d_k);
  if (d->d_v < 16 || d->d_v > 256 || d->d_v % 16 != 0) return bad("d_v=%lld must be a multiple of 16 in [16, 256]", d->d_v);
  if ((d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) || (d->out_dtype != MOE_F32 && d->out_dtype != MOE_BF16))
    return bad("act_dtype=%lld / out_dtype=%lld must be MOE_F32 or MOE_BF16", d->act_dtype, d->out_dtype);
  if (!std::isfinite(d->scale)) return bad("scale must be finite");
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return bad("eps must be finite and >= 0");
  if (B < 0 || B > (1 << 20) || T < 0 || T > (1 << 20)) return bad("B=%lld and T=%lld must be in [0, 2^20]", B, T);
  if (B == 0 || T == 0) return api_ok();
  if (!q || !k || !v || !alpha || !beta || !state || !out) return bad("NULL pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return bad("q, k, v, state and out must be 16-byte aligned, alpha and beta 4-byte aligned");
  const int64_t act = d->act_dtype == MOE_F32 ? 4 : 2, osz = d->out_dtype == MOE_F32 ? 4 : 2;
  const int64_t bt = static_cast<int64_t>(B) * T;
  const int64_t n_q = bt * d->n_k_heads * d->d_k * act, n_v = bt * d->n_v_heads * d->d_v * act;
  const int64_t n_g = bt * d->n_v_heads * 4, n_o = bt * d->n_v_heads * d->d_v * osz;
  const int64_t n_s = static_cast<int64_t>(B) * d->n_v_heads * d->d_v * d->d_k * 4;
  const void* ins[5] = {q, k, v, alpha, beta};
  const int64_t in_n[5] = {n_q, n_q, n_v, n_g, n_g};
  for (int i = 0; i < 5; ++i) {
    if (overlaps(state, n_s, ins[i], in_n[i])) return bad("state overlaps input %lld", i);
    if (overlaps(out, n_o, ins[i], in_n[i])) return bad("out overlaps input %lld", i);
  }
  if (overlaps(state, n_s, out, n_o)) return bad("state and out overlap");

  // one pass of 16 rows per block (measured fastest at every batch size:
  // the most blocks, the most loads in flight)
  const int64_t heads = static_cast<int64_t>(B) * d->n_v_heads;
  const int P = 1;
  const int64_t blocks = heads * (d->d_v / kRowsPerPass);
  if (blocks > 0x7fffffffLL) return bad("B * n_v_heads * d_v = %lld rows is too many for one launch", heads * d->d_v);

  GdnArgs a;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.state = state; a.out = out;
  a.T = T; a.nk = d->n_k_heads; a.nv = d->n_v_heads; a.dv = d->d_v;
  a.scale = d->scale; a.eps = d->eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d->act_dtype == MOE_BF16)
    e = d->out_dtype == MOE_BF16 ? launch_act<kBF16, kBF16>(a, d->d_k, P, blocks, s)
                                 : launch_act<kBF16, kF32>(a, d->d_k, P, blocks, s);
  else
    e = d->out_dtype == MOE_BF16 ? launch_act<kF32, kBF16>(a, d->d_k, P, blocks, s)
                                 : launch_act<kF32, kF32>(a, d->d_k, P, blocks, s);
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof(buf), "gated delta rule launch failed: %s", hipGetErrorString(e));
    return api_fail(MOE_EHIP, buf);
  }
  return api_ok();
}
