// Scalar GPU path of the MoE layer: one thread per output value (a logit, a
// token's gate, one element of h, one element of a down row, one output
// element), no cross-lane operations and none of the fast kernels' helpers.
//
// The pages check their fast GPU kernels against scalar ones that give
// identical output (Swiftlet README translation, "Correctness"; linlog.top
// article, "Correctness guarantees").  For that, this file states on its own
// the order in which the fast kernels associate every sum, and follows it:
//   * a matrix row is cut into segments of 32 codes; a segment's value is
//     fmaf(s, Q, b * X) with X the sum of its 32 inputs and Q the sum of
//     code * input, formed as listed in seg_dot / seg_x below;
//   * the segment values of a row are combined by the butterfly of
//     `butterfly` (the pairing the fast kernels' lane reductions use), and the
//     gate and up rows of full 64-segment rows by `gu_total`;
//   * the layer output is sum_i p_i down_i + sigma down_shared, one FMA chain
//     over the ranks i in order, then the shared expert.
// Routing is the exact order (logit descending, id ascending) with +0 and -0
// ranked equal; weights p_i = exp(l_i - l_0) / sum_j exp(l_j - l_0), the sum
// taken in rank order.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kSegLen = 32;       // codes (or inputs) per segment
constexpr int kMaxSegs = 64;      // segments per row (rows are at most 2048 long)
constexpr uint32_t kBadRange = 1u;

__device__ inline float bf16v(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float -> bf16 bits, nearest even (NaN kept quiet)
__device__ inline uint16_t to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// element j of a stored dense vector (float32 or bf16)
__device__ inline float act_at(const uint8_t* p, int j, int dt) {
  return dt == MOE_F32 ? reinterpret_cast<const float*>(p)[j] : bf16v(reinterpret_cast<const uint16_t*>(p)[j]);
}

// code c of a packed row (int4: low nibble first in little-endian words;
// int8: byte order)
__device__ inline uint32_t code_at(const uint8_t* row, int c, int bits) {
  if (bits == 4) return (row[c >> 1] >> ((c & 1) * 4)) & 0xfu;
  return row[c];
}

// Partner of entry L in each butterfly step: mirror within 16, mirror within
// 8, reversal within 4, swap of neighbours, then L ^ 16 and L ^ 32.
__device__ inline int mirror16(int L) { return (L & ~15) | (15 - (L & 15)); }
__device__ inline int mirror8(int L) { return (L & ~7) | (7 - (L & 7)); }
__device__ inline int reverse4(int L) { return (L & ~3) | (3 - (L & 3)); }

// One step: every entry gets the sum of itself and its partner.
template <typename P>
__device__ inline void pair_step(float (&a)[kMaxSegs], int w, P partner) {
  float b[kMaxSegs];
  for (int L = 0; L < w; ++L) b[L] = a[L] + a[partner(L)];
  for (int L = 0; L < w; ++L) a[L] = b[L];
}

// Total of w segment values (w a power of two <= 64) in the fast kernels'
// order; every entry ends equal, entry 0 is returned.
__device__ inline float butterfly(float (&a)[kMaxSegs], int w) {
  if (w >= 16) pair_step(a, w, [](int L) { return mirror16(L); });
  if (w >= 8) pair_step(a, w, [](int L) { return mirror8(L); });
  if (w >= 4) pair_step(a, w, [](int L) { return reverse4(L); });
  if (w >= 2) pair_step(a, w, [](int L) { return L ^ 1; });
  if (w >= 32) pair_step(a, w, [](int L) { return L ^ 16; });
  if (w >= 64) pair_step(a, w, [](int L) { return L ^ 32; });
  return a[0];
}

// Total of a full row of 64 segment values as the fast kernels form the gate
// and up totals together: segment L and segment L + 32 first, then the
// butterfly over the 32 sums.
__device__ inline float gu_total(const float (&a)[kMaxSegs]) {
  float b[kMaxSegs];
  for (int L = 0; L < 32; ++L) b[L] = a[L] + a[L + 32];
  return butterfly(b, 32);
}

typedef __bf16 bf16pair __attribute__((ext_vector_type(2)));

// v_dot2_f32_bf16: acc + a.lo b.lo + a.hi b.hi (both products exact in float32)
__device__ inline float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16pair, a), __builtin_bit_cast(bf16pair, b), acc,
                                         false);
}

// Segment of a bf16 input row with int4 codes: the inputs in pairs
// (x_2j, x_2j+1) as stored, each code as the bf16 value 128 + q (exact), two
// chains of dot2 over the pairs: chain 0 takes pairs 0, 2, 4, ... chain 1
// pairs 1, 3, 5, ... each in order, then chain 0 + chain 1.  D = sum
// (128 + q) x and X = sum x (the same chains with (1, 1) for the codes);
// Q = D - 128 X.
__device__ inline void seg_bf16_int4(const uint8_t* codes, const uint16_t* x, int seg, float* D, float* X) {
  float d0 = 0.f, d1 = 0.f, s0 = 0.f, s1 = 0.f;
  for (int j = 0; j < kSegLen / 2; ++j) {
    const int c = seg * kSegLen + 2 * j;
    const uint32_t xp = static_cast<uint32_t>(x[c]) | (static_cast<uint32_t>(x[c + 1]) << 16);
    const uint32_t qp = (0x4300u | code_at(codes, c, 4)) | ((0x4300u | code_at(codes, c + 1, 4)) << 16);
    if (j % 2 == 0) {
      d0 = dot2(qp, xp, d0);
      s0 = dot2(0x3f803f80u, xp, s0);
    } else {
      d1 = dot2(qp, xp, d1);
      s1 = dot2(0x3f803f80u, xp, s1);
    }
  }
  *D = d0 + d1;
  *X = s0 + s1;
}

// Any other segment: X is the 32 inputs added in order; Q is two float32
// FMA chains added at the end.  int4: chain 0 takes the even codes, chain 1
// the odd ones, each in code order.  int8: chain 0 codes 4m and 4m + 2,
// chain 1 codes 4m + 1 and 4m + 3, in code order.
__device__ inline void seg_float(const uint8_t* codes, const float* v, int bits, float* Q, float* X) {
  float a0 = 0.f, a1 = 0.f, xs = 0.f;
  for (int c = 0; c < kSegLen; ++c) xs += v[c];
  for (int c = 0; c < kSegLen; ++c) {
    const float q = static_cast<float>(code_at(codes, c, bits));
    if (c % 2 == 0) a0 = fmaf(q, v[c], a0);
    else a1 = fmaf(q, v[c], a1);
  }
  *Q = a0 + a1;
  *X = xs;
}

__device__ inline float silu_fast(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

__device__ inline bool blob_ok(int64_t off, int64_t blob, int64_t pool_bytes) {
  return off >= 0 && (off & 255) == 0 && off <= pool_bytes - blob;
}

struct ScalarArgs {
  const uint8_t* x;
  const uint8_t* router;
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  void* out;
  float* logits;        // [T, E]
  int32_t* ids;         // [T, k]
  float* wts;           // [T, k]
  float* gate;          // [T]
  float* h;             // [T k + T, hs]
  float* part;          // [T k + T, H]
  int32_t* ids_out;
  float* wts_out;
  uint32_t* flags;
  int64_t pool_bytes, shared_stride;
  int T, H, E, k, I, SI, hs, bits, act, sb, out_dt;
};

// code planes and scale planes of a blob of intermediate size `inter`
struct BlobPlanes {
  int64_t q, s, blob;
};

__device__ inline BlobPlanes blob_planes(int H, int inter, int bits, int sb) {
  BlobPlanes p;
  p.q = static_cast<int64_t>(H) * inter * bits / 8;
  p.s = static_cast<int64_t>(H) * (inter / 64) * (sb == MOE_F32 ? 4 : 2);
  p.blob = 3 * p.q + 6 * p.s;
  return p;
}

__device__ inline float scale_at(const uint8_t* plane, int64_t idx, int sb) {
  return sb == MOE_F32 ? reinterpret_cast<const float*>(plane)[idx] : bf16v(reinterpret_cast<const uint16_t*>(plane)[idx]);
}

// logit (t, e): segment s = fmaf chain over its 32 products x * R, the
// segments combined by the butterfly
__global__ void k_sc_router(ScalarArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(a.T) * a.E) return;
  const int t = static_cast<int>(idx / a.E), e = static_cast<int>(idx % a.E);
  const int asz = a.act == MOE_F32 ? 4 : 2;
  const uint8_t* xr = a.x + static_cast<size_t>(t) * a.H * asz;
  const uint8_t* rr = a.router + static_cast<size_t>(e) * a.H * asz;
  const int nseg = a.H / kSegLen;
  float v[kMaxSegs];
  for (int s = 0; s < nseg; ++s) {
    float acc = 0.f;
    for (int c = s * kSegLen; c < (s + 1) * kSegLen; ++c) acc = fmaf(act_at(xr, c, a.act), act_at(rr, c, a.act), acc);
    v[s] = acc;
  }
  a.logits[idx] = butterfly(v, nseg);
}

// order key: larger logit, larger key; +0 and -0 equal; at least 1
__device__ inline uint32_t rank_key(float f) {
  const uint32_t b = __float_as_uint(f);
  uint32_t k = (b & 0x7fffffffu) == 0 ? 0x80000000u : ((b & 0x80000000u) ? ~b : (b | 0x80000000u));
  return k > 1u ? k : 1u;
}

// token t: its k experts by (key descending, id ascending), the weights, and
// its shared-expert gate sigmoid(g . x) (64 segment slots, the empty ones 0)
__global__ void k_sc_topk(ScalarArgs a) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.T) return;
  const float* lg = a.logits + static_cast<size_t>(t) * a.E;
  int prev_id = -1;
  uint32_t prev_key = 0xffffffffu;
  for (int i = 0; i < a.k; ++i) {
    // the best entry strictly after (prev_key, prev_id) in the order
    int best = -1;
    uint32_t bk = 0;
    for (int e = 0; e < a.E; ++e) {
      const uint32_t ke = rank_key(lg[e]);
      const bool after = ke < prev_key || (ke == prev_key && e > prev_id);
      if (after && (best < 0 || ke > bk)) {
        best = e;
        bk = ke;
      }
    }
    a.ids[t * a.k + i] = best;
    prev_id = best;
    prev_key = bk;
  }
  const float top = lg[a.ids[t * a.k]];
  float sum = 0.f;
  for (int i = 0; i < a.k; ++i) sum += expf(lg[a.ids[t * a.k + i]] - top);
  for (int i = 0; i < a.k; ++i) {
    const float p = expf(lg[a.ids[t * a.k + i]] - top) / sum;
    a.wts[t * a.k + i] = p;
    if (a.ids_out) a.ids_out[t * a.k + i] = a.ids[t * a.k + i];
    if (a.wts_out) a.wts_out[t * a.k + i] = p;
  }
  const int asz = a.act == MOE_F32 ? 4 : 2;
  const uint8_t* xr = a.x + static_cast<size_t>(t) * a.H * asz;
  const uint8_t* gv = a.shared + a.shared_stride;
  float v[kMaxSegs];
  for (int s = 0; s < kMaxSegs; ++s) {
    float acc = 0.f;
    if (s < a.H / kSegLen)
      for (int c = s * kSegLen; c < (s + 1) * kSegLen; ++c) acc = fmaf(act_at(xr, c, a.act), act_at(gv, c, a.act), acc);
    v[s] = acc;
  }
  const float g = butterfly(v, kMaxSegs);
  a.gate[t] = 1.0f / (1.0f + expf(-g));
}

// h (t, i, r) = silu(gate row r . x_t) * (up row r . x_t) of the token's rank-i
// expert (i == k: the shared expert)
__global__ void k_sc_gateup(ScalarArgs a) {
  const int rmax = a.I > a.SI ? a.I : a.SI;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(a.T) * (a.k + 1) * rmax) return;
  const int r = static_cast<int>(idx % rmax);
  const int ti = static_cast<int>(idx / rmax);
  const int t = ti / (a.k + 1), i = ti % (a.k + 1);
  const bool sh = i == a.k;
  const int rows = sh ? a.SI : a.I;
  if (r >= rows) return;
  const BlobPlanes pl = blob_planes(a.H, rows, a.bits, a.sb);
  const uint8_t* blob = a.shared;
  bool ok = true;
  if (!sh) {
    const int e = a.ids[t * a.k + i];
    const int64_t off = (e >= 0 && e < a.E) ? a.slot_table[e] : -1;
    ok = blob_ok(off, pl.blob, a.pool_bytes);
    blob = a.pool + (ok ? off : 0);
    if (!ok) __hip_atomic_fetch_or(a.flags, kBadRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const size_t hrow = sh ? static_cast<size_t>(a.T) * a.k + t : static_cast<size_t>(t) * a.k + i;
  if (!ok) {
    a.h[hrow * a.hs + r] = 0.f;
    return;
  }
  const int nseg = a.H / kSegLen;
  const int64_t rowb = static_cast<int64_t>(a.H) * a.bits / 8;
  const uint8_t* cg = blob + r * rowb;
  const uint8_t* cu = blob + pl.q + r * rowb;
  const int gpr = a.H / 64;
  const int asz = a.act == MOE_F32 ? 4 : 2;
  const uint8_t* xr = a.x + static_cast<size_t>(t) * a.H * asz;
  float vg[kMaxSegs], vu[kMaxSegs];
  for (int s = 0; s < nseg; ++s) {
    const int64_t gi = static_cast<int64_t>(r) * gpr + s / 2;
    const float sgv = scale_at(blob + 3 * pl.q, gi, a.sb), suv = scale_at(blob + 3 * pl.q + pl.s, gi, a.sb);
    const float bgv = scale_at(blob + 3 * pl.q + 3 * pl.s, gi, a.sb), buv = scale_at(blob + 3 * pl.q + 4 * pl.s, gi, a.sb);
    if (a.act == MOE_BF16 && a.bits == 4) {
      const uint16_t* x16 = reinterpret_cast<const uint16_t*>(xr);
      float Dg, Du, X;
      seg_bf16_int4(cg, x16, s, &Dg, &X);
      seg_bf16_int4(cu, x16, s, &Du, &X);
      vg[s] = 0.f + fmaf(sgv, Dg - 128.f * X, bgv * X);
      vu[s] = 0.f + fmaf(suv, Du - 128.f * X, buv * X);
    } else {
      float v[kSegLen];
      for (int c = 0; c < kSegLen; ++c) v[c] = act_at(xr, s * kSegLen + c, a.act);
      const int64_t so = static_cast<int64_t>(s) * kSegLen * a.bits / 8;
      float Qg, Qu, X;
      seg_float(cg + so, v, a.bits, &Qg, &X);
      seg_float(cu + so, v, a.bits, &Qu, &X);
      vg[s] = 0.f + fmaf(sgv, Qg, bgv * X);
      vu[s] = 0.f + fmaf(suv, Qu, buv * X);
    }
  }
  float g, u;
  if (nseg == kMaxSegs) {
    g = gu_total(vg);
    u = gu_total(vu);
  } else {
    g = butterfly(vg, nseg);
    u = butterfly(vu, nseg);
  }
  a.h[hrow * a.hs + r] = silu_fast(g) * u;
}

// down element (t, i, n) = row n of the rank-i expert's down matrix . h
__global__ void k_sc_down(ScalarArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(a.T) * (a.k + 1) * a.H) return;
  const int n = static_cast<int>(idx % a.H);
  const int ti = static_cast<int>(idx / a.H);
  const int t = ti / (a.k + 1), i = ti % (a.k + 1);
  const bool sh = i == a.k;
  const int inter = sh ? a.SI : a.I;
  const BlobPlanes pl = blob_planes(a.H, inter, a.bits, a.sb);
  const uint8_t* blob = a.shared;
  bool ok = true;
  if (!sh) {
    const int e = a.ids[t * a.k + i];
    const int64_t off = (e >= 0 && e < a.E) ? a.slot_table[e] : -1;
    ok = blob_ok(off, pl.blob, a.pool_bytes);
    blob = a.pool + (ok ? off : 0);
  }
  const size_t hrow = sh ? static_cast<size_t>(a.T) * a.k + t : static_cast<size_t>(t) * a.k + i;
  if (!ok) {
    a.part[hrow * a.H + n] = 0.f;
    return;
  }
  const int nseg = inter / kSegLen;
  const int64_t rowb = static_cast<int64_t>(inter) * a.bits / 8;
  const uint8_t* cd = blob + 2 * pl.q + n * rowb;
  const int gpr = inter / 64;
  const float* hr = a.h + hrow * a.hs;
  float v[kMaxSegs];
  for (int s = 0; s < nseg; ++s) {
    const int64_t gi = static_cast<int64_t>(n) * gpr + s / 2;
    const float sc = scale_at(blob + 3 * pl.q + 2 * pl.s, gi, a.sb), bi = scale_at(blob + 3 * pl.q + 5 * pl.s, gi, a.sb);
    float Q, X;
    seg_float(cd + static_cast<int64_t>(s) * kSegLen * a.bits / 8, hr + s * kSegLen, a.bits, &Q, &X);
    v[s] = 0.f + fmaf(sc, Q, bi * X);
  }
  a.part[hrow * a.H + n] = butterfly(v, nseg);
}

// out (t, n) = sum over ranks i (in order) of p_i down_i, then + sigma down_shared
__global__ void k_sc_combine(ScalarArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(a.T) * a.H) return;
  const int t = static_cast<int>(idx / a.H), n = static_cast<int>(idx % a.H);
  float acc = 0.f;
  for (int i = 0; i < a.k; ++i) {
    const int e = a.ids[t * a.k + i];
    if (e >= 0 && e < a.E) acc = fmaf(a.wts[t * a.k + i], a.part[(static_cast<size_t>(t) * a.k + i) * a.H + n], acc);
  }
  acc = fmaf(a.gate[t], a.part[(static_cast<size_t>(a.T) * a.k + t) * a.H + n], acc);
  if (a.out_dt == MOE_F32) static_cast<float*>(a.out)[idx] = acc;
  else static_cast<uint16_t*>(a.out)[idx] = to_bf16_bits(acc);
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

}  // namespace

int launch_scalar(const Call& c) {
  const moe_desc& d = c.d;
  ScalarArgs a;
  a.x = static_cast<const uint8_t*>(c.x);
  a.router = static_cast<const uint8_t*>(c.router_w);
  a.slot_table = c.slot_table;
  a.pool = c.pool;
  a.shared = c.shared;
  a.out = c.out;
  a.logits = reinterpret_cast<float*>(c.ws + c.L.logits);
  a.ids = reinterpret_cast<int32_t*>(c.ws + c.L.ids);
  a.wts = reinterpret_cast<float*>(c.ws + c.L.wts);
  a.gate = reinterpret_cast<float*>(c.ws + c.L.gate);
  a.h = reinterpret_cast<float*>(c.ws + c.L.h);
  a.part = reinterpret_cast<float*>(c.ws + c.L.partial);
  a.ids_out = c.ids_out;
  a.wts_out = c.wts_out;
  a.flags = reinterpret_cast<uint32_t*>(c.ws + c.L.ctrl);
  a.pool_bytes = d.pool_bytes;
  a.shared_stride = d.shared_stride;
  a.T = c.T;
  a.H = d.hidden;
  a.E = d.n_experts;
  a.k = d.top_k;
  a.I = d.inter;
  a.SI = d.shared_inter;
  a.hs = c.L.hstride;
  a.bits = d.bits;
  a.act = d.act_dtype;
  a.sb = d.sb_dtype;
  a.out_dt = d.out_dtype;
  const int64_t T = c.T;
  const int rmax = d.inter > d.shared_inter ? d.inter : d.shared_inter;
  launch_kernel(k_sc_router, dim3(blocks_for(T * d.n_experts)), dim3(256), 0, c.stream, a);
  launch_kernel(k_sc_topk, dim3(blocks_for(T)), dim3(256), 0, c.stream, a);
  launch_kernel(k_sc_gateup, dim3(blocks_for(T * (d.top_k + 1) * rmax)), dim3(256), 0, c.stream, a);
  launch_kernel(k_sc_down, dim3(blocks_for(T * (d.top_k + 1) * d.hidden)), dim3(256), 0, c.stream, a);
  launch_kernel(k_sc_combine, dim3(blocks_for(T * d.hidden)), dim3(256), 0, c.stream, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // namespace moe
