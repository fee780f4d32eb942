// Device-side fill of synthetic expert blobs, the same bytes as
// synth.fill_blob() on the host: SplitMix64 read as a counter-based stream
// (G. Steele, D. Lea, C. Flood, OOPSLA 2014), output i of the stream with key K
// being mix64(K + (i + 1) * 0x9E3779B97F4A7C15).  Used to build pools of tens of
// gigabytes in place; holds no part of the MoE layer's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline uint64_t stream_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGamma); }

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

struct FillArgs {
  uint8_t* dst;
  int64_t stride;
  int64_t q_bytes;     // all code planes of one blob
  int64_t s_count;     // scale entries of one blob (all three planes)
  int64_t blob_bytes;
  uint64_t seed, layer;
  uint32_t blob_id0;
  int n_blobs, bits, sb_f32;
};

__global__ void k_fill_codes(FillArgs a) {
  const int b = blockIdx.y;
  const uint64_t key = mix64((a.seed << 40) ^ (a.layer << 20) ^ (uint64_t)(a.blob_id0 + b));
  const int64_t n64 = a.q_bytes / 8;
  uint64_t* out = reinterpret_cast<uint64_t*>(a.dst + b * a.stride);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n64; i += (int64_t)gridDim.x * blockDim.x) {
    out[i] = stream_at(key, (uint64_t)i);   // little-endian: low word first, as on the host
  }
}

__global__ void k_fill_scales(FillArgs a) {
  const int b = blockIdx.y;
  const uint64_t key = mix64((a.seed << 40) ^ (a.layer << 20) ^ (uint64_t)(a.blob_id0 + b));
  const uint64_t skey = mix64(key ^ 1ull);
  uint8_t* base = a.dst + b * a.stride + a.q_bytes;
  const float centre = a.bits == 4 ? -8.0f : -128.0f;
  for (int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; m < a.s_count; m += (int64_t)gridDim.x * blockDim.x) {
    const float u = static_cast<float>(static_cast<uint32_t>(stream_at(skey, (uint64_t)m) >> 40)) * 5.9604644775390625e-08f;
    float s = __fadd_rn(__fmul_rn(0.018f, u), 0.002f);
    if (a.bits == 8) s = __fmul_rn(s, 0.0625f);
    if (a.sb_f32) {
      reinterpret_cast<float*>(base)[m] = s;
      reinterpret_cast<float*>(base)[a.s_count + m] = __fmul_rn(s, centre);
    } else {
      const uint16_t sb = bf16_rne(s);
      reinterpret_cast<uint16_t*>(base)[m] = sb;
      reinterpret_cast<uint16_t*>(base)[a.s_count + m] = bf16_rne(__uint_as_float((uint32_t)sb << 16) * centre);
    }
  }
}

__global__ void k_zero_tail(FillArgs a) {
  const int b = blockIdx.y;
  uint8_t* p = a.dst + b * a.stride;
  for (int64_t i = a.blob_bytes + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.stride;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

extern "C" {

// Fill n_blobs blobs at dst, dst + stride, ... with the synthetic recipe for
// blob ids blob_id0, blob_id0 + 1, ...  Returns 0 or -1 (bad argument) / -3 (launch).
int synth_fill_blobs(void* dst, int64_t stride, int32_t n_blobs, int32_t hidden, int32_t inter, int32_t bits,
                     int32_t sb_f32, uint32_t seed, uint32_t layer, uint32_t blob_id0, void* stream) {
  if (!dst || n_blobs < 0 || n_blobs > 65535 || hidden <= 0 || inter <= 0 || hidden % 64 || inter % 64 ||
      (bits != 4 && bits != 8) || seed >= (1u << 24) || layer >= (1u << 20))
    return -1;
  if (n_blobs == 0) return 0;
  FillArgs a;
  a.dst = static_cast<uint8_t*>(dst);
  a.stride = stride;
  a.q_bytes = 3ll * hidden * inter * bits / 8;
  a.s_count = 3ll * hidden * (inter / 64);
  a.blob_bytes = a.q_bytes + 2 * a.s_count * (sb_f32 ? 4 : 2);
  if (stride < a.blob_bytes || a.q_bytes % 8) return -1;
  a.seed = seed;
  a.layer = layer;
  a.blob_id0 = blob_id0;
  a.n_blobs = n_blobs;
  a.bits = bits;
  a.sb_f32 = sb_f32 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(k_fill_codes, dim3(64, n_blobs), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_fill_scales, dim3(16, n_blobs), dim3(256), 0, s, a);
  if (stride > a.blob_bytes) hipLaunchKernelGGL(k_zero_tail, dim3(4, n_blobs), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
