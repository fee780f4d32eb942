// Arguments and launch plan of the fused decode kernel.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kFusedMaxT = 8;   // tokens per call handled by the fused decode kernel

struct FusedArgs {
  const void* x;
  const void* router;
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  void* out;
  int32_t* ids_out;     // optional [T, k]
  float* wts_out;       // optional [T, k]
  uint64_t* lg;         // [T, E] tagged logits
  uint64_t* hx;         // [T k + T, hs] tagged SwiGLU activations
  uint32_t* ctrl;       // [0] error flags, [1] epoch
  uint32_t* flag_r;     // [nb] per-block "phase R stores done" tags
  uint32_t* flag_g;     // [nb] per-block "phase G stores done" tags
  int64_t pool_bytes;
  int64_t shared_stride;
  int T, H, E, k, I, SI, hs;
  int nb;               // blocks (all resident)
  int rb;               // output rows per block
  int umax;             // min(T k, E)
  int act_sz;
  uint32_t spin_limit;
};

struct FusedPlan {
  int nb;
  int rb;
  int umax;
  size_t lds;
};

}  // namespace moe
