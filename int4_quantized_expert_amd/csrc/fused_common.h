// Arguments and launch plan of the two-launch decode path.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kFusedMaxT = 8;       // tokens per call handled by the two-launch decode path
constexpr int kFusedReplicas = 16;  // copies of the exchanged logits and flags

struct FusedArgs {
  const void* x;
  const void* router;
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  void* out;
  void* x_next;         // optional [T, H] activations: x + out (stack step), out fp32
  int32_t* ids_out;     // optional [T, k]
  float* wts_out;       // optional [T, k]
  uint64_t* lg;         // [kFusedReplicas][T, E] tagged logits
  float* h;             // [T k + T, hs] SwiGLU activations
  float* wts;           // [T, k] renormalised weights (routing record)
  float* sig;           // [T] sigmoid(g . x)
  int32_t* ucount;      // number of distinct experts U
  int32_t* uniq;        // [umax] distinct experts, ascending id
  int64_t* uoff;        // [umax] their blob offsets
  int32_t* pidx;        // [umax, T] rank of expert u for token t, or -1
  uint32_t* ctrl;       // [0] error flags
  uint32_t* epochs;     // [kFusedMaxBlocks] per-block call counters (tag = counter + 1)
  uint32_t* gflags;     // [kFusedReplicas][kFusedMaxBlocks] single launch: tag of each block whose h is written
  size_t lds_b_off;     // single launch: where the down-phase LDS starts
  size_t lds_d_off;     // single launch: where the prefetched down operands start
  int d_slots;          // single launch: down task slots per wave
  int64_t pool_bytes;
  int64_t shared_stride;
  int T, H, E, k, I, SI, hs;
  int nb;               // launch A blocks (all resident)
  int rb;               // launch B output rows per block
  int nslice;           // launch B row slices (blocks: nslice * T)
  int umax;             // min(T k, E)
  int act_sz;
  uint32_t spin_limit;
};

struct FusedPlan {
  int nb;       // launch A grid
  size_t lds;   // launch A dynamic LDS
  int umax;
  int nb_b;     // launch B grid
  int rb_b;     // launch B rows per block
  int nslice;   // launch B row slices
  size_t lds_b; // launch B dynamic LDS
  bool one;     // T = 1 in a single launch (the down phase runs in launch A's blocks)
  size_t lds_one;
  int d_slots;  // single launch: down task slots per wave (operands prefetched into LDS)
};

}  // namespace moe
