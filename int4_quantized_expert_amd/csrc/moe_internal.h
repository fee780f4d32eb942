// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_layer.h"
#include "fused_common.h"

namespace moe {

constexpr int kFusedMaxBlocks = 2048;

// Sets the calling thread's moe_last_error() text and returns `code`;
// api_ok() clears it and returns MOE_OK.
int api_fail(int code, const char* msg);
int api_ok();
constexpr int kMaxExperts = 1024;   // largest n_experts a descriptor may have

// Byte layout of the caller's workspace for calls with up to T_max tokens.
// Every region starts on a 256-byte boundary.  The control words and the
// two-launch decode's tagged logits come first and have the same offsets for
// every T (sized for kFusedMaxT tokens), so that calls with different token
// counts on one workspace agree on the epoch counters and never read another
// region's bytes as a tagged word.
struct WsLayout {
  size_t ctrl;       // uint32 control words: [0] error flags, then the epoch counters
  size_t logits;     // [T, E] float32 router logits
  size_t ids;        // [T, k] int32 chosen experts
  size_t wts;        // [T, k] float32 renormalised weights
  size_t gate;       // [T] float32 sigmoid(g . x)
  size_t ucount;     // int32 number of distinct experts U
  size_t uniq;       // [min(T k, E)] int32 distinct experts, ascending id
  size_t ustart;     // [min(T k, E) + 1] int32 start of each expert's pair list
  size_t plist;      // [T k] int32 pair indices (t * k + i) grouped by expert
  size_t h;          // [T k + T, max(I, SI)] float32 SwiGLU activations
  size_t partial;    // [T k + T, H] per-pair down projections: float32 (decode), float16 (prefill)
  size_t f_lg;       // two-launch path: [kFusedReplicas][Tf, E] tagged logits (uint64), Tf = kFusedMaxT
  size_t f_uoff;     // two-launch path: [min(T k, E)] int64 blob offsets of the distinct experts
  size_t f_pidx;     // two-launch path: [min(T k, E), T] int32 rank of expert u for token t
  size_t f_epoch;    // two-launch path: [kFusedMaxBlocks] uint32 per-block call counters (inside ctrl)
  size_t f_gflag;    // single-launch decode: [kFusedReplicas][kFusedMaxBlocks] uint32 completion tags
  size_t s_lg;       // stack decode (either kernel): tagged words (logits, h, row sums)
  size_t s_x;        // stack decode: tagged next-layer input of each group
  size_t p_x16;      // prefill: [T, H] float16 activations in MFMA k order
  size_t p_meta;     // prefill: int32 [0] number of expert tiles
  size_t p_tstart;   // prefill: [min(T k, E) + 2] int32 first tile of each distinct expert, then of the shared one
  size_t p_tile;     // prefill: [max tiles] int32 distinct-expert rank of each tile (the shared expert is rank U)
  size_t p_estart;   // prefill: [E] int32 start of each expert's pair list
  size_t p_erank;    // prefill: [T k] int32 place of each pair in its expert's list (-1: unusable id)
  size_t total;
  int32_t umax;      // min(T k, E)
  int32_t hstride;   // max(I, SI)
  int32_t max_tiles; // bound on prefill tiles of up to kPrefillChunk tokens
};

constexpr int kPrefillChunk = 64;   // tokens per prefill tile
constexpr int kPrefillMinT = 16;    // fewest tokens that take the prefill path

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Stack decode (T = 1, one persistent launch for one or more layers): the
// shapes it is built for and the sizes of its exchange buffers.
bool stack_supported(const moe_desc& d);
size_t stack_ws_lg();
size_t stack_ws_x();

inline WsLayout ws_layout(const moe_desc& d, int32_t T) {
  WsLayout L{};
  const size_t Tk = static_cast<size_t>(T) * d.top_k;
  const int32_t umax = static_cast<int32_t>(Tk < static_cast<size_t>(d.n_experts) ? Tk : d.n_experts);
  const int32_t hs = d.inter > d.shared_inter ? d.inter : d.shared_inter;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes > 0 ? bytes : 1); return at; };
  L.ctrl = take(256 + static_cast<size_t>(kFusedMaxBlocks) * 4);
  // the stack decode's exchange words and flags: fixed offsets and sizes for
  // every descriptor and T, so that only its own tagged words (with older
  // tags) are ever found there
  L.s_lg = take(stack_ws_lg());
  L.s_x = take(stack_ws_x());
  L.f_epoch = L.ctrl + 256;
  const size_t Tf = kFusedMaxT;
  // sized for the largest E: words of other regions (plain data of calls with
  // another descriptor) never land where tagged words are looked for
  L.f_lg = take(static_cast<size_t>(kFusedReplicas) * Tf * kMaxExperts * 8);
  L.f_gflag = take(static_cast<size_t>(kFusedReplicas) * kFusedMaxBlocks * 4);
  L.logits = take(static_cast<size_t>(T) * d.n_experts * 4);
  L.ids = take(Tk * 4);
  L.wts = take(Tk * 4);
  L.gate = take(static_cast<size_t>(T) * 4);
  L.ucount = take(4);
  L.uniq = take(static_cast<size_t>(umax) * 4);
  L.ustart = take((static_cast<size_t>(umax) + 1) * 4);
  L.plist = take(Tk * 4);
  L.h = take((Tk + T) * static_cast<size_t>(hs) * 4);
  L.partial = take((Tk + T) * static_cast<size_t>(d.hidden) * 4);
  L.f_uoff = take(static_cast<size_t>(umax) * 8);
  L.f_pidx = take(static_cast<size_t>(umax) * T * 4);
  const size_t chunks = (Tk + kPrefillChunk - 1) / kPrefillChunk + (static_cast<size_t>(T) + kPrefillChunk - 1) / kPrefillChunk;
  L.max_tiles = static_cast<int32_t>(umax + chunks);
  L.p_x16 = take(static_cast<size_t>(T) * d.hidden * 2);
  L.p_meta = take(16);
  L.p_tstart = take((static_cast<size_t>(umax) + 2) * 4);
  L.p_tile = take(static_cast<size_t>(L.max_tiles) * 4);
  L.p_estart = take(static_cast<size_t>(d.n_experts) * 4);
  L.p_erank = take(Tk * 4);
  L.total = o;
  L.umax = umax;
  L.hstride = hs;
  return L;
}

// Per-call view of the inputs handed to the launchers.
struct Call {
  moe_desc d;
  int32_t T;
  const void* x;
  const void* router_w;
  const int64_t* slot_table;
  const uint8_t* pool;
  const uint8_t* shared;
  void* out;
  void* x_next;           // optional: x + out into the next layer's input (fp32 out only)
  uint8_t* ws;
  WsLayout L;
  const int32_t* ids;     // routing used by the expert kernels
  const float* wts;
  int32_t* ids_out;       // optional extra copies of the routing
  float* wts_out;
  hipStream_t stream;
};

// Takes the next pair of caller-supplied timing events (moe_set_launch_events)
// for the kernel about to launch; false when none is armed.
bool next_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of a forward call launches through here.  With timing events
// armed, the launch carries them (hipExtLaunchKernel), so the runtime stamps
// them with that dispatch's own start and end.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                          Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (next_launch_events(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0u, static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<KArgs>(args)...);
}

int launch_router_topk(const Call& c, int32_t* ids_dst, float* wts_dst);
int launch_experts(const Call& c);
// Pieces of the staged path the prefill path shares: per-token top-k of given
// logits, and the ordered combine of per-pair partial rows.
int launch_topk(const Call& c, const float* logits, int32_t* ids, float* wts, int32_t* ids2, float* wts2);
int launch_combine(const Call& c, const float* partial, const float* gate);      // fp32 partial rows
int launch_combine(const Call& c, const _Float16* partial, const float* gate);   // float16 partial rows
int launch_ws_init(uint8_t* ws, size_t bytes, hipStream_t stream);
// Scalar path: one thread per output value, the fast kernels' order of sums.
int launch_scalar(const Call& c);
int launch_take_flags(uint32_t* flags, uint32_t* status, hipStream_t stream);
int launch_residual(int act_dtype, const void* x, const float* y, void* x_next, int64_t n, hipStream_t stream);

// Prefill path (many tokens): MFMA router and grouped expert GEMMs.
bool prefill_supported(const moe_desc& d, int T);
int launch_prefill_router(const Call& c, int32_t* ids_dst, float* wts_dst);
int launch_prefill_experts(const Call& c);

// Stack decode: layer l reads x + l x_stride (or, when x_chain is set and
// l > 0, x_chain + (l - 1) chain_stride), router_w + l router_stride,
// slot_table + l slot_stride (bytes), shared + l shared_stride, and writes
// out + l out_stride and, when x_chain is set, x_chain + l chain_stride =
// its input + its output.
struct StackCall {
  moe_desc d;
  int32_t n_layers;
  int32_t T;              // tokens per layer (1: k_decode_stack, 2..8: k_decode_stack_t)
  const void* x;
  int64_t x_stride;
  const void* router_w;
  int64_t router_stride;
  const int64_t* slot_table;
  int64_t slot_stride;
  const uint8_t* pool;
  const uint8_t* shared;
  int64_t shared_stride;
  void* out;
  int64_t out_stride;
  void* x_chain;
  int64_t chain_stride;
  int32_t* ids_out;       // optional [n_layers][T][k]
  float* wts_out;
  uint8_t* ws;
  WsLayout L;
  hipStream_t stream;
};

struct StackPlan {
  int nb, rb, rpb, spb, gpb;
  size_t lds;
};

int stack_plan(const moe_desc& d, StackPlan* plan);
int launch_decode_stack(const StackCall& c, const StackPlan& plan);

// Stack decode of 2..8 tokens per layer (unchained): the same shapes, its
// exchange words in the same workspace region (tags grow across both kernels).
bool stack_t_supported(const moe_desc& d, int T);
size_t stack_t_ws_words();
int stack_t_plan(const moe_desc& d, StackPlan* plan);
int launch_decode_stack_t(const StackCall& c, const StackPlan& plan);

// Two-launch decode (T <= kFusedMaxT).
bool fused_supported(const moe_desc& d, int T);
int fused_plan(const moe_desc& d, int T, FusedPlan* plan);
int launch_decode_fused(const Call& c, const FusedPlan& plan);

}  // namespace moe
