/*
 * gdn_recurrence.h - C ABI of the gated-delta-rule decode recurrence (gfx950).
 *
 * The fixed-size recurrent state of a Gated DeltaNet layer, advanced one token
 * at a time.  Sources:
 *   - linlog.top article, section "Four core designs", design 4 (Gated DeltaNet
 *     linear attention): three quarters of the Qwen3-Next layers use Gated
 *     DeltaNet, which keeps a state matrix of fixed dimensions updated per
 *     token by a gated delta rule instead of a growing KV cache (a method from
 *     NVIDIA and MIT research).
 *   - Swiftlet README translation, section "How it works", closing paragraph:
 *     the same fixed-size state at any context length.
 *   - same page, section "Correctness": incremental decoding is checked against
 *     processing the full sequence (here: T tokens in one call equal T calls of
 *     one token, bit for bit).
 *
 * The pages name the rule but print no equation.  This library computes the
 * rule as its authors publish it (Gated Delta Networks, Yang, Kautz and
 * Hatamizadeh), per sequence b, token t and value head h, with kh = h / (n_v /
 * n_k) the query/key head that h reads and S = state[b][h] of shape [d_v, d_k]:
 *   k' = k / sqrt(sum k^2 + eps)        q' = scale * q / sqrt(sum q^2 + eps)
 *   S  <- alpha S (I - beta k' k'^T) + beta v k'^T
 *   out = S q'                          (with the updated S)
 * evaluated as S <- alpha S + u k'^T with u = beta (v - alpha (S k')), which is
 * the same expression expanded, every row of S on its own.
 *
 * Conventions as in moe_layer.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t, NULL = null stream), MOE_OK or a
 * negative MOE_E* code with the reason in moe_last_error(), every argument
 * checked before anything is enqueued, deterministic results.
 */
#ifndef GDN_RECURRENCE_H
#define GDN_RECURRENCE_H

#include <stdint.h>

#include "moe_layer.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_desc {
  int32_t n_k_heads;  /* query/key heads, >= 1                                  */
  int32_t n_v_heads;  /* value heads: a multiple of n_k_heads, at most 1024     */
  int32_t d_k;        /* key width: 64 or 128                                   */
  int32_t d_v;        /* value width: a multiple of 16 in [16, 256]             */
  int32_t act_dtype;  /* q, k, v: MOE_F32 or MOE_BF16                          */
  int32_t out_dtype;  /* out: MOE_F32 or MOE_BF16 (round to nearest even)      */
  float scale;        /* factor on the normalised q (finite)                    */
  float eps;          /* added under the square root of both norms (>= 0)      */
} gdn_desc;

/* Advance B independent sequences by T tokens each.
 *   q, k   [B][T][n_k_heads][d_k]   act_dtype, 16-byte aligned
 *   v      [B][T][n_v_heads][d_v]   act_dtype, 16-byte aligned
 *   alpha  [B][T][n_v_heads] fp32   the gate (decay) of each token and head
 *   beta   [B][T][n_v_heads] fp32   the write strength
 *   state  [B][n_v_heads][d_v][d_k] fp32, read and replaced in place
 *   out    [B][T][n_v_heads][d_v]   out_dtype
 * The tokens of a sequence are applied in order inside the call; the state
 * stays on chip between them, so one call with T tokens gives the same bits
 * as T calls with one token each.  B = 0 or T = 0 enqueues nothing.
 * Errors: MOE_EINVAL for a bad descriptor, negative or too large B or T, a
 * NULL or misaligned pointer, or a state or out buffer that overlaps another
 * argument; MOE_EHIP if the launch fails. */
int gdn_recurrence_forward(const gdn_desc* d, int32_t B, int32_t T, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, float* state, void* out,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_RECURRENCE_H */
