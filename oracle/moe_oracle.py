"""Plain, slow CPU oracle for one sparse MoE layer with int4/int8 affine
group-quantized SwiGLU experts held as fixed-stride blobs.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP path: it has its own blob parser, its own bf16 decoding and its own
arithmetic, all in float64, written from the layer's definition below.

Sources.  The pages describe Swiftlet, an expert-streaming runtime:
  * "Swiftlet README translation" (news.paixiangai.cn), section "How it works"
    (工作原理): each layer routes every token to 10 of 512 experts (80B) or 8 of
    256 (35B); the dense core (router, shared expert, ...) stays resident; the
    routed experts are repacked as fixed-stride blobs so one fetch is one read,
    and hot experts live in a bounded slot pool.
  * same page, section "Relation to TurboFieldfare" (与 TurboFieldfare 的关系):
    MLX affine int4/int8 group quantization computed on the GPU with
    byte-addressed kernels and 64-bit offsets; a sparse MoE with a shared expert.
  * same page, section "Correctness" (正确性): Metal kernels are tested against
    an exact CPU reference; expert placement (cache or disk) never changes the
    answer.
  * "linlog.top article", section "Why MoE can stream" (MoE 架构为什么能流式加载):
    512 routed experts + 1 shared expert per layer, 10 selected per token.

The pages do not print the quantization formula, the packing order, the router
equation, the shared-expert gate or the expert nonlinearity.  The readings this
oracle takes (each also listed in the design notes) are:
  R1  affine dequantisation per 64-element group along the input axis:
      w[r, c] = s[r, c // 64] * q[r, c] + b[r, c // 64], q unsigned;
      int4: element c of a row sits in 32-bit little-endian word c // 8 at bits
      4*(c % 8) .. +3 (low nibble first); int8: word c // 4, bits 8*(c % 4).
  R2  router: logits l = R x (R row-major [E, H]); the k experts are the first
      k of all experts ordered by (-l, id), so ties go to the lower id and the
      ids come out in descending-logit order; weights are the softmax over all E
      experts renormalised over the chosen k, which equals
      p_i = exp(l_i - m) / sum_{j in S} exp(l_j - m).
  R3  expert: E(x) = Wd (silu(Wg x) * (Wu x)), silu(a) = a / (1 + exp(-a)).
  R4  layer: y = sum_i p_i E_{S_i}(x) + sigmoid(g . x) * E_shared(x), with g a
      dense gate vector of length H and the shared expert quantized like the
      routed ones.
  R5  blob layout (our own format; the pages give none): the nine planes
      gate_q, up_q, down_q, gate_s, up_s, down_s, gate_b, up_b, down_b back to
      back, matrices row-major [out, in] (gate/up [I, H], down [H, I]), the
      blob padded to a multiple of 4096 bytes to form the stride.  Expert e
      starts at byte slot_table[e] of the pool.  The shared-expert buffer holds
      one such blob (with the shared intermediate size) followed, at byte
      offset shared_stride, by the gate vector [H].
Dense data (x, router, gate vector) is float32 or bfloat16; scales and biases
are float32 or bfloat16.  All arithmetic here is float64 on the stored values.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64


@dataclass(frozen=True)
class LayerShape:
    """Shapes and storage types of one MoE layer (oracle's own description)."""

    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    bits: int = 4
    act_dtype: str = "bf16"   # x, router matrix, shared gate vector: "bf16" | "f32"
    sb_dtype: str = "bf16"    # quantization scales and biases: "bf16" | "f32"


def _dtype_size(name: str) -> int:
    return {"f32": 4, "bf16": 2}[name]


def decode_dense(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored float32 / bfloat16 values -> exact float64.

    A bfloat16 value is the upper half of a float32 bit pattern, so widening is
    exact: place the 16 stored bits above 16 zero bits and read a float32.
    """
    raw = np.ascontiguousarray(raw)
    if dtype == "f32":
        return raw.view(np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = raw.view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- blob format

def matrix_plane_bytes(rows: int, cols: int, bits: int) -> int:
    return rows * cols * bits // 8


def scale_plane_bytes(rows: int, cols: int, sb_dtype: str) -> int:
    return rows * (cols // GROUP) * _dtype_size(sb_dtype)


def blob_bytes(hidden: int, inter: int, bits: int, sb_dtype: str) -> int:
    """Unpadded size of one expert blob (reading R5)."""
    q = 2 * matrix_plane_bytes(inter, hidden, bits) + matrix_plane_bytes(hidden, inter, bits)
    s = 2 * scale_plane_bytes(inter, hidden, sb_dtype) + scale_plane_bytes(hidden, inter, sb_dtype)
    return q + 2 * s


def blob_stride(hidden: int, inter: int, bits: int, sb_dtype: str) -> int:
    """Fixed stride of the pool: the blob rounded up to 4096 bytes."""
    n = blob_bytes(hidden, inter, bits, sb_dtype)
    return (n + 4095) // 4096 * 4096


def unpack_q(words: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """Packed little-endian uint32 words -> unsigned codes q [rows, cols] (R1).

    int4: code c of a row is bits 4*(c % 8)..+3 of word c // 8 (low nibble
    first).  int8: bits 8*(c % 4)..+7 of word c // 4.
    """
    per_word = 32 // bits
    w = np.asarray(words, dtype=np.uint32).reshape(rows, cols // per_word)
    q = np.empty((rows, cols // per_word, per_word), dtype=np.uint8)
    mask = np.uint32((1 << bits) - 1)
    for j in range(per_word):
        q[:, :, j] = (w >> np.uint32(bits * j)) & mask
    return q.reshape(rows, cols)


def dequantize(q: np.ndarray, s: np.ndarray, b: np.ndarray) -> np.ndarray:
    """w[r, c] = s[r, c // 64] * q[r, c] + b[r, c // 64]  (R1), float64."""
    rows, cols = q.shape
    qg = q.reshape(rows, cols // GROUP, GROUP).astype(np.float64)
    return (s[:, :, None] * qg + b[:, :, None]).reshape(rows, cols)


def parse_blob(blob: np.ndarray, hidden: int, inter: int, bits: int, sb_dtype: str):
    """One expert blob (bytes) -> dequantized (Wg [I,H], Wu [I,H], Wd [H,I]) in float64.

    Plane order (R5): gate_q, up_q, down_q, gate_s, up_s, down_s, gate_b, up_b, down_b.
    """
    blob = np.ascontiguousarray(np.asarray(blob, dtype=np.uint8))
    shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
    off = 0
    qs = []
    for rows, cols in shapes:
        n = matrix_plane_bytes(rows, cols, bits)
        qs.append(unpack_q(blob[off:off + n].view(np.uint32), rows, cols, bits))
        off += n
    scales = []
    for rows, cols in shapes:
        n = scale_plane_bytes(rows, cols, sb_dtype)
        scales.append(decode_dense(blob[off:off + n], sb_dtype).reshape(rows, cols // GROUP))
        off += n
    biases = []
    for rows, cols in shapes:
        n = scale_plane_bytes(rows, cols, sb_dtype)
        biases.append(decode_dense(blob[off:off + n], sb_dtype).reshape(rows, cols // GROUP))
        off += n
    return tuple(dequantize(q, s, b) for q, s, b in zip(qs, scales, biases))


# ------------------------------------------------------------------ the layer

def router_logits(x: np.ndarray, router: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * R[e, h]  (R2), float64 matmul."""
    return x @ router.T


def select_topk(logits_row: np.ndarray, k: int) -> np.ndarray:
    """First k experts of the order (-logit, id): ties go to the lower id (R2)."""
    ids = np.arange(logits_row.shape[0])
    order = np.lexsort((ids, -logits_row))
    return order[:k].astype(np.int32)


def renormalised_weights(selected_logits: np.ndarray) -> np.ndarray:
    """Softmax over all experts renormalised over the chosen ones (R2).

    The full softmax denominator cancels, leaving exp(l_i - m) / sum_j exp(l_j - m)
    over the chosen logits, m their maximum.
    """
    m = np.max(selected_logits)
    e = np.exp(selected_logits - m)
    return e / np.sum(e)


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def expert_forward(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """SwiGLU expert (R3): Wd (silu(Wg x) * (Wu x))."""
    return wd @ (silu(wg @ x) * (wu @ x))


def _dense(buf, dtype, count):
    raw = np.ascontiguousarray(buf).view(np.uint8)
    return decode_dense(raw[: count * _dtype_size(dtype)], dtype)


def load_inputs(shape: LayerShape, T: int, x, router_w, shared_w):
    """Decode the dense inputs: x [T,H], router [E,H], gate vector [H] as float64."""
    H, E = shape.hidden, shape.n_experts
    xs = _dense(x, shape.act_dtype, T * H).reshape(T, H)
    rw = _dense(router_w, shape.act_dtype, E * H).reshape(E, H)
    sh_stride = blob_stride(H, shape.shared_inter, shape.bits, shape.sb_dtype)
    sh = np.ascontiguousarray(shared_w).view(np.uint8)
    gvec = decode_dense(sh[sh_stride: sh_stride + H * _dtype_size(shape.act_dtype)], shape.act_dtype)
    return xs, rw, gvec


def expert_blob(shape: LayerShape, pool: np.ndarray, slot_table: np.ndarray, e: int) -> np.ndarray:
    """The bytes of expert e: pool[slot_table[e] : slot_table[e] + blob size] (R5)."""
    pool = np.ascontiguousarray(pool).view(np.uint8)
    off = int(slot_table[e])
    n = blob_bytes(shape.hidden, shape.inter, shape.bits, shape.sb_dtype)
    if off < 0 or off + n > pool.nbytes:
        raise IndexError(f"expert {e}: slot offset {off} outside the pool")
    return pool[off: off + n]


def moe_layer(shape: LayerShape, T: int, x, router_w, slot_table, pool, shared_w,
              tokens=None):
    """Forward pass of one MoE layer (R1-R5), one token at a time, float64.

    Every chosen blob is parsed from its packed bytes on each use (no cached
    dequantized weights).  `tokens` optionally restricts the work to a subset of
    token indices (results for the others are left as NaN / -1).

    Returns (y [T, H] float64, topk_ids [T, k] int32, topk_w [T, k] float64,
             logits [T, E] float64).
    """
    H, k = shape.hidden, shape.top_k
    xs, rw, gvec = load_inputs(shape, T, x, router_w, shared_w)
    sh = np.ascontiguousarray(shared_w).view(np.uint8)
    sh_blob = sh[: blob_bytes(H, shape.shared_inter, shape.bits, shape.sb_dtype)]
    y = np.full((T, H), np.nan)
    ids = np.full((T, k), -1, dtype=np.int32)
    ws = np.full((T, k), np.nan)
    logits = router_logits(xs, rw)
    todo = range(T) if tokens is None else tokens
    for t in todo:
        xt = xs[t]
        sel = select_topk(logits[t], k)
        p = renormalised_weights(logits[t, sel])
        acc = np.zeros(H)
        for i, e in enumerate(sel):
            wg, wu, wd = parse_blob(expert_blob(shape, pool, slot_table, int(e)),
                                    H, shape.inter, shape.bits, shape.sb_dtype)
            acc += p[i] * expert_forward(wg, wu, wd, xt)
        wg, wu, wd = parse_blob(sh_blob, H, shape.shared_inter, shape.bits, shape.sb_dtype)
        acc += sigmoid(float(gvec @ xt)) * expert_forward(wg, wu, wd, xt)
        y[t], ids[t], ws[t] = acc, sel, p
    return y, ids, ws, logits


def moe_layer_dense(shape: LayerShape, T: int, x, router_w, slot_table, pool, shared_w):
    """Second formulation, for tiny shapes only: evaluate every expert densely.

    y = sum_e 1[e in S] * (softmax(l)_e / sum_{j in S} softmax(l)_j) * E_e(x)
        + sigmoid(g . x) * E_shared(x)
    with S the chosen set; the full softmax is formed explicitly and masked.
    """
    H, E, k = shape.hidden, shape.n_experts, shape.top_k
    xs, rw, gvec = load_inputs(shape, T, x, router_w, shared_w)
    sh = np.ascontiguousarray(shared_w).view(np.uint8)
    experts = [parse_blob(expert_blob(shape, pool, slot_table, e), H, shape.inter,
                          shape.bits, shape.sb_dtype) for e in range(E)]
    shared = parse_blob(sh[: blob_bytes(H, shape.shared_inter, shape.bits, shape.sb_dtype)],
                        H, shape.shared_inter, shape.bits, shape.sb_dtype)
    y = np.zeros((T, H))
    for t in range(T):
        xt = xs[t]
        l = rw @ xt
        full = np.exp(l - l.max())
        full /= full.sum()
        chosen = np.zeros(E, dtype=bool)
        chosen[select_topk(l, k)] = True
        mass = full[chosen].sum()
        outs = np.stack([expert_forward(*experts[e], xt) for e in range(E)])
        coef = np.where(chosen, full / mass, 0.0)
        y[t] = coef @ outs + sigmoid(float(gvec @ xt)) * expert_forward(*shared, xt)
    return y


def moe_layer_by_expert(shape: LayerShape, T: int, x, router_w, slot_table, pool, shared_w):
    """Third formulation, for many tokens: the routed sum taken expert by expert.

    y_t = sum_{e in S_t} p_{t,e} E_e(x_t) + sigmoid(g . x_t) E_shared(x_t) is the
    masked dense sum of moe_layer_dense with its zero terms skipped: every
    expert that some token chose is parsed once, applied to all the tokens
    that chose it (one float64 matrix product per matrix), and its weighted
    output added to those tokens' rows.  Routing (R2) is the same
    select_topk / renormalised_weights as the other formulations.  The
    additions into a row run in ascending expert id rather than rank order,
    which changes float64 rounding only.

    Returns (y [T, H] float64, topk_ids [T, k] int32, topk_w [T, k] float64).
    """
    H, k = shape.hidden, shape.top_k
    xs, rw, gvec = load_inputs(shape, T, x, router_w, shared_w)
    logits = router_logits(xs, rw)
    ids = np.stack([select_topk(logits[t], k) for t in range(T)]) if T else np.zeros((0, k), np.int32)
    w = np.stack([renormalised_weights(logits[t, ids[t]]) for t in range(T)]) if T else np.zeros((0, k))
    y = np.zeros((T, H))
    for e in np.unique(ids):
        tok, rank = np.nonzero(ids == e)
        wg, wu, wd = parse_blob(expert_blob(shape, pool, slot_table, int(e)), H, shape.inter, shape.bits,
                                shape.sb_dtype)
        xe = xs[tok].T                                      # [H, n]
        h = silu(wg @ xe) * (wu @ xe)                       # [I, n]
        y[tok] += (wd @ h).T * w[tok, rank][:, None]
    sh = np.ascontiguousarray(shared_w).view(np.uint8)
    wg, wu, wd = parse_blob(sh[: blob_bytes(H, shape.shared_inter, shape.bits, shape.sb_dtype)], H,
                            shape.shared_inter, shape.bits, shape.sb_dtype)
    xa = xs.T
    y += (wd @ (silu(wg @ xa) * (wu @ xa))).T * sigmoid(xs @ gvec)[:, None]
    return y, ids, w


def summation_bound(x_row: np.ndarray, router: np.ndarray, exact_products: bool) -> np.ndarray:
    """Worst-case float32 error of each logit under any summation order.

    With n terms whose products are exact in float32 (bf16 x bf16), any order of
    float32 additions errs by at most gamma_{n-1} * sum |x_h R_eh|, where
    gamma_m = m u / (1 - m u), u = 2^-24 (Higham, Accuracy and Stability of
    Numerical Algorithms, Lemma 3.1 / eq. 3.5).  When products are themselves
    rounded (float32 x float32), one more rounding per term gives gamma_n.
    x_row may also be a [T, H] batch of tokens; the result is then [T, E].
    """
    n = x_row.shape[-1]
    m = n if not exact_products else n - 1
    u = 2.0 ** -24
    gamma = m * u / (1.0 - m * u)
    return gamma * (np.abs(x_row) @ np.abs(router).T)


# ---------------------------------------------------------------- layer stack

def bf16_round_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even (NaN stays a
    quiet NaN); returns the 16-bit patterns.  Written from the definition:
    keep the top 16 bits, and add one unit of the kept part when the dropped
    16 bits exceed half a unit, or equal it and the kept part is odd."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi, lo = u >> 16, u & 0xFFFF
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    out = (hi + up.astype(np.uint64)) & 0xFFFF
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    out = np.where(nan, hi | 0x40, out)
    return out.astype(np.uint16)


def residual_next(x_raw: np.ndarray, y: np.ndarray, act_dtype: str) -> np.ndarray:
    """Input of the next layer in a stack: x + y, with y the layer's output.
    Reading (the pages run the whole layer stack per token but print no
    formula; plain residual chaining): the sum is taken in float32, the
    precision of the stored result, and rounded to nearest even for bf16
    activations, so that both paths take the same rounding decision.
    x_raw holds the stored activations (uint16 bf16 patterns or float32)."""
    x32 = decode_dense(x_raw, act_dtype).astype(np.float32)
    s = x32 + np.asarray(y, dtype=np.float32)
    if act_dtype == "bf16":
        return bf16_round_bits(s)
    return s.astype(np.float32)

