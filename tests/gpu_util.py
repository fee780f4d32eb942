"""Helpers for the GPU parity tests: seeded layer inputs, device upload, the
HIP call through the binding, the oracle beside it and the tolerance checks.

Inputs come from synth (shared by both sides); expected values come only from
the oracle.  Tokens are margin-filtered with the oracle so that top-k ids are
unambiguous under any float32 summation order (see oracle.summation_bound).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import int4_quantized_expert_amd as M
import synth
from oracle import moe_oracle as O

DEV = torch.device("cuda:0")


@dataclass
class LayerData:
    geo: synth.Geometry
    x: np.ndarray        # raw activations [T, H]
    R: np.ndarray        # raw router [E, H]
    pool: np.ndarray     # uint8 pool (host); see device_fill
    slots: np.ndarray    # int64 [E]
    shared: np.ndarray   # uint8 shared buffer
    seed: int = 0
    layer: int = 0
    device_fill: bool = False   # device pool made by the device generator; the
                                # host pool then holds only the blobs the oracle reads

    @property
    def T(self):
        return self.x.shape[0]


def oracle_shape(geo: synth.Geometry) -> O.LayerShape:
    return O.LayerShape(geo.hidden, geo.n_experts, geo.top_k, geo.inter, geo.shared_inter, geo.bits, geo.act,
                        geo.sb)


def unambiguous(geo: synth.Geometry, x_raw: np.ndarray, R_raw: np.ndarray, margin_scale: float = 1.0) -> np.ndarray:
    """Per token: True if every adjacent gap among the top k+1 logits exceeds
    margin_scale times the sum of both experts' worst-case float32 summation
    errors (2 for logits summed on MFMA, whose internal rounding is not
    specified as round-to-nearest per addition)."""
    shape = oracle_shape(geo)
    xs = O.decode_dense(x_raw, geo.act).reshape(-1, geo.hidden)
    rs = O.decode_dense(R_raw, geo.act).reshape(geo.n_experts, geo.hidden)
    k = min(shape.top_k + 1, geo.n_experts)
    if k < 2:
        return np.ones(xs.shape[0], dtype=bool)
    logits = O.router_logits(xs, rs)
    bound = O.summation_bound(xs, rs, exact_products=(geo.act == "bf16"))
    # a stable sort of -logit keeps lower ids first among equal logits, the oracle's order
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(logits, order, 1)
    b = np.take_along_axis(bound, order, 1)
    return np.all(top[:, :-1] - top[:, 1:] > margin_scale * (b[:, :-1] + b[:, 1:]), axis=1)


HOST_POOL_LIMIT = 64 << 20


def make_layer(geo: synth.Geometry, seed: int, layer: int, T: int, routing: str = "normal",
               n_cand: int | None = None, filter_margin: bool = True, margin_scale: float = 1.0,
               oracle_tokens=None) -> LayerData:
    """Seeded layer inputs.  Pools above 64 MiB are generated on the device by
    the counter-based generator (bit-identical to the host one, which a test
    checks); the host copy then only holds the blobs of the experts that the
    oracle's own routing of these tokens (or of oracle_tokens only) selects."""
    n_cand = n_cand or max(4 * T, 16)
    cand = synth.tokens(geo, seed, layer, n_cand)
    if routing == "zipf":
        R = synth.router_zipf(geo, seed, layer, cand)
    else:
        R = synth.router_normal(geo, seed, layer)
    if filter_margin:
        ok = unambiguous(geo, cand, R, margin_scale)
        idx = np.nonzero(ok)[0]
        assert idx.size >= T, f"only {idx.size} of {n_cand} candidate tokens have unambiguous routing"
        x = cand[idx[:T]]
    else:
        x = cand[:T]
    shared = synth.make_shared(geo, seed, layer)
    stride = geo.blob_stride
    if geo.n_experts * stride <= HOST_POOL_LIMIT:
        pool, slots = synth.make_pool(geo, seed, layer)
        return LayerData(geo, np.ascontiguousarray(x), R, pool, slots, shared, seed, layer, False)
    slots = np.arange(geo.n_experts, dtype=np.int64) * stride
    pool = np.zeros(geo.n_experts * stride, dtype=np.uint8)
    xs = O.decode_dense(x, geo.act).reshape(-1, geo.hidden)
    rs = O.decode_dense(R, geo.act).reshape(geo.n_experts, geo.hidden)
    logits = O.router_logits(xs, rs)
    rows = range(xs.shape[0]) if oracle_tokens is None else oracle_tokens
    needed = sorted({int(e) for t in rows for e in O.select_topk(logits[t], geo.top_k)})
    for e in needed:
        synth.fill_blob(geo, geo.inter, synth.blob_key(seed, layer, e), pool[e * stride:(e + 1) * stride])
    return LayerData(geo, np.ascontiguousarray(x), R, pool, slots, shared, seed, layer, True)


def put(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(DEV)


@dataclass
class DeviceLayer:
    desc: M.MoeDesc
    x: torch.Tensor
    R: torch.Tensor
    pool: torch.Tensor
    slots: torch.Tensor
    shared: torch.Tensor


def upload(data: LayerData, out: str = "f32", pool=None, slots=None) -> DeviceLayer:
    g = data.geo
    if pool is not None:
        pool_d = pool
    elif data.device_fill:
        from synth import gpu
        pool_d = torch.empty(g.n_experts * g.blob_stride, dtype=torch.uint8, device=DEV)
        gpu.fill_blobs(g, pool_d.data_ptr(), g.n_experts, data.seed, data.layer, 0,
                       stream=torch.cuda.current_stream().cuda_stream)
    else:
        pool_d = put(data.pool)
    slots_d = torch.from_numpy(np.asarray(data.slots if slots is None else slots, dtype=np.int64)).to(DEV)
    d = M.desc_for(g.hidden, g.n_experts, g.top_k, g.inter, g.shared_inter, g.bits, g.act, g.sb, out,
                   pool_bytes=pool_d.numel())
    return DeviceLayer(d, put(data.x), put(data.R), pool_d, slots_d, put(data.shared))


def run(dl: DeviceLayer, T: int, x: torch.Tensor | None = None, ws: torch.Tensor | None = None,
        staged: bool = False):
    """moe_layer_forward (or the staged variant) through the binding; returns (out tensor, ids, wts)."""
    g_out = torch.float32 if dl.desc.out_dtype == M.MOE_F32 else torch.bfloat16
    H, k = dl.desc.hidden, dl.desc.top_k
    out = torch.full((max(T, 1), H), float("nan"), dtype=g_out, device=DEV)
    ids = torch.full((max(T, 1), k), -7, dtype=torch.int32, device=DEV)
    wts = torch.full((max(T, 1), k), float("nan"), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = torch.zeros(M.workspace_bytes(dl.desc, max(T, 1)), dtype=torch.uint8, device=DEV)
        M.workspace_init(ws)
    fwd = M.layer_forward_staged if staged else M.layer_forward
    fwd(dl.desc, T, dl.x if x is None else x, dl.R, dl.slots, dl.pool, dl.shared, out, ws, ids, wts)
    torch.cuda.synchronize()
    M.status_check(ws)
    return out, ids, wts


def oracle_routing(data: LayerData):
    """The oracle's ids and renormalised weights for every token (cheap: no experts)."""
    g = data.geo
    xs = O.decode_dense(data.x, g.act).reshape(-1, g.hidden)
    rs = O.decode_dense(data.R, g.act).reshape(g.n_experts, g.hidden)
    logits = O.router_logits(xs, rs)
    ids = np.stack([O.select_topk(logits[t], g.top_k) for t in range(xs.shape[0])])
    w = np.stack([O.renormalised_weights(logits[t, ids[t]]) for t in range(xs.shape[0])])
    return ids, w


def oracle_run(data: LayerData, tokens=None):
    return O.moe_layer(oracle_shape(data.geo), data.T, data.x, data.R, data.slots, data.pool, data.shared,
                       tokens=tokens)


def oracle_run_all(data: LayerData):
    """Every token of the batch through the oracle's expert-major formulation
    (each chosen blob parsed once for all the tokens that chose it): fast
    enough for thousands of tokens.  Returns (y, ids, w)."""
    return O.moe_layer_by_expert(oracle_shape(data.geo), data.T, data.x, data.R, data.slots, data.pool,
                                 data.shared)


def relocate(dl: DeviceLayer, data: LayerData, seed: int = 0):
    """The same blobs in one pool of more than 4 GiB at a permuted placement:
    every odd expert above byte offset 2^32 (offsets that do not fit 32 bits),
    every even one below it.  Returns (big pool, slot table), ready for
    upload(data, pool=..., slots=...)."""
    g = data.geo
    stride = g.blob_stride
    E = g.n_experts
    n_lo, n_hi = (E + 1) // 2, E // 2
    base = (1 << 32) + 3 * 256
    big = torch.zeros(base + (n_hi + 1) * stride, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(seed)
    lo_perm, hi_perm = rng.permutation(n_lo + 1)[:n_lo], rng.permutation(n_hi + 1)[:n_hi]
    slots = np.empty(E, dtype=np.int64)
    src = np.asarray(data.slots, dtype=np.int64)
    for e in range(E):
        off = base + int(hi_perm[e // 2]) * stride if e % 2 else int(lo_perm[e // 2]) * stride
        slots[e] = off
        big[off: off + stride] = dl.pool[int(src[e]): int(src[e]) + stride]
    torch.cuda.synchronize()
    assert slots.max() > (1 << 32) and slots.min() < (1 << 32)
    return big, slots


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1e-38)))
    return np.where(a > 0, 2.0 ** (e - 8), 2.0 ** -134)


def check_close(y_gpu: torch.Tensor, y_ref: np.ndarray, act: str, tokens=None) -> float:
    """max|y - y_ref| <= tol * max|y_ref| (+ half a bf16 ulp per element for a
    bf16 output).  tol = 1e-5 for float32 activations, 2e-3 for bfloat16."""
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        y, y_ref = y[tokens], y_ref[tokens]
    tol = 1e-5 if act == "f32" else 2e-3
    scale = np.max(np.abs(y_ref))
    err = np.abs(y - y_ref)
    allow = tol * scale
    if y_gpu.dtype == torch.bfloat16:
        allow = allow + bf16_half_ulp(y_ref)
    assert np.all(np.isfinite(y)), "non-finite output"
    assert np.all(err <= allow), f"max err {err.max():.3e} vs scale {scale:.3e} (tol {tol})"
    return float(err.max() / scale)


def check_routing(ids: torch.Tensor, wts: torch.Tensor, ids_ref: np.ndarray, w_ref: np.ndarray, tokens=None):
    i = ids.cpu().numpy()
    w = wts.cpu().numpy().astype(np.float64)
    if tokens is not None:
        i, w, ids_ref, w_ref = i[tokens], w[tokens], ids_ref[tokens], w_ref[tokens]
    np.testing.assert_array_equal(i, ids_ref)
    # p in float32 from float32 logits: the logit error is tiny against the
    # enforced gaps, exp/divide add a few ulp
    assert np.max(np.abs(w - w_ref)) <= 1e-4, f"weights differ by {np.max(np.abs(w - w_ref)):.3e}"
