"""Seeded synthetic inputs for the MoE layer: tokens, router matrices, gate
vectors and packed expert blobs.

This module only draws numbers and lays them out in the storage format; it
computes nothing the layer computes.  Both the CPU oracle's callers and the HIP
path's callers take their inputs from here, so the two sides see the same bytes.

Blob contents come from a counter-based generator so that a device-side fill
(synth/csrc/synth_fill.hip) can produce the same bytes in place for pools of
tens of gigabytes: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), read as a counter-based stream:
output i of the stream with key K is mix64(K + (i + 1) * 0x9E3779B97F4A7C15),
mix64(z) = z3 with z1 = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9,
z2 = (z1 ^ (z1 >> 27)) * 0x94D049BB133111EB, z3 = z2 ^ (z2 >> 31)  (mod 2^64).

Value recipe (the pages give none; these are the synthetic workloads' recipe):
  q     uniform codes: every packed 32-bit word is a uniform random word.
  s     U(0.002, 0.02) for int4, U(0.002, 0.02) / 16 for int8, formed in float32
        as 0.002f + 0.018f * u with u = (r >> 40) * 2^-24, then rounded to the
        scale dtype (bf16: round to nearest even).
  b     -8 s (int4) or -128 s (int8), exact in either dtype, so q is centred.
  x     N(0, 1); router N(0, 0.05) or Zipf(1.1)-skewed (router_zipf); gate
        vector N(0, 0.05); all drawn in float32 by numpy PCG64 and rounded to
        the activation dtype.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GROUP = 64
GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
SHARED_BLOB_ID = 0xFFFFF


@dataclass(frozen=True)
class Geometry:
    """Layer geometry used by the generators (kept separate from both paths)."""

    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    bits: int = 4
    act: str = "bf16"
    sb: str = "bf16"

    @property
    def act_size(self) -> int:
        return 4 if self.act == "f32" else 2

    @property
    def sb_size(self) -> int:
        return 4 if self.sb == "f32" else 2

    def planes(self, inter: int):
        """(q bytes, s bytes) of the gate, up and down matrices for intermediate `inter`."""
        H = self.hidden
        shapes = [(inter, H), (inter, H), (H, inter)]
        q = [r * c * self.bits // 8 for r, c in shapes]
        s = [r * (c // GROUP) * self.sb_size for r, c in shapes]
        return q, s

    def blob_bytes(self, inter: int) -> int:
        q, s = self.planes(inter)
        return sum(q) + 2 * sum(s)

    def stride(self, inter: int) -> int:
        return (self.blob_bytes(inter) + 4095) // 4096 * 4096

    @property
    def blob_stride(self) -> int:
        return self.stride(self.inter)

    @property
    def shared_stride(self) -> int:
        return self.stride(self.shared_inter)

    @property
    def shared_bytes(self) -> int:
        """Shared buffer: blob padded to its stride, then the gate vector [H]."""
        n = self.shared_stride + self.hidden * self.act_size
        return (n + 255) // 256 * 256


PRESETS = {
    # Tiny layer: fp32 activations and scales.
    "tiny": Geometry(hidden=256, n_experts=16, top_k=2, inter=128, shared_inter=128,
                     bits=4, act="f32", sb="f32"),
    # 35B-A3B-shaped decode layer.
    "35b": Geometry(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512),
    # 80B-A3B-shaped layer (decode and prefill).
    "80b": Geometry(hidden=2048, n_experts=512, top_k=10, inter=512, shared_inter=512),
    # 35B-A3B shape with int8 experts.
    "35b_int8": Geometry(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512,
                         bits=8),
}


# ------------------------------------------------------------ counter-based RNG

def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def stream(key: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the SplitMix64 stream with key `key`."""
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + (idx + np.uint64(1)) * GAMMA)


def blob_key(seed: int, layer: int, blob_id: int) -> int:
    """Key of one blob's stream: mix64((seed << 40) ^ (layer << 20) ^ blob_id)."""
    assert 0 <= seed < (1 << 24) and 0 <= layer < (1 << 20) and 0 <= blob_id <= SHARED_BLOB_ID
    z = np.uint64((seed << 40) ^ (layer << 20) ^ blob_id)
    return int(mix64(z))


def scale_key(key: int) -> int:
    """Key of the scale sub-stream of a blob: mix64(key ^ 1)."""
    return int(mix64(np.uint64(key ^ 1)))


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_act(f32: np.ndarray, act: str) -> np.ndarray:
    """Round float32 draws to the activation storage dtype (raw array)."""
    if act == "f32":
        return np.ascontiguousarray(f32, dtype=np.float32)
    return bf16_bits(f32)


def act_values(raw: np.ndarray, act: str) -> np.ndarray:
    """Stored activation values as float32 (exact)."""
    if act == "f32":
        return np.asarray(raw, dtype=np.float32)
    return bf16_to_f32(raw)


# ----------------------------------------------------------------- blobs

def fill_blob(geo: Geometry, inter: int, key: int, out: np.ndarray | None = None) -> np.ndarray:
    """Bytes of one blob (padded to its stride) from the counter-based stream."""
    stride = geo.stride(inter)
    if out is None:
        out = np.zeros(stride, dtype=np.uint8)
    else:
        out[:] = 0
    q, s = geo.planes(inter)
    nq_words = sum(q) // 4
    r = stream(key, 0, (nq_words + 1) // 2)
    words = np.empty(2 * r.shape[0], dtype=np.uint32)
    words[0::2] = (r & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    words[1::2] = (r >> np.uint64(32)).astype(np.uint32)
    out[: sum(q)] = words[:nq_words].view(np.uint8)
    ns = sum(s) // geo.sb_size
    u = (stream(scale_key(key), 0, ns) >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    s32 = np.float32(0.018) * u
    s32 = (s32 + np.float32(0.002)).astype(np.float32)
    if geo.bits == 8:
        s32 = (s32 * np.float32(0.0625)).astype(np.float32)
    centre = np.float32(-8.0 if geo.bits == 4 else -128.0)
    if geo.sb == "bf16":
        sbits = bf16_bits(s32)
        bbits = bf16_bits(bf16_to_f32(sbits) * centre)
        sraw, braw = sbits.view(np.uint8), bbits.view(np.uint8)
    else:
        sraw = s32.view(np.uint8)
        braw = (s32 * centre).astype(np.float32).view(np.uint8)
    o = sum(q)
    out[o: o + sum(s)] = sraw
    out[o + sum(s): o + 2 * sum(s)] = braw
    return out


def make_pool(geo: Geometry, seed: int, layer: int, n_blobs: int | None = None):
    """Pool of n_blobs expert blobs (default all experts) at identity placement.

    Returns (pool uint8 [n_blobs * stride], slot_table int64 [E]) where
    slot_table[e] = e * stride.
    """
    n = geo.n_experts if n_blobs is None else n_blobs
    stride = geo.blob_stride
    pool = np.zeros(n * stride, dtype=np.uint8)
    for e in range(n):
        fill_blob(geo, geo.inter, blob_key(seed, layer, e), pool[e * stride:(e + 1) * stride])
    slots = np.arange(geo.n_experts, dtype=np.int64) * stride
    return pool, slots


def make_shared(geo: Geometry, seed: int, layer: int) -> np.ndarray:
    """Shared-expert buffer: blob padded to shared_stride, then the gate vector [H]."""
    buf = np.zeros(geo.shared_bytes, dtype=np.uint8)
    fill_blob(geo, geo.shared_inter, blob_key(seed, layer, SHARED_BLOB_ID), buf[: geo.shared_stride])
    rng = np.random.Generator(np.random.PCG64([seed, layer, 0x6A7E]))
    g = (rng.standard_normal(geo.hidden, dtype=np.float32) * np.float32(0.05)).astype(np.float32)
    raw = to_act(g, geo.act)
    buf[geo.shared_stride: geo.shared_stride + raw.nbytes] = raw.view(np.uint8)
    return buf


# --------------------------------------------------------- dense activations

def tokens(geo: Geometry, seed: int, layer: int, T: int, stream_id: int = 0, std: float = 1.0) -> np.ndarray:
    """x [T, H] ~ N(0, std^2), raw activation storage."""
    rng = np.random.Generator(np.random.PCG64([seed, layer, 0x70C5, stream_id]))
    x = rng.standard_normal((T, geo.hidden), dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return to_act(x, geo.act)


def router_normal(geo: Geometry, seed: int, layer: int, std: float = 0.05) -> np.ndarray:
    """Router [E, H] ~ N(0, std), raw activation storage."""
    rng = np.random.Generator(np.random.PCG64([seed, layer, 0x2007]))
    r = rng.standard_normal((geo.n_experts, geo.hidden), dtype=np.float32) * np.float32(std)
    return to_act(r.astype(np.float32), geo.act)


def zipf_target_logits(geo: Geometry, seed: int, layer: int, n_tokens: int, alpha: float = 1.1):
    """Target logits z [n_tokens, E] whose top-k is a Zipf(alpha) sample.

    A per-layer random permutation maps popularity rank to expert id; each
    token's targets are log p_rank + Gumbel(0, 1) noise, whose top-k is a sample
    without replacement from the Zipf law (Gumbel-top-k: W. Kool, H. van Hoof,
    M. Welling, "Stochastic Beams and Where to Find Them", ICML 2019).
    """
    rng = np.random.Generator(np.random.PCG64([seed, layer, 0x21BF]))
    E = geo.n_experts
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logp = -alpha * np.log(ranks)
    logp -= np.log(np.exp(logp).sum())
    perm = rng.permutation(E)                  # perm[rank] = expert id
    base = np.empty(E)
    base[perm] = logp
    gumbel = -np.log(-np.log(rng.uniform(1e-300, 1.0, size=(n_tokens, E))))
    return base[None, :] + gumbel, perm


def router_zipf(geo: Geometry, seed: int, layer: int, x_raw: np.ndarray, alpha: float = 1.1,
                std: float = 0.05) -> np.ndarray:
    """Router [E, H] whose logits on the given tokens follow Zipf(alpha) popularity.

    R = R0 + (Z - R0 X)(X^T X)^{-1} X^T with X = [H, N] the stored tokens as
    columns, Z the target logits (zipf_target_logits) and R0 ~ N(0, std); then
    R is rounded to the activation dtype.  Routing is whatever the stored R and
    x give; the construction only skews it.  Needs N <= H.
    """
    X = act_values(x_raw, geo.act).astype(np.float64).reshape(-1, geo.hidden).T   # [H, N]
    N = X.shape[1]
    assert N <= geo.hidden, "Zipf router construction needs at most H tokens"
    Z, _ = zipf_target_logits(geo, seed, layer, N, alpha)
    rng = np.random.Generator(np.random.PCG64([seed, layer, 0x2008]))
    R0 = rng.standard_normal((geo.n_experts, geo.hidden)) * std
    G = X.T @ X
    C = np.linalg.solve(G, (Z.T - R0 @ X).T).T     # [E, N]
    R = R0 + C @ X.T
    return to_act(R.astype(np.float32), geo.act)
