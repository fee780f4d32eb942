"""Pins for the CPU oracle: hand-worked values, closed forms, invariants and
brute force, each chosen so that a plausible slip in the oracle (wrong nibble
order, transposed matrix, wrong group axis, dropped shared term, sign error in
the gate, wrong renormalisation, wrong tie order) fails at least one test.

Sources of the facts pinned: the Swiftlet README translation (sections "How it
works", "Correctness", "Relation to TurboFieldfare") and the linlog.top article
(section "Why MoE can stream"); formulas the pages leave open follow the
oracle's stated readings R1-R5.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import synth
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- test-side packing
# Independent of the oracle's parser: the packing written out from the format text.

def pack_rows(q, bits):
    """Codes q [rows, cols] -> little-endian uint32 words, low code first."""
    rows, cols = q.shape
    per = 32 // bits
    words = np.zeros((rows, cols // per), dtype=np.uint64)
    for c in range(cols):
        words[:, c // per] |= (q[:, c].astype(np.uint64) << np.uint64(bits * (c % per)))
    return words.astype(np.uint32)


def build_blob(H, I, bits, q3, s3, b3, sb="f32"):
    """Blob bytes from codes/scales/biases of gate [I,H], up [I,H], down [H,I]."""
    parts = [pack_rows(q, bits).tobytes() for q in q3]
    dt = np.float32 if sb == "f32" else None
    for arrs in (s3, b3):
        for a in arrs:
            if sb == "f32":
                parts.append(np.asarray(a, dtype=dt).tobytes())
            else:
                parts.append(synth.bf16_bits(np.asarray(a, dtype=np.float32)).tobytes())
    raw = b"".join(parts)
    stride = (len(raw) + 4095) // 4096 * 4096
    out = np.zeros(stride, dtype=np.uint8)
    out[: len(raw)] = np.frombuffer(raw, dtype=np.uint8)
    return out


def shared_buffer(blob, gate, act="f32"):
    g = np.asarray(gate, dtype=np.float32)
    graw = g.tobytes() if act == "f32" else synth.bf16_bits(g).tobytes()
    out = np.zeros(blob.nbytes + len(graw), dtype=np.uint8)
    out[: blob.nbytes] = blob
    out[blob.nbytes:] = np.frombuffer(graw, dtype=np.uint8)
    return out


def const_blob(H, I, c, bits=4):
    """Blob whose every weight equals c: q = 9 everywhere, s = 1/64, b = c - 9/64."""
    q3 = [np.full((I, H), 9), np.full((I, H), 9), np.full((H, I), 9)]
    s3 = [np.full((I, H // 64), 1 / 64), np.full((I, H // 64), 1 / 64), np.full((H, I // 64), 1 / 64)]
    b3 = [np.full(s.shape, c - 9 / 64) for s in s3]
    return build_blob(H, I, bits, q3, s3, b3)


# ----------------------------------------------------------------- hand-worked unpack

def test_unpack_int4_hand_worked():
    for ex in golden("unpack_examples.json")["int4"]:
        word = np.array([int(ex["word"], 16)], dtype=np.uint32)
        q = O.unpack_q(word, 1, 8, 4)[0]
        assert list(q) == ex["q"]
        # one group needs 64 codes: repeat the word 8 times
        q64 = O.unpack_q(np.repeat(word, 8), 1, 64, 4)
        w = O.dequantize(q64, np.array([[ex["s"]]]), np.array([[ex["b"]]]))[0, :8]
        assert list(w) == ex["w"]


def test_unpack_int8_hand_worked():
    for ex in golden("unpack_examples.json")["int8"]:
        word = np.array([int(ex["word"], 16)], dtype=np.uint32)
        q = O.unpack_q(word, 1, 4, 8)[0]
        assert list(q) == ex["q"]
        q64 = O.unpack_q(np.repeat(word, 16), 1, 64, 8)
        w = O.dequantize(q64, np.array([[ex["s"]]]), np.array([[ex["b"]]]))[0, :4]
        assert list(w) == ex["w"]


def test_bf16_decode_hand_worked():
    for ex in golden("unpack_examples.json")["bf16"]:
        raw = np.array([int(ex["bits"], 16)], dtype=np.uint16)
        assert O.decode_dense(raw, "bf16")[0] == ex["value"]


# ----------------------------------------------------------------- layout pins

@pytest.mark.parametrize("bits,sb", [(4, "f32"), (8, "f32"), (4, "bf16")])
def test_blob_layout_orientation_and_groups(bits, sb):
    """Every plane, orientation and group axis is recovered element by element."""
    H, I = 192, 128
    m = (1 << bits) - 1
    r_i, c_h = np.meshgrid(np.arange(I), np.arange(H), indexing="ij")
    r_h, c_i = np.meshgrid(np.arange(H), np.arange(I), indexing="ij")
    qg = (3 * r_i + 5 * c_h) % (m + 1)
    qu = (r_i + 7 * c_h + 1) % (m + 1)
    qd = (2 * r_h + c_i + 3) % (m + 1)

    def sgrid(rows, groups, k):
        r, g = np.meshgrid(np.arange(rows), np.arange(groups), indexing="ij")
        return 2.0 ** -(1 + (r + 2 * g + k) % 5)

    sg, su, sd = sgrid(I, H // 64, 0), sgrid(I, H // 64, 1), sgrid(H, I // 64, 2)
    bg, bu, bd = -sg * 3, -su * 5, -sd * 7
    blob = build_blob(H, I, bits, [qg, qu, qd], [sg, su, sd], [bg, bu, bd], sb)
    assert blob.nbytes == O.blob_stride(H, I, bits, sb)
    assert O.blob_bytes(H, I, bits, sb) == (3 * H * I * bits // 8
                                            + 6 * H * I // 64 * (4 if sb == "f32" else 2))
    wg, wu, wd = O.parse_blob(blob, H, I, bits, sb)
    for w, q, s, b in ((wg, qg, sg, bg), (wu, qu, su, bu), (wd, qd, sd, bd)):
        rows, cols = q.shape
        expect = np.empty((rows, cols))
        for r in range(rows):
            for c in range(cols):
                expect[r, c] = s[r, c // 64] * q[r, c] + b[r, c // 64]
        np.testing.assert_array_equal(w, expect)


def test_blob_sizes_of_named_shapes():
    """Blob and stride sizes of the three layer shapes (hand arithmetic)."""
    # int4, H=2048, I=512, bf16 s/b: 3 * (524288 + 2*32768) = 1769472 = 432 * 4096
    assert O.blob_bytes(2048, 512, 4, "bf16") == 1769472
    assert O.blob_stride(2048, 512, 4, "bf16") == 1769472
    # int8: 3 * (1048576 + 2*32768) = 3342336 = 816 * 4096
    assert O.blob_bytes(2048, 512, 8, "bf16") == 3342336
    # tiny: H=256, I=128, fp32 s/b: 3 * (16384 + 2*2048) = 61440
    assert O.blob_bytes(256, 128, 4, "f32") == 61440


# ----------------------------------------------------------------- router pins

def test_router_orientation_one_hot():
    """x = e_j gives logits = column j of R [E, H]."""
    E, H = 5, 64
    R = (np.arange(E * H).reshape(E, H) % 13 - 6).astype(np.float64) / 8
    for j in (0, 17, 63):
        x = np.zeros((1, H))
        x[0, j] = 1.0
        np.testing.assert_array_equal(O.router_logits(x, R)[0], R[:, j])


def test_topk_order_and_ties():
    l = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 0.5, 3.0])
    assert list(O.select_topk(l, 4)) == [6, 1, 2, 4]
    assert list(O.select_topk(l, 6)) == [6, 1, 2, 4, 0, 5]
    assert list(O.select_topk(l, 1)) == [6]


def test_renormalisation_closed_form():
    g = golden("closed_forms.json")["renormalisation"]
    p = O.renormalised_weights(np.array(g["selected_logits"]))
    np.testing.assert_allclose(p, g["p"], rtol=0, atol=1e-16)
    assert abs(p.sum() - 1.0) < 1e-15


def test_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(3)
    l = rng.standard_normal(12) * 3
    ids = O.select_topk(l, 12)
    p = O.renormalised_weights(l[ids])
    np.testing.assert_allclose(p, softmax(l)[ids], rtol=1e-14, atol=0)
    assert list(ids) == list(np.argsort(-l, kind="stable"))


def test_renormalised_equals_masked_full_softmax():
    rng = np.random.default_rng(4)
    l = rng.standard_normal(40) * 2
    ids = O.select_topk(l, 7)
    full = softmax(l)
    np.testing.assert_allclose(O.renormalised_weights(l[ids]), full[ids] / full[ids].sum(),
                               rtol=1e-14, atol=0)


# ----------------------------------------------------------------- layer closed forms

def test_uniform_layer_closed_form():
    c = golden("closed_forms.json")["uniform_layer"]
    sh = c["shape"]
    H, I, E = sh["hidden"], sh["inter"], sh["n_experts"]
    shape = O.LayerShape(H, E, sh["top_k"], I, sh["shared_inter"], 4, "f32", "f32")
    blob = const_blob(H, I, 1 / 64)
    pool = np.concatenate([blob] * E)
    slots = np.arange(E, dtype=np.int64) * blob.nbytes
    shared = shared_buffer(blob, np.zeros(H))
    x = np.ones((1, H), dtype=np.float32)
    R = np.zeros((E, H), dtype=np.float32)
    y, ids, w, _ = O.moe_layer(shape, 1, x, R, slots, pool, shared)
    np.testing.assert_allclose(y[0], c["y_each"], rtol=1e-15, atol=0)
    assert list(ids[0]) == [0]          # exact tie between the two experts -> lower id
    assert w[0, 0] == 1.0


def test_zero_experts_leave_only_shared():
    """q = 8 and b = -8s give zero routed experts, so y = sigmoid(g.x) * S(x)."""
    H, I, E, k = 128, 64, 4, 2
    shape = O.LayerShape(H, E, k, I, I, 4, "f32", "f32")
    z3 = [np.full((I, H), 8), np.full((I, H), 8), np.full((H, I), 8)]
    s3 = [np.full((I, H // 64), 0.01), np.full((I, H // 64), 0.02), np.full((H, I // 64), 0.03)]
    b3 = [-8 * s for s in s3]
    zero = build_blob(H, I, 4, z3, s3, b3)
    shared_blob = const_blob(H, I, 1 / 128)
    rng = np.random.default_rng(5)
    gate = (rng.standard_normal(H) * 0.05).astype(np.float32)
    shared = shared_buffer(shared_blob, gate)
    pool = np.concatenate([zero] * E)
    slots = np.arange(E, dtype=np.int64) * zero.nbytes
    x = rng.standard_normal((3, H)).astype(np.float32)
    R = rng.standard_normal((E, H)).astype(np.float32)
    y, _, _, _ = O.moe_layer(shape, 3, x, R, slots, pool, shared)
    for t in range(3):
        S = float(np.sum(x[t].astype(np.float64)))
        c = 1 / 128
        f = c * I * (c * S / (1 + math.exp(-c * S))) * (c * S)
        gx = float(gate.astype(np.float64) @ x[t].astype(np.float64))
        np.testing.assert_allclose(y[t], f / (1 + math.exp(-gx)), rtol=1e-12, atol=0)


def test_constant_experts_closed_form():
    """Experts with constant weights c_e give E_e(x) = c I silu(cS) cS per output.

    x = a * e_j with dyadic a and router column so that logits are exact; the
    whole layer is then a closed form in exp().
    """
    H, I, E, k = 64, 64, 6, 3
    shape = O.LayerShape(H, E, k, I, I, 4, "f32", "f32")
    consts = [(e + 1) / 64 for e in range(E)]
    pool = np.concatenate([const_blob(H, I, c) for c in consts])
    stride = pool.nbytes // E
    slots = np.arange(E, dtype=np.int64) * stride
    c_sh = 3 / 128
    j, a = 5, 1.5
    gate = np.zeros(H, dtype=np.float32)
    gate[j] = -0.75
    shared = shared_buffer(const_blob(H, I, c_sh), gate)
    R = np.zeros((E, H), dtype=np.float32)
    col = np.array([0.25, 1.0, -0.5, 0.75, 1.0, 0.125], dtype=np.float32)
    R[:, j] = col
    x = np.zeros((1, H), dtype=np.float32)
    x[0, j] = a
    y, ids, w, _ = O.moe_layer(shape, 1, x, R, slots, pool, shared)
    logits = col.astype(np.float64) * a          # exact: (0.375, 1.5, -0.75, 1.125, 1.5, 0.1875)
    sel = [1, 4, 3]                               # 1.5 (id 1), 1.5 (id 4, tie -> after 1), 1.125
    assert list(ids[0]) == sel
    ex = [math.exp(logits[e] - 1.5) for e in sel]
    p = [v / sum(ex) for v in ex]
    np.testing.assert_allclose(w[0], p, rtol=1e-15)

    def f(c):
        s = c * a
        return c * I * (s / (1 + math.exp(-s))) * s

    expect = sum(pi * f(consts[e]) for pi, e in zip(p, sel))
    expect += f(c_sh) / (1 + math.exp(-(-0.75 * a)))
    np.testing.assert_allclose(y[0], expect, rtol=1e-14, atol=0)


def test_identical_experts_routed_part_is_expert():
    """All routed experts identical: the routed sum is E(x) for any routing (sum p = 1)."""
    g = synth.PRESETS["tiny"]
    shape = O.LayerShape(g.hidden, g.n_experts, g.top_k, g.inter, g.shared_inter, 4, "f32", "f32")
    blob = synth.fill_blob(g, g.inter, synth.blob_key(7, 0, 0))
    pool = np.concatenate([blob] * g.n_experts)
    slots = np.arange(g.n_experts, dtype=np.int64) * blob.nbytes
    shared = synth.make_shared(g, 7, 0)
    zero_gate = shared.copy()
    zero_gate[g.shared_stride:] = 0          # sigmoid(0) = 1/2 exactly
    x = synth.tokens(g, 7, 0, 3)
    R = synth.router_normal(g, 7, 0)
    y, _, _, _ = O.moe_layer(shape, 3, x, R, slots, pool, zero_gate)
    wg, wu, wd = O.parse_blob(blob, g.hidden, g.inter, 4, "f32")
    sg, su, sd = O.parse_blob(shared[: g.shared_stride], g.hidden, g.shared_inter, 4, "f32")
    for t in range(3):
        xt = x[t].astype(np.float64)
        e = wd @ (O.silu(wg @ xt) * (wu @ xt))
        s = sd @ (O.silu(sg @ xt) * (su @ xt))
        np.testing.assert_allclose(y[t], e + 0.5 * s, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- brute force

@pytest.mark.parametrize("preset,E,k,bits", [("tiny", 16, 2, 4), ("tiny", 8, 8, 4),
                                              ("tiny", 12, 1, 8), ("tiny", 16, 5, 4)])
def test_routed_loop_matches_dense_masked(preset, E, k, bits):
    base = synth.PRESETS[preset]
    g = synth.Geometry(base.hidden, E, k, base.inter, base.shared_inter, bits, "f32", "f32")
    shape = O.LayerShape(g.hidden, E, k, g.inter, g.shared_inter, bits, "f32", "f32")
    pool, slots = synth.make_pool(g, 11, 2)
    shared = synth.make_shared(g, 11, 2)
    x = synth.tokens(g, 11, 2, 4)
    R = synth.router_normal(g, 11, 2)
    y, _, _, _ = O.moe_layer(shape, 4, x, R, slots, pool, shared)
    yd = O.moe_layer_dense(shape, 4, x, R, slots, pool, shared)
    assert np.max(np.abs(y - yd)) <= 1e-12 * np.max(np.abs(y))


@pytest.mark.parametrize("E,k,bits,sb,T", [(16, 2, 4, "f32", 6), (12, 3, 8, "bf16", 9), (16, 16, 4, "bf16", 3)])
def test_expert_major_matches_token_loop_and_dense(E, k, bits, sb, T):
    """The expert-by-expert formulation (used for whole-batch checks of many
    tokens) agrees with the per-token loop and the dense masked sum."""
    base = synth.PRESETS["tiny"]
    g = synth.Geometry(base.hidden, E, k, base.inter, 2 * base.shared_inter, bits, "f32", sb)
    shape = O.LayerShape(g.hidden, E, k, g.inter, g.shared_inter, bits, "f32", sb)
    pool, slots = synth.make_pool(g, 31, 1)
    slots = slots[::-1].copy()                      # a permuted placement
    shared = synth.make_shared(g, 31, 1)
    x = synth.tokens(g, 31, 1, T)
    R = synth.router_normal(g, 31, 1)
    y, ids, w, _ = O.moe_layer(shape, T, x, R, slots, pool, shared)
    yb, idb, wb = O.moe_layer_by_expert(shape, T, x, R, slots, pool, shared)
    yd = O.moe_layer_dense(shape, T, x, R, slots, pool, shared)
    np.testing.assert_array_equal(ids, idb)
    np.testing.assert_allclose(wb, w, rtol=0, atol=1e-15)
    assert np.max(np.abs(yb - y)) <= 1e-12 * np.max(np.abs(y))
    assert np.max(np.abs(yb - yd)) <= 1e-12 * np.max(np.abs(y))


def test_gemv_core_against_scalar_loop():
    """Dequantized matvec vs a scalar loop over the packed words (64 x 64)."""
    rng = np.random.default_rng(8)
    H = I = 64
    q3 = [rng.integers(0, 16, (I, H)), rng.integers(0, 16, (I, H)), rng.integers(0, 16, (H, I))]
    s3 = [rng.uniform(0.002, 0.02, (I, 1)), rng.uniform(0.002, 0.02, (I, 1)), rng.uniform(0.002, 0.02, (H, 1))]
    b3 = [-8 * s for s in s3]
    blob = build_blob(H, I, 4, q3, s3, b3)
    wg, _, _ = O.parse_blob(blob, H, I, 4, "f32")
    x = rng.standard_normal(H)
    words = blob[: H * I // 2].view(np.uint32)
    sv = blob[3 * H * I // 2: 3 * H * I // 2 + 4 * I].view(np.float32)
    bv = blob[3 * H * I // 2 + 12 * I: 3 * H * I // 2 + 16 * I].view(np.float32)
    for r in range(I):
        acc = 0.0
        for c in range(H):
            word = int(words[r * (H // 8) + c // 8])
            qv = (word >> (4 * (c % 8))) & 15
            acc += (float(sv[r]) * qv + float(bv[r])) * float(x[c])
        assert abs(acc - float(wg[r] @ x)) <= 1e-12 * (1 + abs(acc))


# ----------------------------------------------------------------- invariants

def test_placement_invariance_in_oracle():
    """Any slot placement of the same blobs gives the same output (pages: the
    answer is identical whether an expert comes from cache or disk)."""
    g = synth.PRESETS["tiny"]
    shape = O.LayerShape(g.hidden, g.n_experts, g.top_k, g.inter, g.shared_inter, 4, "f32", "f32")
    pool, slots = synth.make_pool(g, 13, 0)
    shared = synth.make_shared(g, 13, 0)
    x = synth.tokens(g, 13, 0, 4)
    R = synth.router_normal(g, 13, 0)
    y0, i0, w0, _ = O.moe_layer(shape, 4, x, R, slots, pool, shared)
    stride = g.blob_stride
    perm = np.random.default_rng(1).permutation(g.n_experts + 3)[: g.n_experts]
    pool2 = np.zeros((g.n_experts + 3) * stride, dtype=np.uint8)
    slots2 = perm.astype(np.int64) * stride
    for e in range(g.n_experts):
        pool2[slots2[e]: slots2[e] + stride] = pool[slots[e]: slots[e] + stride]
    y1, i1, w1, _ = O.moe_layer(shape, 4, x, R, slots2, pool2, shared)
    np.testing.assert_array_equal(y0, y1)
    np.testing.assert_array_equal(i0, i1)


def test_summation_bound_holds_float32():
    """The stated float32 error bound covers sequential and pairwise float32 sums."""
    rng = np.random.default_rng(9)
    g = synth.PRESETS["80b"]
    x = synth.act_values(synth.tokens(g, 1, 0, 1), "bf16")[0]
    R = synth.act_values(synth.router_normal(g, 1, 0), "bf16")[:8]
    exact = R.astype(np.float64) @ x.astype(np.float64)
    bound = O.summation_bound(x.astype(np.float64), R.astype(np.float64), True)
    prod = (R * x[None, :]).astype(np.float32)
    seq = np.zeros(8, dtype=np.float32)
    for h in rng.permutation(x.shape[0]):
        seq = (seq + prod[:, h]).astype(np.float32)
    pair = prod.sum(axis=1, dtype=np.float32)
    assert np.all(np.abs(seq - exact) <= bound)
    assert np.all(np.abs(pair - exact) <= bound)


def test_summation_bound_fixed_values_and_attained():
    """Hand-worked values of the bound, and a sum whose float32 error reaches it.

    x = (1, -2, 0.5), rows (1, 1, 1) and (2, 0, -4): sum |x_h R_eh| = 3.5 and 4.
    With exact products n - 1 = 2 additions, so the bound is gamma_2 times
    that, gamma_m = m 2^-24 / (1 - m 2^-24); with rounded products, gamma_3.
    Summing (1, 2^-24, 2^-24) left to right in float32 rounds both additions
    back to 1 (ties to even), an error of exactly 2^-23, while the bound is
    gamma_2 (1 + 2^-23) = 2^-23 (1 + 2^-23) / (1 - 2^-23): a bound one
    notch smaller (gamma_1, or u / 2 per addition) would not cover it."""
    u = 2.0 ** -24
    g2, g3 = 2 * u / (1 - 2 * u), 3 * u / (1 - 3 * u)
    x = np.array([1.0, -2.0, 0.5])
    R = np.array([[1.0, 1.0, 1.0], [2.0, 0.0, -4.0]])
    assert np.array_equal(O.summation_bound(x, R, True), np.array([g2 * 3.5, g2 * 4.0]))
    assert np.array_equal(O.summation_bound(x, R, False), np.array([g3 * 3.5, g3 * 4.0]))
    terms = np.array([1.0, u, u])
    s = np.float32(0.0)
    for v in terms.astype(np.float32):
        s = np.float32(s + v)
    err = abs(float(s) - terms.sum())
    assert err == 2.0 ** -23
    bound = float(O.summation_bound(np.ones(3), terms[None, :], True)[0])
    assert err <= bound < err * (1 + 2.0 ** -21)
    assert err > (u / (1 - u)) * terms.sum()        # gamma_1 would be too small


def test_splitmix64_published_outputs():
    c = golden("closed_forms.json")["splitmix64_seed0"]
    got = [int(v) for v in synth.stream(0, 0, 4)]
    assert got == [int(v, 16) for v in c["outputs"]]
