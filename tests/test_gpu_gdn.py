"""The gated-delta-rule recurrence on the GPU (gdn_recurrence_forward through
the C ABI) against the fp64 oracle, every output and every state element, to a
bound derived from the fp32 arithmetic (below); one call of T tokens against T
calls of one token, bit for bit (the pages check incremental decoding against
full-sequence processing: Swiftlet README translation, "Correctness").

Error bound.  u = 2^-24, g(m) = m u / (1 - m u), n = d_k.  Per token and row r
of S (the state before the token, exact), with k' and q' the normalised keys:
  k' and q' carry a relative error of at most e_k = g(n/2 + 5), e_q = g(n/2 + 6)
  (a length-n sum of squares, a square root, a division, a product);
  w = S_r . k' has error dw <= (g(n) + e_k) A_r,  A_r = sum_c |S_rc k'_c|;
  u_r = beta (v_r - alpha w) has error du <= beta alpha dw
        + g(3) beta (|v_r| + alpha |w| + alpha dw);
  the new row alpha S_r + u_r k'^T gains at most, in 2-norm,
        d_r = du + |u_r| e_k + g(2) (alpha ||S_r|| + |u_r|)      (||k'|| <= 1);
  an earlier error E is carried as alpha E (I - beta k' k'^T), whose rows do
  not grow (alpha <= 1, 0 <= beta <= 1), so E_t <= alpha E_{t-1} + d_t;
  the output o_r = S'_r . q' then has error <= E_t ||q'|| + (g(n) + e_q) sum_c |S'_rc q'_c|,
  plus half a bf16 unit (2^-9 |o_r|) when the output is stored as bf16.
The test asserts twice these first-order bounds (the factor covers the second-
order terms the derivation drops)."""

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from oracle import gdn_oracle as G
from synth.gdn import GDN_PRESETS, gdn_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


def g(m):
    return m * U / (1 - m * U)


class Case:
    def __init__(self, n_k_heads, n_v_heads, d_k, d_v, B, T, seed, act="bf16", out="f32", alpha=None, beta=None,
                 zero_k=False):
        nk, nv, dk, dv = n_k_heads, n_v_heads, d_k, d_v
        self.shape = G.GdnShape(nk, nv, dk, dv, dk ** -0.5, 1e-6)
        self.desc = M.gdn_desc(nk, nv, dk, dv, act=act, out=out)
        self.B, self.T, self.act, self.out = B, T, act, out
        q, k, v, al, be, st = gdn_inputs(nk, nv, dk, dv, B, T, seed, act)
        if alpha is not None:
            al[...] = alpha
        if beta is not None:
            be[...] = beta
        if zero_k:
            k[...] = 0
        self.raw = (q, k, v, al, be, st)
        self.vals = tuple(synth.act_values(a, act).astype(np.float64) for a in (q, k, v)) + (
            al.astype(np.float64), be.astype(np.float64), st.astype(np.float64))

    def device(self):
        q, k, v, al, be, st = self.raw
        put = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        odt = torch.float32 if self.out == "f32" else torch.bfloat16
        out = torch.full((self.B, self.T, self.shape.n_v_heads, self.shape.d_v), float("nan"), dtype=odt, device=DEV)
        return put(q), put(k), put(v), put(al), put(be), put(st), out


def run_gpu(c: Case, split=None):
    """One call over all T tokens, or consecutive calls of the token counts in `split`."""
    q, k, v, al, be, st, out = c.device()
    if split is None:
        M.gdn_forward(c.desc, c.B, c.T, q, k, v, al, be, st, out)
    else:
        t0 = 0
        for n in split:
            sl = slice(t0, t0 + n)
            o = torch.empty_like(out[:, sl]).contiguous()
            M.gdn_forward(c.desc, c.B, n, q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                          al[:, sl].contiguous(), be[:, sl].contiguous(), st, o)
            out[:, sl] = o
            t0 += n
        assert t0 == c.T
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64)


def oracle_with_bounds(c: Case):
    """Oracle outputs and state, with the derived per-element bounds."""
    sh = c.shape
    q, k, v, al, be, S = c.vals
    B, T, nv, dv, dk = c.B, c.T, sh.n_v_heads, sh.d_v, sh.d_k
    e_k, e_q, gn = g(dk / 2 + 5), g(dk / 2 + 6), g(dk)
    outs = np.zeros((B, T, nv, dv))
    obnd = np.zeros((B, T, nv, dv))
    E = np.zeros((B, nv, dv))
    S = S.copy()
    for t in range(T):
        o_t, S_new = G.gdn_recurrence(sh, q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], al[:, t:t + 1],
                                      be[:, t:t + 1], S)
        outs[:, t] = o_t[:, 0]
        kh = np.array([G.key_head(sh, h) for h in range(nv)])
        kn = G.l2_normalize(k[:, t][:, kh], sh.eps)                     # [B, nv, dk]
        qn = sh.scale * G.l2_normalize(q[:, t][:, kh], sh.eps)
        a = al[:, t][:, :, None]
        b = be[:, t][:, :, None]
        A = np.einsum("bhrc,bhc->bhr", np.abs(S), np.abs(kn))
        w = np.einsum("bhrc,bhc->bhr", S, kn)
        dw = (gn + e_k) * A
        u = b * (v[:, t] - a * w)
        du = b * a * dw + g(3) * b * (np.abs(v[:, t]) + a * np.abs(w) + a * dw)
        d = du + np.abs(u) * e_k + g(2) * (a * np.linalg.norm(S, axis=3) + np.abs(u))
        E = a * E + d
        Bq = np.einsum("bhrc,bhc->bhr", np.abs(S_new), np.abs(qn))
        ob = E * np.linalg.norm(qn, axis=2)[:, :, None] + (gn + e_q) * Bq
        if c.out == "bf16":
            ob = ob + 2.0 ** -9 * np.abs(o_t[:, 0])
        obnd[:, t] = ob
        S = S_new
    return outs, S, obnd, E


def check(c: Case, split=None):
    o_ref, s_ref, ob, E = oracle_with_bounds(c)
    o, s = run_gpu(c, split)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    err_o = np.abs(o - o_ref)
    err_s = np.abs(s - s_ref)
    assert np.all(err_o <= 2 * ob), f"output: worst err/bound {np.max(err_o / (2 * ob)):.3f}"
    assert np.all(err_s <= 2 * E[..., None]), f"state: worst err/bound {np.max(err_s / (2 * E[..., None])):.3f}"
    return o, s, np.max(err_o / (2 * ob))


@pytest.mark.parametrize("name,kw", [
    ("tiny-f32", dict(**GDN_PRESETS["tiny"], B=3, T=5, seed=1, act="f32")),
    ("tiny-bf16-out", dict(**GDN_PRESETS["tiny"], B=2, T=4, seed=2, act="bf16", out="bf16")),
    ("80b-B4-T4", dict(**GDN_PRESETS["80b"], B=4, T=4, seed=3)),
    ("80b-B8-T2-bf16-out", dict(**GDN_PRESETS["80b"], B=8, T=2, seed=4, out="bf16")),
    ("dk128-dv256", dict(n_k_heads=1, n_v_heads=2, d_k=128, d_v=256, B=2, T=3, seed=5)),
    ("dk64-dv48-ragged", dict(n_k_heads=3, n_v_heads=6, d_k=64, d_v=48, B=5, T=3, seed=6, act="f32")),
])
def test_matches_oracle_within_derived_bound(name, kw):
    check(Case(**kw))


@pytest.mark.parametrize("B", [1, 8, 64])
def test_decode_step_at_the_benchmark_sizes(B):
    """One token for B sequences of the 80B-shaped layer (B = 1: a single
    stream; B = 64: the batched figure), every element against the oracle."""
    check(Case(**GDN_PRESETS["80b"], B=B, T=1, seed=10 + B))


def test_one_call_of_T_tokens_equals_T_calls_bitwise():
    c = Case(**GDN_PRESETS["80b"], B=2, T=16, seed=20)
    o_full, s_full = run_gpu(c)
    o_inc, s_inc = run_gpu(c, split=[1] * 16)
    o_mix, s_mix = run_gpu(c, split=[5, 8, 3])
    assert np.array_equal(o_full, o_inc) and np.array_equal(s_full, s_inc)
    assert np.array_equal(o_full, o_mix) and np.array_equal(s_full, s_mix)
    check(c)


@pytest.mark.parametrize("name,kw", [
    ("reset-alpha0", dict(alpha=0.0)),
    ("no-write-beta0", dict(beta=0.0)),
    ("full-write", dict(alpha=1.0, beta=1.0)),
    ("zero-key", dict(zero_k=True)),
])
def test_degenerate_gates_and_keys(name, kw):
    check(Case(**GDN_PRESETS["tiny"], B=2, T=3, seed=30, act="f32", **kw))


def test_long_sequence_in_one_call():
    """T = 256 tokens in one call: the bound grows with T and still holds."""
    check(Case(n_k_heads=1, n_v_heads=2, d_k=128, d_v=128, B=1, T=256, seed=40))


def test_zero_batch_or_tokens_leave_the_state_alone():
    c = Case(**GDN_PRESETS["tiny"], B=2, T=2, seed=50)
    q, k, v, al, be, st, out = c.device()
    before = st.clone()
    M.gdn_forward(c.desc, 0, 2, q, k, v, al, be, st, out)
    M.gdn_forward(c.desc, 2, 0, q, k, v, al, be, st, out)
    torch.cuda.synchronize()
    assert torch.equal(st, before)
