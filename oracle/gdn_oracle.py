"""Plain, slow CPU oracle for the gated delta rule: the fixed-size recurrent
state that Gated DeltaNet layers carry from token to token at decode time.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP path and computes in float64 on the stored input values.

Sources.
  * "linlog.top article", section "Four core designs" (Swiftlet 的四个核心设计),
    design 4 (Gated DeltaNet linear attention): three quarters of the layers
    of the Qwen3-Next models replace self-attention with Gated DeltaNet, which
    keeps a state matrix of fixed dimensions and updates it incrementally for
    every token with a gated delta rule, so no KV cache grows with the context;
    the method comes from NVIDIA and MIT research.
  * "Swiftlet README translation" (news.paixiangai.cn), section "How it works"
    (工作原理), closing paragraph: the DeltaNet layers hold a fixed-size
    recurrent state at any context length.
  * same page, section "Correctness" (正确性): incremental decoding is checked
    against processing the full sequence.

The pages name the rule but print no equation and no sizes.  The readings taken
here (each also listed in the design notes):
  G1  the gated delta rule as its authors publish it (Yang, Kautz and
      Hatamizadeh, "Gated Delta Networks", NVIDIA and MIT), per head, with the
      state S of shape [d_v, d_k]:
          S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
          o_t = S_t q_t
      alpha_t in [0, 1] is the gate (decay), beta_t in [0, 1] the write
      strength.  Both are inputs, one per (token, value head).
  G2  q and k enter L2-normalised, x / sqrt(sum x^2 + eps), and q is then
      multiplied by a scale (1/sqrt(d_k) unless stated); v enters as given.
  G3  grouped heads: n_v value heads share n_k query/key heads, value head h
      using key head h // (n_v / n_k).
  G4  decode: every sequence of a batch carries its own state; T tokens of one
      sequence are applied in order.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class GdnShape:
    n_k_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    scale: float
    eps: float = 1e-6


def l2_normalize(x, eps):
    """x / sqrt(sum(x^2) + eps) over the last axis (reading G2)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def delta_rule_step(S, q_hat, k_hat, v, alpha, beta):
    """One token of the gated delta rule on one head (reading G1), written as
    the matrix expression itself: S' = alpha S (I - beta k k^T) + beta v k^T,
    o = S' q.  q_hat and k_hat are already normalised (and q scaled)."""
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k_hat, dtype=np.float64).reshape(-1, 1)
    v = np.asarray(v, dtype=np.float64).reshape(-1, 1)
    eye = np.eye(S.shape[1])
    S_new = alpha * (S @ (eye - beta * (k @ k.T))) + beta * (v @ k.T)
    o = S_new @ np.asarray(q_hat, dtype=np.float64)
    return S_new, o


def key_head(shape: GdnShape, h):
    """The query/key head that value head h reads (reading G3)."""
    return h // (shape.n_v_heads // shape.n_k_heads)


def gdn_recurrence(shape: GdnShape, q, k, v, alpha, beta, state):
    """T tokens for each of B sequences.

    q, k: [B, T, n_k, d_k]; v: [B, T, n_v, d_v]; alpha, beta: [B, T, n_v];
    state: [B, n_v, d_v, d_k] (not modified).  Returns (out [B, T, n_v, d_v],
    new state [B, n_v, d_v, d_k]), float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    S = np.array(state, dtype=np.float64, copy=True)
    B, T = v.shape[0], v.shape[1]
    out = np.zeros((B, T, shape.n_v_heads, shape.d_v))
    for b in range(B):
        for t in range(T):
            for h in range(shape.n_v_heads):
                kh = key_head(shape, h)
                q_hat = shape.scale * l2_normalize(q[b, t, kh], shape.eps)
                k_hat = l2_normalize(k[b, t, kh], shape.eps)
                S[b, h], out[b, t, h] = delta_rule_step(S[b, h], q_hat, k_hat, v[b, t, h],
                                                        alpha[b, t, h], beta[b, t, h])
    return out, S
