"""Seeded synthetic inputs for the gated-delta-rule recurrence.

This module only draws numbers; it computes nothing of the rule.  The oracle's
callers and the HIP path's callers take their inputs from here.

Sizes.  The pages print no DeltaNet sizes.  "80b" takes 16 query/key heads and
32 value heads of width 128 (the published configuration of the Qwen3-Next
80B model the pages run); "tiny" is a small case for fast parity checks.

Value recipe: q, k, v ~ N(0, 1) rounded to the activation dtype; alpha (the
gate) ~ U(0.5, 1); beta (the write strength) ~ U(0, 1); the incoming state
~ N(0, 0.5^2) in float32, standing for a state part-way through a sequence.
All draws come from numpy's PCG64 keyed by (seed, B, T).
"""

from __future__ import annotations

import numpy as np

from . import to_act

GDN_PRESETS = {
    "tiny": dict(n_k_heads=2, n_v_heads=4, d_k=64, d_v=32),
    "80b": dict(n_k_heads=16, n_v_heads=32, d_k=128, d_v=128),
}


def gdn_inputs(n_k_heads: int, n_v_heads: int, d_k: int, d_v: int, B: int, T: int, seed: int,
               act: str = "bf16", state_std: float = 0.5):
    """Returns raw q, k [B, T, n_k, d_k], v [B, T, n_v, d_v] (activation
    storage), alpha, beta [B, T, n_v] float32 and state [B, n_v, d_v, d_k]
    float32."""
    rng = np.random.Generator(np.random.PCG64([seed, 0x6D17, B, T]))
    q = to_act(rng.standard_normal((B, T, n_k_heads, d_k), dtype=np.float32), act)
    k = to_act(rng.standard_normal((B, T, n_k_heads, d_k), dtype=np.float32), act)
    v = to_act(rng.standard_normal((B, T, n_v_heads, d_v), dtype=np.float32), act)
    alpha = (np.float32(0.5) + np.float32(0.5) * rng.random((B, T, n_v_heads), dtype=np.float32)).astype(np.float32)
    beta = rng.random((B, T, n_v_heads), dtype=np.float32)
    state = (rng.standard_normal((B, n_v_heads, d_v, d_k), dtype=np.float32) * np.float32(state_std)).astype(np.float32)
    return q, k, v, alpha, beta, state
