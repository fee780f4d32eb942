"""The pins catch plausible oracle mistakes: each mutation below plants one slip
in the oracle (on the CPU, via monkeypatch) and at least one pin must fail."""

import numpy as np
import pytest

from oracle import moe_oracle as O
import test_oracle as P

PINS = [
    P.test_unpack_int4_hand_worked,
    P.test_unpack_int8_hand_worked,
    lambda: P.test_blob_layout_orientation_and_groups(4, "f32"),
    lambda: P.test_blob_layout_orientation_and_groups(8, "f32"),
    P.test_router_orientation_one_hot,
    P.test_topk_order_and_ties,
    P.test_renormalisation_closed_form,
    P.test_uniform_layer_closed_form,
    P.test_zero_experts_leave_only_shared,
    P.test_constant_experts_closed_form,
    P.test_identical_experts_routed_part_is_expert,
]


def _high_nibble_first(words, rows, cols, bits):
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint32).reshape(rows, cols // per)
    q = np.empty((rows, cols // per, per), dtype=np.uint8)
    for j in range(per):
        q[:, :, j] = (w >> np.uint32(bits * (per - 1 - j))) & np.uint32((1 << bits) - 1)
    return q.reshape(rows, cols)


def _group_along_rows(q, s, b):
    rows, cols = q.shape
    out = np.empty((rows, cols))
    for r in range(rows):
        for c in range(cols):
            gi = (r // 64) % s.shape[1] if s.shape[1] else 0
            out[r, c] = s[r % s.shape[0], gi] * q[r, c] + b[r % s.shape[0], gi]
    return out


_orig_parse = O.parse_blob
_orig_topk = O.select_topk
_orig_expert = O.expert_forward


def _swap_gate_up(blob, H, I, bits, sb):
    g, u, d = _orig_parse(blob, H, I, bits, sb)
    return u, g, d


def _transpose_down(blob, H, I, bits, sb):
    g, u, d = _orig_parse(blob, H, I, bits, sb)
    return g, u, d.reshape(I, H).T.copy()


def _ties_to_higher(l, k):
    ids = np.arange(l.shape[0])
    return np.lexsort((-ids, -l))[:k].astype(np.int32)


def _silu_on_up(wg, wu, wd, x):
    return wd @ ((wg @ x) * O.silu(wu @ x))


MUTATIONS = {
    "high_nibble_first": ("unpack_q", _high_nibble_first),
    "group_axis_rows": ("dequantize", _group_along_rows),
    "swap_gate_up": ("parse_blob", _swap_gate_up),
    "transpose_down": ("parse_blob", _transpose_down),
    "router_transposed": ("router_logits", lambda x, R: (x @ R.reshape(R.shape[1], R.shape[0]))
                          if R.shape[0] != R.shape[1] else x @ R),
    "ties_to_higher_id": ("select_topk", _ties_to_higher),
    "no_renormalisation": ("renormalised_weights", lambda sl: np.exp(sl) / (np.exp(sl).sum() + 1.0)),
    "gate_sign": ("sigmoid", lambda a: 1.0 / (1.0 + np.exp(a))),
    "silu_on_up": ("expert_forward", _silu_on_up),
    "bias_dropped": ("dequantize", lambda q, s, b: (s[:, :, None] * q.reshape(
        q.shape[0], -1, 64).astype(np.float64)).reshape(q.shape)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"mutation {name} passed every pin"
