"""Placement invariance with 64-bit slot offsets, on every kernel family.

The pages: expert placement (cache or disk) never changes the answer (Swiftlet
README translation, "Correctness"), and the kernels are byte-addressed with
64-bit offsets so that multi-gigabyte pools can be addressed (same page,
"Relation to TurboFieldfare").  Each case runs a layer with its blobs at the
identity placement, then with the same blobs in one pool of more than 4 GiB,
every odd expert above byte offset 2^32 and the rest below, at a permuted
placement: outputs, ids and weights must be bitwise equal, and the relocated
run must also match the oracle.  The cases cover the single-launch T = 1
decode kernel, the two-launch T = 8 decode, the int8 decode, the staged
kernels and the MFMA prefill kernels (int4 and int8).
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_close, check_routing, make_layer, oracle_run, relocate, run, upload

pytestmark = pytest.mark.gpu

CASES = [
    # preset, T, routing, out, staged, oracle tokens
    ("80b", 1, "zipf", "f32", False, None),          # single launch
    ("80b", 8, "zipf", "f32", False, None),          # two launches
    ("80b", 1, "zipf", "f32", True, None),           # staged kernels
    ("35b_int8", 2, "zipf", "f32", False, None),     # int8 decode
    ("80b", 64, "normal", "bf16", False, [0, 31, 63]),       # MFMA prefill, int4
    ("35b_int8", 64, "zipf", "bf16", False, [0, 40, 63]),    # MFMA prefill, int8
]


@pytest.mark.parametrize("preset,T,routing,out,staged,tokens", CASES,
                         ids=[f"{c[0]}-T{c[1]}{'-staged' if c[4] else ''}" for c in CASES])
def test_offsets_beyond_4gib_bitwise(preset, T, routing, out, staged, tokens):
    margin = 2.0 if T >= 16 else 1.0
    data = make_layer(synth.PRESETS[preset], 41, T, T, routing=routing, n_cand=max(96, 16 * T),
                      margin_scale=margin, oracle_tokens=tokens)
    dl = upload(data, out)
    y0, i0, w0 = run(dl, T, staged=staged)
    big, slots = relocate(dl, data, seed=T)
    dl2 = upload(data, out, pool=big, slots=slots)
    assert dl2.desc.pool_bytes > (1 << 32)
    y1, i1, w1 = run(dl2, T, staged=staged)
    assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(w0, w1)
    y_ref, ids_ref, w_ref, _ = oracle_run(data, tokens=tokens)
    check_routing(i1, w1, ids_ref, w_ref, tokens=tokens)
    check_close(y1, y_ref, data.geo.act, tokens=tokens)
    del big, dl2
    torch.cuda.empty_cache()
