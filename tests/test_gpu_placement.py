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
kernels, the MFMA prefill kernels (int4 and int8) and the stack kernel for
2..8 tokens.
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


@pytest.mark.parametrize("T", [2, 8])
def test_stack_kernel_offsets_beyond_4gib_bitwise(T):
    """The stack kernel for 2..8 tokens (moe_stack_forward, one layer) at the
    identity placement and relocated into one pool of more than 4 GiB: the
    same bits, and the oracle."""
    import int4_quantized_expert_amd as M
    from gpu_util import DEV
    data = make_layer(synth.PRESETS["80b"], 43, T, T, routing="zipf", n_cand=max(96, 16 * T))
    dl = upload(data)
    H, k = dl.desc.hidden, dl.desc.top_k

    def stack(d):
        out = torch.full((1, T, H), float("nan"), dtype=torch.float32, device=DEV)
        ids = torch.full((1, T, k), -7, dtype=torch.int32, device=DEV)
        wts = torch.full((1, T, k), float("nan"), dtype=torch.float32, device=DEV)
        ws = torch.zeros(M.workspace_bytes(d.desc, T), dtype=torch.uint8, device=DEV)
        M.workspace_init(ws)
        M.stack_forward(d.desc, 1, T, d.x, 0, d.R, 0, d.slots, 0, d.pool, d.shared, 0, out, 0, ws,
                        topk_ids=ids, topk_w=wts)
        torch.cuda.synchronize()
        M.status_check(ws)
        return out[0], ids[0], wts[0]

    y0, i0, w0 = stack(dl)
    big, slots = relocate(dl, data, seed=100 + T)
    dl2 = upload(data, pool=big, slots=slots)
    assert dl2.desc.pool_bytes > (1 << 32) and int(dl2.slots.max().item()) > (1 << 32)
    y1, i1, w1 = stack(dl2)
    assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(w0, w1)
    y_ref, ids_ref, w_ref, _ = oracle_run(data)
    check_routing(i1, w1, ids_ref, w_ref)
    check_close(y1, y_ref, data.geo.act)
    del big, dl2
    torch.cuda.empty_cache()
