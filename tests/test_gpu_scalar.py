"""The scalar kernels (moe_layer_forward_scalar: one GPU thread per output
value, no cross-lane operations) against the fast kernels, bit for bit: the
pages check their fast kernels against scalar ones that give identical output
(Swiftlet README translation, "Correctness").  For T <= 8 the fast path is
the decode kernels of moe_layer_forward (the one-launch stack kernel at T = 1
on the 80B/35B shapes, the fused kernels otherwise); for any T it is the
staged kernels.  Outputs, ids and weights must be equal, and the scalar path
must also match the oracle."""

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from gpu_util import DEV, check_close, check_routing, make_layer, oracle_run, run, upload

pytestmark = pytest.mark.gpu


def run_scalar(dl, T):
    g_out = torch.float32 if dl.desc.out_dtype == M.MOE_F32 else torch.bfloat16
    H, k = dl.desc.hidden, dl.desc.top_k
    out = torch.full((T, H), float("nan"), dtype=g_out, device=DEV)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    wts = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(M.workspace_bytes(dl.desc, T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    M.layer_forward_scalar(dl.desc, T, dl.x, dl.R, dl.slots, dl.pool, dl.shared, out, ws, ids, wts)
    torch.cuda.synchronize()
    M.status_check(ws)
    return out, ids, wts


@pytest.mark.parametrize("preset,T,out", [
    ("80b", 1, "f32"),        # fast: the stack kernel
    ("35b", 1, "bf16"),       # the stack kernel, bf16 output
    ("80b", 8, "f32"),        # fused, two launches
    ("80b", 3, "bf16"),
    ("35b_int8", 2, "f32"),   # int8 codes
    ("tiny", 4, "f32"),       # float32 activations and scales
])
def test_scalar_equals_fast_decode(preset, T, out):
    geo = synth.PRESETS[preset]
    data = make_layer(geo, 81, T, T, routing="zipf" if preset != "tiny" else "normal", n_cand=max(64, 8 * T))
    dl = upload(data, out)
    fast = run(dl, T)
    scal = run_scalar(dl, T)
    for p, q in zip(fast, scal):
        assert torch.equal(p, q), preset
    y_ref, ids_ref, w_ref, _ = oracle_run(data)
    check_routing(scal[1], scal[2], ids_ref, w_ref)
    check_close(scal[0], y_ref, geo.act)


@pytest.mark.parametrize("H,E,k,I,SI,bits,act,T", [
    (64, 1, 1, 64, 64, 4, "f32", 3),         # single expert, two-segment rows
    (256, 16, 16, 128, 128, 4, "f32", 5),    # k == E
    (128, 33, 3, 256, 64, 8, "f32", 9),      # ragged E, int8, narrow rows
    (512, 100, 6, 64, 128, 4, "bf16", 17),   # ragged T, v_dot2 rows of 16 segments
    (1024, 64, 4, 512, 512, 8, "bf16", 2),
    (2048, 512, 10, 512, 512, 4, "bf16", 20),  # 80B shape beyond decode sizes
])
def test_scalar_equals_staged(H, E, k, I, SI, bits, act, T):
    geo = synth.Geometry(H, E, k, I, SI, bits, act, act)
    data = make_layer(geo, 82, H + E, T, n_cand=max(64, 8 * T), filter_margin=False)
    dl = upload(data)
    staged = run(dl, T, staged=True)
    scal = run_scalar(dl, T)
    for p, q in zip(staged, scal):
        assert torch.equal(p, q)
