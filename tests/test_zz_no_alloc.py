"""The no-allocation entry point (moe_layer_forward_noalloc): the library's
own fixed scratch array instead of a caller workspace.  Called through the C
ABI, two calls in a row on each shape (the second with fewer tokens), its
results must equal moe_layer_forward on a caller workspace bit for bit, and a
bad slot offset must come back through its status word."""

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from gpu_util import DEV, make_layer, run, upload

pytestmark = pytest.mark.gpu


def _noalloc(dl, T, x=None, slots=None, status=None):
    H, k = dl.desc.hidden, dl.desc.top_k
    g_out = torch.float32 if dl.desc.out_dtype == M.MOE_F32 else torch.bfloat16
    out = torch.full((T, H), float("nan"), dtype=g_out, device=DEV)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    wts = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    M.layer_forward_noalloc(dl.desc, T, dl.x if x is None else x, dl.R, dl.slots if slots is None else slots,
                            dl.pool, dl.shared, out, ids, wts, status=status)
    torch.cuda.synchronize()
    return out, ids, wts


@pytest.mark.parametrize("preset,T1,T2,out", [("tiny", 4, 2, "f32"), ("80b", 8, 1, "f32"), ("35b_int8", 64, 16, "bf16"),
                                              ("80b", 1, 1, "f32")])
def test_noalloc_equals_workspace_call_twice(preset, T1, T2, out):
    geo = synth.PRESETS[preset]
    print(f"noalloc {preset} T={T1} then T={T2}", flush=True)
    data = make_layer(geo, 71, T1, T1, routing="zipf" if preset != "tiny" else "normal", n_cand=max(64, 4 * T1),
                      filter_margin=False)
    dl = upload(data, out)
    for T in (T1, T2):
        x = dl.x[: T * geo.hidden * geo.act_size]
        want = run(dl, T, x=x)
        got = _noalloc(dl, T, x=x)
        for p, q in zip(want, got):
            assert torch.equal(p, q), f"{preset} T={T}"


def test_noalloc_status_word_and_size_limit():
    geo = synth.PRESETS["35b"]
    data = make_layer(geo, 72, 0, 2, routing="zipf", n_cand=64, filter_margin=False)
    dl = upload(data)
    status = torch.full((1,), 0x7777, dtype=torch.int32, device=DEV)
    _, ids, _ = _noalloc(dl, 2, status=status)
    assert status.item() == 0
    slots = data.slots.copy()
    slots[int(ids[0, 0].item())] = dl.pool.numel()             # past the end of the pool
    bad = torch.from_numpy(slots).to(DEV)
    y_bad, _, _ = _noalloc(dl, 2, slots=bad, status=status)
    assert status.item() & 1
    y_ok, _, _ = _noalloc(dl, 1, status=status)                 # a good, smaller call: flags were cleared
    assert status.item() == 0
    want = run(dl, 1)
    assert torch.equal(want[0], y_ok)
    big = M.desc_for(2048, 512, 10, 512, 512, 4, "bf16", "bf16", "bf16", pool_bytes=dl.desc.pool_bytes)
    assert M.workspace_bytes(big, 2048) > (16 << 20)
    with pytest.raises(M.MoeError) as ei:
        M.layer_forward_noalloc(big, 2048, dl.x, dl.R, dl.slots, dl.pool, dl.shared,
                                torch.empty(1, device=DEV), None, None)
    assert ei.value.code == -4
