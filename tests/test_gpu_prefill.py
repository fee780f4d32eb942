"""GPU parity of the prefill path against the CPU oracle.

Calls with T >= 16 tokens and bf16 activations run the router and the expert
products on MFMA (float16 dequantized weights, float16 activations and h, fp32
sums): the pages' expert computation (Swiftlet README translation, "How it
works") at a batch size where each expert sees many tokens.  Routing is
compared exactly on margin-filtered tokens (2x the float32 summation bound,
since MFMA's internal rounding is not specified per addition); outputs within
2e-3 of max|y| (+ half a bf16 ulp for bf16 outputs).
"""

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from gpu_util import (DEV, check_close, check_routing, make_layer, oracle_routing, oracle_run, oracle_run_all,
                      run, upload)

pytestmark = pytest.mark.gpu

PF = 2.0   # margin scale for MFMA router logits


def _parity(data, out="f32", tokens=None):
    """Checks routing and outputs (check_close asserts the tolerance, with half a
    bf16 ulp per element for bf16 outputs); returns max error / max|y_ref| of
    float32 outputs, 0 for bf16 ones, whose rounding alone can exceed 2e-3."""
    dl = upload(data, out)
    y, ids, wts = run(dl, data.T)
    ids_all, w_all = oracle_routing(data)
    check_routing(ids, wts, ids_all, w_all)
    y_ref, _, _, _ = oracle_run(data, tokens=tokens)
    r = check_close(y, y_ref, data.geo.act, tokens=tokens)
    return r if out == "f32" else 0.0


@pytest.mark.parametrize("bits,out,T", [(4, "f32", 100), (4, "bf16", 16), (8, "f32", 77), (8, "bf16", 130)])
def test_small_prefill_every_token(bits, out, T):
    """H = 256, 16 experts, I = 256, SI = 512: several tiles, ragged tails, every token checked."""
    geo = synth.Geometry(256, 16, 2, 256, 512, bits, "bf16", "bf16")
    data = make_layer(geo, 13, bits, T, n_cand=4 * T, margin_scale=PF)
    assert _parity(data, out) <= 2e-3


def test_small_prefill_f32_scales():
    geo = synth.Geometry(512, 32, 4, 256, 256, 4, "bf16", "f32")
    data = make_layer(geo, 14, 0, 48, n_cand=256, margin_scale=PF)
    assert _parity(data) <= 2e-3


def test_80b_prefill_T2048_bf16_out():
    """80B-A3B layer shape at T = 2048 with near-uniform routing (~40 tokens per
    expert, all 512 experts used), bf16 output: routing and outputs checked on
    every token, against the oracle's expert-major formulation.  Every
    expert's pair list, and with it the first and last column of every
    64-pair tile and every ragged tail, is covered."""
    T = 2048
    data = make_layer(synth.PRESETS["80b"], 15, 0, T, n_cand=16000, margin_scale=PF)
    dl = upload(data, "bf16")
    y, ids, wts = run(dl, T)
    y_ref, ids_ref, w_ref = oracle_run_all(data)
    counts = np.bincount(ids_ref.reshape(-1), minlength=data.geo.n_experts)
    assert counts.min() > 0 and (counts % 64 != 0).any()
    check_routing(ids, wts, ids_ref, w_ref)
    check_close(y, y_ref, data.geo.act)


def test_80b_prefill_hot_experts_span_tiles():
    """Zipf routing over 40 distinct tokens repeated to T = 256: the hottest experts
    get several 64-pair tiles, and a repeated token gives bitwise equal rows
    wherever its pairs land in the tiles."""
    T, U = 256, 40
    data = make_layer(synth.PRESETS["80b"], 16, 2, U, routing="zipf", n_cand=600, margin_scale=PF,
                      oracle_tokens=[0, 7, 13, 39])
    data.x = np.ascontiguousarray(np.tile(data.x, (T // U + 1, 1))[:T])
    ids_all, _ = oracle_routing(data)
    counts = np.bincount(ids_all.reshape(-1), minlength=data.geo.n_experts)
    assert counts.max() > 128, "routing should put more than two tiles on one expert"
    dl = upload(data)
    y, ids, wts = run(dl, T)
    check_routing(ids, wts, ids_all, oracle_routing(data)[1])
    for t in (0, 7, 13, 39):
        for rep in (t + U, t + 4 * U):
            assert torch.equal(y[rep], y[t])
    sample = [0, 7, 13, 39]
    y_ref, _, _, _ = oracle_run(data, tokens=sample)
    assert check_close(y, y_ref, "bf16", tokens=sample) <= 2e-3


def test_35b_prefill_int8():
    """35B-A3B shape with int8 experts at T = 64, every token checked."""
    T = 64
    data = make_layer(synth.PRESETS["35b_int8"], 17, 3, T, routing="zipf", n_cand=4 * T, margin_scale=PF)
    dl = upload(data, "bf16")
    y, ids, wts = run(dl, T)
    y_ref, ids_ref, w_ref = oracle_run_all(data)
    check_routing(ids, wts, ids_ref, w_ref)
    check_close(y, y_ref, data.geo.act)


def test_prefill_split_api_and_repeat_bitwise():
    data = make_layer(synth.PRESETS["35b"], 18, 1, 64, routing="zipf", n_cand=256, margin_scale=PF,
                      oracle_tokens=[0])
    dl = upload(data)
    T, k, H = data.T, dl.desc.top_k, dl.desc.hidden
    ws = torch.zeros(M.workspace_bytes(dl.desc, T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    y0, i0, w0 = run(dl, T, ws=ws)
    y1, i1, w1 = run(dl, T, ws=ws)
    assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(w0, w1)
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = torch.empty(T, H, dtype=torch.float32, device=DEV)
    M.router_topk(dl.desc, T, dl.x, dl.R, ids, wts, ws)
    M.experts_forward(dl.desc, T, dl.x, ids, wts, dl.slots, dl.pool, dl.shared, out, ws)
    torch.cuda.synchronize()
    M.status_check(ws)
    assert torch.equal(ids, i0) and torch.equal(wts, w0) and torch.equal(out, y0)


def test_prefill_tokens_match_single_token_decode():
    """Per-token invariance across paths: the prefill rows equal T = 1 decode calls
    within the tolerance, with identical ids."""
    data = make_layer(synth.PRESETS["80b"], 19, 4, 32, n_cand=400, margin_scale=PF, oracle_tokens=[0])
    dl = upload(data)
    yp, ip, _ = run(dl, 32)
    H = data.geo.hidden
    scale = yp.abs().max().item()
    for t in (0, 5, 31):
        y1, i1, _ = run(dl, 1, x=dl.x[t * H * 2:(t + 1) * H * 2].clone())
        assert torch.equal(i1[0], ip[t])
        assert (y1[0] - yp[t]).abs().max().item() <= 2e-3 * scale


def test_prefill_bad_slot_reports_erange_and_drops_the_expert():
    geo = synth.Geometry(256, 16, 2, 256, 256, 4, "bf16", "bf16")
    data = make_layer(geo, 20, 0, 32, n_cand=128, margin_scale=PF)
    dl = upload(data)
    _, ids, _ = run(dl, 32)
    used = int(ids[0, 0].item())
    slots = data.slots.copy()
    slots[used] = dl.pool.numel()
    with pytest.raises(M.MoeError) as ei:
        run(upload(data, pool=dl.pool, slots=slots), 32)
    assert ei.value.code == -5


def test_prefill_bad_expert_id_reports_erange_and_drops_only_that_pair():
    """An id outside [0, E) handed to the split API is reported (MOE_ERANGE) and
    its pair contributes nothing: the output equals the call with that pair's
    weight set to zero, bit for bit, for every token."""
    geo = synth.Geometry(256, 16, 2, 256, 256, 4, "bf16", "bf16")
    data = make_layer(geo, 21, 0, 48, n_cand=128, margin_scale=PF)
    dl = upload(data)
    T, k, H, E = data.T, dl.desc.top_k, dl.desc.hidden, dl.desc.n_experts
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ws = torch.zeros(M.workspace_bytes(dl.desc, T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    M.router_topk(dl.desc, T, dl.x, dl.R, ids, wts, ws)
    torch.cuda.synchronize()
    bad_ids = ids.clone()
    bad_ids[3, 1] = E + 7
    out_bad = torch.empty(T, H, dtype=torch.float32, device=DEV)
    M.experts_forward(dl.desc, T, dl.x, bad_ids, wts, dl.slots, dl.pool, dl.shared, out_bad, ws)
    torch.cuda.synchronize()
    with pytest.raises(M.MoeError) as ei:
        M.status_check(ws)
    assert ei.value.code == -5
    zero_w = wts.clone()
    zero_w[3, 1] = 0.0
    ws2 = torch.zeros_like(ws)
    M.workspace_init(ws2)
    out_zero = torch.empty(T, H, dtype=torch.float32, device=DEV)
    M.experts_forward(dl.desc, T, dl.x, ids, zero_w, dl.slots, dl.pool, dl.shared, out_zero, ws2)
    torch.cuda.synchronize()
    M.status_check(ws2)
    assert torch.equal(out_bad, out_zero)


@pytest.mark.parametrize("where", ["input", "h"])
def test_prefill_float16_range_reports_eoverflow(where):
    """The prefill path keeps x, h and the partial down rows in float16, so
    they must stay inside its range (reading R11).  A value that leaves it is
    reported by the status check (MOE_EOVERFLOW) instead of passing silently
    as inf: an input of 1e5 (over 65504), or inputs of about 3000 on one
    token, whose h products reach about 1e6 while every input fits."""
    geo = synth.Geometry(256, 16, 2, 256, 256, 4, "bf16", "bf16")
    data = make_layer(geo, 23, 0, 32, n_cand=128, margin_scale=PF)
    dl = upload(data)
    run(dl, 32)                                   # in range: no flag
    x = dl.x.clone().view(torch.int16)
    if where == "input":
        x[5 * geo.hidden + 17] = 0x47C3           # bf16 1.0e5
    else:
        x[:geo.hidden] = 0x453B                   # bf16 2992 on token 0
    with pytest.raises(M.MoeError) as ei:
        run(dl, 32, x=x.view(torch.uint8))
    assert ei.value.code == -9
    run(dl, 32)                                   # the flag was cleared by the check
