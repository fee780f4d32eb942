"""GPU parity of the decode path against the CPU oracle, element by element,
plus the pages' invariants (placement never changes the answer: Swiftlet README
translation, section "Correctness") at the layer shapes of the workloads."""

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from gpu_util import DEV, check_close, check_routing, make_layer, oracle_run, oracle_run_all, put, run, upload

pytestmark = pytest.mark.gpu


def _parity(data, out="f32", tokens=None, staged=False):
    dl = upload(data, out)
    y, ids, wts = run(dl, data.T, staged=staged)
    y_ref, ids_ref, w_ref, _ = oracle_run(data, tokens=tokens)
    check_routing(ids, wts, ids_ref, w_ref, tokens=tokens)
    return check_close(y, y_ref, data.geo.act, tokens=tokens)


def test_tiny_fp32_parity():
    data = make_layer(synth.PRESETS["tiny"], 1, 0, 4)
    assert _parity(data) <= 1e-5


@pytest.mark.parametrize("T", [1, 8])
def test_80b_decode_full_layer(T):
    """80B-A3B-shaped layer, all 512 experts resident, Zipf-skewed routing."""
    data = make_layer(synth.PRESETS["80b"], 2, 5, T, routing="zipf", n_cand=96)
    assert _parity(data) <= 2e-3


@pytest.mark.parametrize("T", [1, 8])
def test_80b_decode_staged_path(T):
    data = make_layer(synth.PRESETS["80b"], 2, 6, T, routing="zipf", n_cand=96)
    assert _parity(data, staged=True) <= 2e-3


@pytest.mark.parametrize("preset,T,out", [("80b", 1, "f32"), ("80b", 3, "bf16"), ("80b", 8, "f32"),
                                          ("35b", 2, "f32"), ("35b_int8", 8, "bf16"), ("35b_int8", 1, "f32"),
                                          ("tiny", 5, "f32")])
def test_fused_and_staged_paths_bitwise_equal(preset, T, out):
    """The single-launch decode kernel and the staged kernels give the same bits."""
    data = make_layer(synth.PRESETS[preset], 21, T, T, routing="zipf" if preset != "tiny" else "normal",
                      n_cand=64, filter_margin=False)
    dl = upload(data, out)
    ws = torch.zeros(M.workspace_bytes(dl.desc, T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    a = run(dl, T, ws=ws)
    b = run(dl, T, ws=ws, staged=True)
    c = run(dl, T, ws=ws)            # fused again after a staged call on the same workspace
    for p, q, r in zip(a, b, c):
        assert torch.equal(p, q) and torch.equal(p, r)


def test_35b_decode_full_layer():
    data = make_layer(synth.PRESETS["35b"], 3, 7, 1, routing="zipf", n_cand=32)
    assert _parity(data) <= 2e-3


def test_35b_int8_T64_resident():
    """T = 64 takes the MFMA prefill path: routing margins at twice the float32
    bound; every token checked (the oracle's expert-major formulation)."""
    data = make_layer(synth.PRESETS["35b_int8"], 4, 1, 64, routing="zipf", n_cand=256, margin_scale=2.0)
    dl = upload(data)
    y, ids, wts = run(dl, data.T)
    y_ref, ids_ref, w_ref = oracle_run_all(data)
    check_routing(ids, wts, ids_ref, w_ref)
    assert check_close(y, y_ref, data.geo.act) <= 2e-3


def test_bf16_output():
    data = make_layer(synth.PRESETS["80b"], 5, 0, 8, routing="zipf", n_cand=64)
    dl = upload(data, "bf16")
    y, ids, wts = run(dl, data.T)
    y_ref, ids_ref, w_ref, _ = oracle_run(data)
    check_routing(ids, wts, ids_ref, w_ref)
    check_close(y, y_ref, "bf16")


@pytest.mark.parametrize("H,E,k,I,SI,bits,act,T", [
    (64, 1, 1, 64, 64, 4, "f32", 3),        # single expert, smallest rows
    (256, 16, 16, 128, 128, 4, "f32", 5),   # k == E: full softmax
    (256, 16, 1, 128, 256, 4, "f32", 7),    # k == 1, shared intermediate differs
    (128, 33, 3, 256, 64, 8, "f32", 9),     # ragged E, int8, narrow rows
    (512, 100, 6, 64, 128, 4, "bf16", 17),  # ragged token count
    (1024, 64, 4, 512, 512, 8, "bf16", 2),
])
def test_edge_shapes(H, E, k, I, SI, bits, act, T):
    geo = synth.Geometry(H, E, k, I, SI, bits, act, act)
    data = make_layer(geo, 6, H + E, T, n_cand=max(64, 8 * T))
    _parity(data)


def test_zero_tokens_leaves_output_untouched():
    data = make_layer(synth.PRESETS["tiny"], 1, 0, 4)
    dl = upload(data)
    y, ids, _ = run(dl, 0)
    assert torch.isnan(y).all() and (ids == -7).all()


def test_placement_invariance_bitwise_and_64bit_offsets():
    """Same blobs at a permuted placement, some beyond 4 GiB: bitwise equal output."""
    data = make_layer(synth.PRESETS["tiny"], 7, 0, 4)
    dl = upload(data)
    y0, i0, w0 = run(dl, data.T)
    g = data.geo
    stride = g.blob_stride
    base = (1 << 32) + 3 * 256        # beyond 32-bit byte offsets, still 256-aligned
    big = torch.zeros(base + (g.n_experts + 2) * stride, dtype=torch.uint8, device=DEV)
    perm = np.random.default_rng(0).permutation(g.n_experts + 2)[: g.n_experts]
    slots = np.empty(g.n_experts, dtype=np.int64)
    for e in range(g.n_experts):
        off = (base if e % 2 else 0) + int(perm[e]) * stride
        slots[e] = off
        big[off: off + stride] = dl.pool[e * stride:(e + 1) * stride]
    assert slots.max() > (1 << 32)
    dl2 = upload(data, pool=big, slots=slots)
    y1, i1, w1 = run(dl2, data.T)
    assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(w0, w1)
    del big
    torch.cuda.empty_cache()


def test_bad_slot_offset_reports_erange():
    data = make_layer(synth.PRESETS["tiny"], 8, 0, 4)
    dl = upload(data)
    _, ids, _ = run(dl, data.T)
    used = int(ids[0, 0].item())
    slots = data.slots.copy()
    slots[used] = dl.pool.numel()          # past the end of the pool
    dl2 = upload(data, pool=dl.pool, slots=slots)
    with pytest.raises(M.MoeError) as ei:
        run(dl2, data.T)
    assert ei.value.code == -5
    slots[used] = 8                        # misaligned
    dl3 = upload(data, pool=dl.pool, slots=slots)
    with pytest.raises(M.MoeError):
        run(dl3, data.T)


def test_split_api_matches_forward_bitwise():
    data = make_layer(synth.PRESETS["80b"], 9, 3, 8, routing="zipf", n_cand=64)
    dl = upload(data)
    y0, i0, w0 = run(dl, data.T)
    T, k, H = data.T, dl.desc.top_k, dl.desc.hidden
    ws = torch.zeros(M.workspace_bytes(dl.desc, T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, k, dtype=torch.float32, device=DEV)
    out = torch.empty(T, H, dtype=torch.float32, device=DEV)
    M.router_topk(dl.desc, T, dl.x, dl.R, ids, wts, ws)
    M.experts_forward(dl.desc, T, dl.x, ids, wts, dl.slots, dl.pool, dl.shared, out, ws)
    torch.cuda.synchronize()
    M.status_check(ws)
    assert torch.equal(ids, i0) and torch.equal(wts, w0) and torch.equal(out, y0)


def test_repeat_calls_bitwise_identical():
    data = make_layer(synth.PRESETS["35b"], 10, 2, 8, routing="zipf", n_cand=64)
    dl = upload(data)
    ws = torch.zeros(M.workspace_bytes(dl.desc, data.T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    a = run(dl, data.T, ws=ws)
    b = run(dl, data.T, ws=ws)
    assert all(torch.equal(p, q) for p, q in zip(a, b))


def test_batched_tokens_match_single_token_calls():
    """The layer is per token: T = 8 rows equal T = 1 calls within tolerance, ids exactly."""
    data = make_layer(synth.PRESETS["80b"], 11, 4, 8, routing="zipf", n_cand=64)
    dl = upload(data)
    y8, i8, _ = run(dl, 8)
    act_sz = 2
    for t in range(8):
        xt = dl.x[t * data.geo.hidden * act_sz:(t + 1) * data.geo.hidden * act_sz].clone()
        y1, i1, _ = run(dl, 1, x=xt)
        assert torch.equal(i1[0], i8[t])
        scale = y8.abs().max().item()
        assert (y1[0] - y8[t]).abs().max().item() <= 1e-6 * scale


@pytest.mark.parametrize("shift", [5, -5])
def test_exact_tie_goes_to_lower_id(shift):
    """A duplicated router row gives bitwise equal logits; the lower id ranks first."""
    geo = synth.PRESETS["tiny"]
    data = make_layer(geo, 12, 0, 1)
    top = int(oracle_run(data)[1][0, 0])
    twin = (top + shift) % geo.n_experts
    R = data.R.copy().reshape(geo.n_experts, -1)
    R[twin] = R[top]
    data.R = R.reshape(data.R.shape)
    _, ids, _ = run(upload(data), 1)
    got = ids.cpu().numpy()[0]
    assert sorted(got) == sorted([top, twin])        # k = 2: both copies are chosen
    assert got[0] == min(top, twin)


def test_device_fill_matches_host_generator():
    from synth import gpu
    for geo in (synth.PRESETS["80b"], synth.PRESETS["35b_int8"], synth.PRESETS["tiny"]):
        n = 3
        buf = torch.zeros(n * geo.blob_stride, dtype=torch.uint8, device=DEV)
        gpu.fill_blobs(geo, buf.data_ptr(), n, seed=5, layer=9, blob_id0=40)
        torch.cuda.synchronize()
        got = buf.cpu().numpy()
        for i in range(n):
            ref = synth.fill_blob(geo, geo.inter, synth.blob_key(5, 9, 40 + i))
            assert np.array_equal(got[i * geo.blob_stride:(i + 1) * geo.blob_stride], ref)
        sh = torch.zeros(geo.shared_stride, dtype=torch.uint8, device=DEV)
        gpu.fill_blobs(geo, sh.data_ptr(), 1, seed=5, layer=9, shared=True)
        torch.cuda.synchronize()
        ref = synth.fill_blob(geo, geo.shared_inter, synth.blob_key(5, 9, synth.SHARED_BLOB_ID))
        assert np.array_equal(sh.cpu().numpy(), ref)


def test_launch_event_hook_times_each_kernel():
    """moe_set_launch_events: a start and an end event per kernel, consumed by exactly one
    call; timing does not change the result."""
    data = make_layer(synth.PRESETS["80b"], 4, 9, 1, routing="zipf", n_cand=32)
    dl = upload(data, "f32")
    ref = run(dl, 1)
    for staged, kernels in ((False, 1), (True, 6)):   # T = 1 runs in one launch
        timer = M.LaunchTimer(16)
        timer.arm()
        got = run(dl, 1, staged=staged)
        assert timer.n_recorded == 2 * kernels
        us = timer.kernel_us()
        assert len(us) == kernels and all(u > 0 for u in us), us
        for p, q in zip(ref, got):
            assert torch.equal(p, q)
        n_before = timer.n_recorded
        run(dl, 1, staged=staged)          # not armed: records nothing more
        assert timer.n_recorded == n_before
