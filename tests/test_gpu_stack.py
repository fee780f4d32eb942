"""A stack of layers chained on the GPU: the input of layer l + 1 is
x_l + y_l (moe_residual_add).  At every layer the GPU's output is checked
against the oracle run on the GPU's own input of that layer (routing exact on
every token whose top-k margin is unambiguous for float32 summation; the other
tokens are reported, not compared), and the next input must equal the
oracle's stack step of the GPU's input and output bit for bit."""

import dataclasses

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from gpu_util import DEV, check_close, check_routing, make_layer, oracle_run, put, run, unambiguous, upload
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.Geometry(hidden=512, n_experts=32, top_k=4, inter=256, shared_inter=256)


@pytest.mark.parametrize("name,T,tol", [("tiny", 4, 1e-5), ("small_bf16", 2, 2e-3), ("small_bf16", 1, 2e-3)])
def test_layer_stack_chained_parity(name, T, tol):
    geo = synth.PRESETS["tiny"] if name == "tiny" else SMALL_BF16
    L, H = 4, geo.hidden
    xdt = np.float32 if geo.act == "f32" else np.uint16
    layers = [make_layer(geo, 21, l, T) for l in range(L)]
    assert not any(d.device_fill for d in layers), "the oracle needs every blob on the host"
    x = put(layers[0].x)
    compared = 0
    for l, data in enumerate(layers):
        print(f"layer {l} T={T} {name}", flush=True)
        dl = upload(data)
        y, ids, wts = run(dl, T, x=x)
        x_host = x.cpu().numpy().view(xdt).reshape(T, H)
        mine = dataclasses.replace(data, x=x_host)
        tokens = np.nonzero(unambiguous(geo, x_host, data.R))[0]
        y_ref, ids_ref, w_ref, _ = oracle_run(mine)
        if tokens.size:
            check_routing(ids, wts, ids_ref, w_ref, tokens=tokens)
            assert check_close(y, y_ref, geo.act, tokens=tokens) <= tol
            compared += tokens.size
        x_next = torch.empty_like(x)
        M.residual_add(T, H, geo.act, x, y, x_next)
        # the chained entry point: the same output and the same next input
        y2 = torch.full_like(y, float("nan"))
        x_next2 = torch.empty_like(x)
        ws = torch.zeros(M.workspace_bytes(dl.desc, T), dtype=torch.uint8, device=DEV)
        M.workspace_init(ws)
        M.layer_forward_chain(dl.desc, T, x, dl.R, dl.slots, dl.pool, dl.shared, y2, x_next2, ws)
        torch.cuda.synchronize()
        M.status_check(ws)
        assert torch.equal(y2, y), f"layer {l}: chained output differs"
        assert torch.equal(x_next2, x_next), f"layer {l}: chained next input differs"

        want = O.residual_next(x_host, y.cpu().numpy(), geo.act)
        got = x_next.cpu().numpy().view(xdt).reshape(T, H)
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), f"layer {l} step"
        x = x_next
    assert compared >= L * T // 2, f"only {compared} of {L * T} layer-tokens had unambiguous routing"


def test_residual_add_in_place_and_rejects_bad_arguments():
    T, H = 3, 1000                      # not a multiple of the block size
    rng = np.random.default_rng(3)
    xs = synth.bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    y = rng.standard_normal((T, H)).astype(np.float32) * 1e-2
    x_d = put(xs)
    y_d = torch.from_numpy(y).to(DEV)
    M.residual_add(T, H, "bf16", x_d, y_d, x_d)           # in place
    torch.cuda.synchronize()
    assert np.array_equal(x_d.cpu().numpy().view(np.uint16).reshape(T, H), O.residual_next(xs, y, "bf16"))
    with pytest.raises(M.MoeError):
        M.residual_add(T, 0, "bf16", x_d, y_d, x_d)
    with pytest.raises(M.MoeError):
        M.residual_add(T, H, "bf16", None, y_d, x_d)
