"""The stack entry point (moe_stack_forward): L layers of one token each in
one call, all experts of all layers in ONE pool with per-layer slot tables
(offsets beyond 2^32 from the fifth 80B layer on).  At T = 1 on the 80B/35B
layer shapes the whole stack is one persistent launch; its results must equal
the staged kernels called layer by layer, bit for bit (outputs, ids, weights
and, in a chain, every next-layer input), and each layer must match the
oracle.  The pages run every token through the whole layer stack and report
the loop as bound by dispatch (Swiftlet README translation, "How it works"
and "Status")."""

import dataclasses

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from gpu_util import DEV, check_close, check_routing, make_layer, oracle_run, put, unambiguous
from oracle import moe_oracle as O
from synth import gpu as sgpu

pytestmark = pytest.mark.gpu


class Stack:
    """L layers of one geometry in one device pool: layer l's expert e at byte
    offset (l E + e) stride; per-layer x, routers, shared buffers and slot
    tables stacked with fixed strides."""

    def __init__(self, geo, L, T, seed, routing="zipf"):
        self.geo, self.L, self.T, self.seed = geo, L, T, seed
        E, H, stride = geo.n_experts, geo.hidden, geo.blob_stride
        print(f"stack: {L} layers of E={E} H={H}, T={T}, seed {seed}", flush=True)
        self.pool = torch.empty(L * E * stride, dtype=torch.uint8, device=DEV)
        self.layers = []
        for l in range(L):
            sgpu.fill_blobs(geo, self.pool.data_ptr() + l * E * stride, E, seed, l, 0,
                            stream=torch.cuda.current_stream().cuda_stream)
            self.layers.append(make_layer(geo, seed, l, T, routing=routing, n_cand=64))
        torch.cuda.synchronize()
        self.x = put(np.concatenate([d.x.reshape(-1) for d in self.layers]))
        self.R = put(np.concatenate([d.R.reshape(-1) for d in self.layers]))
        self.shared = put(np.concatenate([d.shared for d in self.layers]))
        self.slots = (torch.arange(L * E, dtype=torch.int64, device=DEV) * stride).reshape(L, E).contiguous()
        self.desc = M.desc_for(H, E, geo.top_k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, "f32",
                               pool_bytes=self.pool.numel())
        self.xb = T * H * geo.act_size
        self.rb = E * H * geo.act_size
        self.sb = geo.shared_bytes

    def ws(self):
        w = torch.zeros(M.workspace_bytes(self.desc, self.T), dtype=torch.uint8, device=DEV)
        M.workspace_init(w)
        return w

    def run_stack(self, chain=False, slots=None):
        L, T, H, k = self.L, self.T, self.geo.hidden, self.geo.top_k
        slots = self.slots if slots is None else slots
        out = torch.full((L, T, H), float("nan"), dtype=torch.float32, device=DEV)
        ids = torch.full((L, T, k), -7, dtype=torch.int32, device=DEV)
        wts = torch.full((L, T, k), float("nan"), dtype=torch.float32, device=DEV)
        xc = torch.zeros(L * self.xb, dtype=torch.uint8, device=DEV) if chain else None
        ws = self.ws()
        M.stack_forward(self.desc, L, T, self.x, self.xb, self.R, self.rb, slots, self.desc.n_experts * 8,
                        self.pool, self.shared, self.sb, out, T * H * 4, ws, x_chain=xc,
                        chain_stride=self.xb if chain else 0, topk_ids=ids, topk_w=wts)
        torch.cuda.synchronize()
        M.status_check(ws)
        return out, ids, wts, xc

    def run_layers(self, chain=False, slots=None):
        """The same layers one staged call after another (plus moe_residual_add in a chain)."""
        L, T, H, k = self.L, self.T, self.geo.hidden, self.geo.top_k
        slots = self.slots if slots is None else slots
        out = torch.full((L, T, H), float("nan"), dtype=torch.float32, device=DEV)
        ids = torch.full((L, T, k), -7, dtype=torch.int32, device=DEV)
        wts = torch.full((L, T, k), float("nan"), dtype=torch.float32, device=DEV)
        xc = torch.zeros(L * self.xb, dtype=torch.uint8, device=DEV) if chain else None
        ws = self.ws()
        for l in range(L):
            xl = (xc.data_ptr() + (l - 1) * self.xb) if (chain and l > 0) else self.x.data_ptr() + l * self.xb
            M.layer_forward_staged(self.desc, T, xl, self.R.data_ptr() + l * self.rb, slots[l], self.pool,
                                   self.shared.data_ptr() + l * self.sb, out[l], ws, ids[l], wts[l])
            if chain:
                M.residual_add(T, H, self.geo.act, xl, out[l], xc.data_ptr() + l * self.xb)
        torch.cuda.synchronize()
        M.status_check(ws)
        return out, ids, wts, xc


@pytest.mark.parametrize("preset,L", [("80b", 5), ("35b", 3)])
def test_stack_unchained_bitwise_and_oracle(preset, L):
    st = Stack(synth.PRESETS[preset], L, 1, 61)
    if preset == "80b":
        assert st.slots.max().item() > (1 << 32)
    a = st.run_stack()
    b = st.run_layers()
    for p, q in zip(a[:3], b[:3]):
        assert torch.equal(p, q)
    for l, data in enumerate(st.layers):
        y_ref, ids_ref, w_ref, _ = oracle_run(data)
        check_routing(a[1][l], a[2][l], ids_ref, w_ref)
        assert check_close(a[0][l], y_ref, data.geo.act) <= 2e-3


def test_stack_chained_bitwise_and_oracle():
    geo = synth.PRESETS["80b"]
    st = Stack(geo, 4, 1, 62)
    a = st.run_stack(chain=True)
    b = st.run_layers(chain=True)
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    # each layer against the oracle on its own (GPU-computed) input
    H, xb = geo.hidden, st.xb
    compared = 0
    for l, data in enumerate(st.layers):
        if l == 0:
            x_host = data.x
        else:
            x_host = a[3][(l - 1) * xb: l * xb].cpu().numpy().view(np.uint16).reshape(1, H)
        if not unambiguous(geo, x_host, data.R)[0]:
            continue
        # the oracle needs this layer's blobs for the chained input's routing
        mine = dataclasses.replace(data, x=x_host)
        xs = O.decode_dense(x_host, geo.act).reshape(1, H)
        rs = O.decode_dense(data.R, geo.act).reshape(geo.n_experts, H)
        for e in O.select_topk(O.router_logits(xs, rs)[0], geo.top_k):
            e = int(e)
            synth.fill_blob(geo, geo.inter, synth.blob_key(st.seed, l, e),
                            mine.pool[e * geo.blob_stride:(e + 1) * geo.blob_stride])
        y_ref, ids_ref, w_ref, _ = oracle_run(mine)
        check_routing(a[1][l], a[2][l], ids_ref, w_ref)
        assert check_close(a[0][l], y_ref, geo.act) <= 2e-3
        want = O.residual_next(x_host, a[0][l].cpu().numpy(), geo.act)
        got = a[3][l * xb:(l + 1) * xb].cpu().numpy().view(np.uint16).reshape(1, H)
        assert np.array_equal(got, want)
        compared += 1
    assert compared >= 2


def test_stack_bad_slot_reports_erange_like_layer_calls():
    st = Stack(synth.PRESETS["35b"], 3, 1, 63)
    _, ids, _, _ = st.run_stack()
    slots = st.slots.clone()
    slots[1, int(ids[1, 0, 0].item())] = st.pool.numel()        # layer 1's top expert: past the pool
    with pytest.raises(M.MoeError) as ei:
        st.run_stack(slots=slots)
    assert ei.value.code == -5
    with pytest.raises(M.MoeError):
        st.run_layers(slots=slots)
    # both paths drop the pair the same way
    L, H = st.L, st.geo.hidden
    a_out = torch.empty(L, 1, H, dtype=torch.float32, device=DEV)
    b_out = torch.empty_like(a_out)
    ws = st.ws()
    M.stack_forward(st.desc, L, 1, st.x, st.xb, st.R, st.rb, slots, st.desc.n_experts * 8, st.pool, st.shared,
                    st.sb, a_out, H * 4, ws)
    for l in range(L):
        M.layer_forward_staged(st.desc, 1, st.x.data_ptr() + l * st.xb, st.R.data_ptr() + l * st.rb, slots[l],
                               st.pool, st.shared.data_ptr() + l * st.sb, b_out[l], ws)
    torch.cuda.synchronize()
    with pytest.raises(M.MoeError):
        M.status_check(ws)
    assert torch.equal(a_out, b_out)


def test_stack_T2_runs_layer_by_layer():
    """T > 1 is not the one-launch case: the stack entry point runs the layers as separate calls."""
    st = Stack(synth.PRESETS["35b"], 2, 2, 64)
    a = st.run_stack(chain=True)
    b = st.run_layers(chain=True)
    # the layer calls pick the fused decode path, the reference the staged one: same bits
    for p, q in zip(a, b):
        assert torch.equal(p, q)


def test_stack_repeat_calls_on_one_workspace():
    """The per-call tags advance by the number of layers: repeated stacks and
    single-layer calls on one workspace keep giving the same bits."""
    st = Stack(synth.PRESETS["80b"], 3, 1, 65)
    L, H, k = st.L, st.geo.hidden, st.geo.top_k
    ws = st.ws()
    outs = []
    for rep in range(3):
        out = torch.empty(L, 1, H, dtype=torch.float32, device=DEV)
        M.stack_forward(st.desc, L, 1, st.x, st.xb, st.R, st.rb, st.slots, st.desc.n_experts * 8, st.pool,
                        st.shared, st.sb, out, H * 4, ws)
        one = torch.empty(1, H, dtype=torch.float32, device=DEV)
        M.layer_forward(st.desc, 1, st.x.data_ptr() + st.xb, st.R.data_ptr() + st.rb, st.slots[1], st.pool,
                        st.shared.data_ptr() + st.sb, one, ws)
        torch.cuda.synchronize()
        M.status_check(ws)
        assert torch.equal(one[0], out[1, 0])
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("preset,L,T,routing", [("80b", 3, 8, "zipf"), ("80b", 2, 8, "normal"), ("80b", 2, 2, "zipf"),
                                                ("35b", 3, 5, "zipf")])
def test_stack_multi_token_bitwise_and_oracle(preset, L, T, routing):
    """2..8 tokens per layer: one persistent launch for the stack (unchained),
    equal bit for bit to the staged kernels layer by layer, and to the oracle."""
    st = Stack(synth.PRESETS[preset], L, T, 70 + T, routing=routing)
    a = st.run_stack()
    b = st.run_layers()
    for p, q in zip(a[:3], b[:3]):
        assert torch.equal(p, q)
    for l, data in enumerate(st.layers):
        y_ref, ids_ref, w_ref, _ = oracle_run(data)
        check_routing(a[1][l], a[2][l], ids_ref, w_ref)
        assert check_close(a[0][l], y_ref, data.geo.act) <= 2e-3


def test_stack_multi_token_bad_slot_reports_erange_like_layer_calls():
    st = Stack(synth.PRESETS["35b"], 3, 4, 80)
    _, ids, _, _ = st.run_stack()
    slots = st.slots.clone()
    slots[2, int(ids[2, 1, 0].item())] = st.pool.numel() + 256        # layer 2, token 1's top expert: past the pool
    L, T, H = st.L, st.T, st.geo.hidden
    a_out = torch.empty(L, T, H, dtype=torch.float32, device=DEV)
    b_out = torch.empty_like(a_out)
    ws = st.ws()
    M.stack_forward(st.desc, L, T, st.x, st.xb, st.R, st.rb, slots, st.desc.n_experts * 8, st.pool, st.shared,
                    st.sb, a_out, T * H * 4, ws)
    torch.cuda.synchronize()
    with pytest.raises(M.MoeError) as ei:
        M.status_check(ws)
    assert ei.value.code == -5
    for l in range(L):
        M.layer_forward_staged(st.desc, T, st.x.data_ptr() + l * st.xb, st.R.data_ptr() + l * st.rb, slots[l],
                               st.pool, st.shared.data_ptr() + l * st.sb, b_out[l], ws)
    torch.cuda.synchronize()
    with pytest.raises(M.MoeError):
        M.status_check(ws)
    assert torch.equal(a_out, b_out)


def test_stack_one_and_many_tokens_share_a_workspace():
    """The one-token and the multi-token stack kernels keep their exchange
    words in one workspace region; calls of both, alternating on one
    workspace, keep giving the same bits."""
    geo = synth.PRESETS["35b"]
    s1, s4 = Stack(geo, 2, 1, 81), Stack(geo, 2, 4, 82)
    H = geo.hidden
    ws = torch.zeros(M.workspace_bytes(s4.desc, 4), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    first = {}
    for rep in range(3):
        for st in (s4, s1, s4):
            out = torch.empty(st.L, st.T, H, dtype=torch.float32, device=DEV)
            M.stack_forward(st.desc, st.L, st.T, st.x, st.xb, st.R, st.rb, st.slots, st.desc.n_experts * 8, st.pool,
                            st.shared, st.sb, out, st.T * H * 4, ws)
            torch.cuda.synchronize()
            M.status_check(ws)
            if st.T not in first:
                first[st.T] = out
            assert torch.equal(out, first[st.T])
    assert torch.equal(first[4], s4.run_layers()[0])


@pytest.mark.parametrize("T", [1, 4])
def test_stack_zero_input_ties_go_to_lowest_ids(T):
    """A zero token gives E equal logits (all 0), which the top-k takes by its
    tie path: experts 0..k-1 in order with weights 1/k, and y = 0 (h = 0 for
    every expert).  Both stack kernels equal the staged ones bit for bit."""
    st = Stack(synth.PRESETS["80b"], 2, T, 90 + T)
    st.x.zero_()
    a = st.run_stack()
    b = st.run_layers()
    for p, q in zip(a[:3], b[:3]):
        assert torch.equal(p, q)
    k = st.geo.top_k
    assert torch.equal(a[1].cpu(), torch.arange(k, dtype=torch.int32).expand(st.L, T, k))
    assert torch.equal(a[2].cpu(), torch.full((st.L, T, k), 1.0 / k, dtype=torch.float32))
    assert torch.count_nonzero(a[0]).item() == 0
