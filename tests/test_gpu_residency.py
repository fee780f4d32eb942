"""Partial residency on the GPU: a slot pool holding ~40% of the int8 experts,
refilled from pinned host memory by the cache, gives the same bits as the
fully resident pool (the pages' own check that streaming changes no answer:
Swiftlet README translation, "Correctness"), with misses, hits and evictions."""

import numpy as np
import pytest
import torch

import int4_quantized_expert_amd as M
import synth
from synth import gpu as sgpu
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [64, 8])
def test_partial_residency_bitwise_equals_resident(T):
    geo = synth.PRESETS["35b_int8"]
    L, E, k, H = 4, geo.n_experts, geo.top_k, geo.hidden
    stride = geo.blob_stride
    n_slots = (L * E * 2) // 5 if T >= 64 else 96    # 40% of the experts; fewer for small calls
    seed = 31
    cur = torch.cuda.current_stream()
    pool = torch.empty(L * E * stride, dtype=torch.uint8, device=DEV)
    for l in range(L):
        sgpu.fill_blobs(geo, pool.data_ptr() + l * E * stride, E, seed, l, 0, stream=cur.cuda_stream)
    shared = torch.from_numpy(np.concatenate([synth.make_shared(geo, seed, l) for l in range(L)])).to(DEV)
    xs, rs = [], []
    for l in range(L):
        x = synth.tokens(geo, seed, l, 2 * T)
        xs.append(x)
        rs.append(synth.router_zipf(geo, seed, l, x))
    x_d = torch.from_numpy(np.stack(xs).view(np.uint8)).to(DEV)
    r_d = torch.from_numpy(np.stack(rs).view(np.uint8)).to(DEV)
    desc = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, "f32", pool_bytes=E * stride)
    ws = torch.zeros(M.workspace_bytes(desc, T), dtype=torch.uint8, device=DEV)
    M.workspace_init(ws)
    slots_res = torch.arange(E, dtype=torch.int64, device=DEV) * stride

    def x_ptr(l, s):
        return x_d.data_ptr() + (l * 2 * T + s * T) * H * 2

    def args(l):
        return r_d.data_ptr() + l * E * H * 2, shared.data_ptr() + l * geo.shared_bytes

    # resident reference
    ref = {}
    for s in range(2):
        for l in range(L):
            out = torch.empty(T, H, dtype=torch.float32, device=DEV)
            R, sh = args(l)
            M.layer_forward(desc, T, x_ptr(l, s), R, slots_res, pool.data_ptr() + l * E * stride, sh, out, ws)
            ref[(s, l)] = out
    torch.cuda.synchronize()
    M.status_check(ws)

    # partial: pinned host store, slot pool of 40% of the experts
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    host.copy_(pool)
    torch.cuda.synchronize()
    slot_pool = torch.empty(n_slots * stride, dtype=torch.uint8, device=DEV)
    desc_p = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, "f32",
                        pool_bytes=n_slots * stride)
    cache = M.ExpertCache(n_slots, stride, slot_pool, host, L, E)
    copy_stream = torch.cuda.Stream()
    ready = torch.cuda.Event()
    done = [torch.cuda.Event() for _ in range(L)]
    ids = torch.empty(T, k, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, k, dtype=torch.float32, device=DEV)
    table_h = np.zeros(E, dtype=np.int64)
    table_d = torch.zeros(E, dtype=torch.int64, device=DEV)
    distinct = 0
    # layer-major for small calls, so a layer's hot experts are reused before eviction
    order = [(s, l) for s in range(2) for l in range(L)] if T >= 64 else [(s, l) for l in range(L) for s in range(2)]
    for s, l in order:
        R, sh = args(l)
        M.router_topk(desc_p, T, x_ptr(l, s), R, ids, wts, ws)
        ids_h = ids.cpu().numpy()
        distinct += len(np.unique(ids_h))
        cache.acquire(l, ids_h, table_h, copy_stream, ready)
        cur.wait_event(ready)
        table_d.copy_(torch.from_numpy(table_h))
        out = torch.empty(T, H, dtype=torch.float32, device=DEV)
        M.experts_forward(desc_p, T, x_ptr(l, s), ids, wts, table_d, slot_pool, sh, out, ws)
        done[l].record(cur)
        cache.release(l, done[l])
        torch.cuda.synchronize()
        M.status_check(ws)
        assert torch.equal(out, ref[(s, l)]), f"step {s} layer {l} differs from the resident run"
    hits, misses, evictions = cache.stats()
    assert hits + misses == distinct
    assert misses > 0 and evictions > 0 and hits > 0
    cache.close()
