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


def _resident_reference(T, L, seed):
    """Inputs of an L-layer 35B int8 run and its fully resident outputs."""
    geo = synth.PRESETS["35b_int8"]
    E, k, H = geo.n_experts, geo.top_k, geo.hidden
    stride = geo.blob_stride
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
    ctx = dict(geo=geo, L=L, T=T, pool=pool, shared=shared, x_d=x_d, r_d=r_d, ws=ws)
    ref = {}
    for s in range(2):
        for l in range(L):
            out = torch.empty(T, H, dtype=torch.float32, device=DEV)
            R, sh = _layer_args(ctx, l)
            M.layer_forward(desc, T, _x_ptr(ctx, l, s), R, slots_res, pool.data_ptr() + l * E * stride, sh, out, ws)
            ref[(s, l)] = out
    torch.cuda.synchronize()
    M.status_check(ws)
    ctx["ref"] = ref
    return ctx


def _x_ptr(ctx, l, s):
    T, H = ctx["T"], ctx["geo"].hidden
    return ctx["x_d"].data_ptr() + (l * 2 * T + s * T) * H * 2


def _layer_args(ctx, l):
    geo = ctx["geo"]
    E, H = geo.n_experts, geo.hidden
    return ctx["r_d"].data_ptr() + l * E * H * 2, ctx["shared"].data_ptr() + l * geo.shared_bytes


def _run_partial(ctx, cache, n_slots, slot_pool):
    """Every (step, layer) call through the cache; each output must equal the
    resident one bit for bit.  Returns (hits, misses, evictions, distinct)."""
    geo, L, T, ws = ctx["geo"], ctx["L"], ctx["T"], ctx["ws"]
    E, k, H = geo.n_experts, geo.top_k, geo.hidden
    cur = torch.cuda.current_stream()
    desc_p = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, "f32",
                        pool_bytes=n_slots * geo.blob_stride)
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
        R, sh = _layer_args(ctx, l)
        M.router_topk(desc_p, T, _x_ptr(ctx, l, s), R, ids, wts, ws)
        ids_h = ids.cpu().numpy()
        distinct += len(np.unique(ids_h))
        cache.acquire(l, ids_h, table_h, copy_stream, ready)
        cur.wait_event(ready)
        table_d.copy_(torch.from_numpy(table_h))
        out = torch.empty(T, H, dtype=torch.float32, device=DEV)
        M.experts_forward(desc_p, T, _x_ptr(ctx, l, s), ids, wts, table_d, slot_pool, sh, out, ws)
        done[l].record(cur)
        cache.release(l, done[l])
        torch.cuda.synchronize()
        M.status_check(ws)
        assert torch.equal(out, ctx["ref"][(s, l)]), f"step {s} layer {l} differs from the resident run"
    return (*cache.stats(), distinct)


@pytest.mark.parametrize("T", [64, 8])
def test_partial_residency_bitwise_equals_resident(T):
    L, seed = 4, 31
    ctx = _resident_reference(T, L, seed)
    geo = ctx["geo"]
    E, stride = geo.n_experts, geo.blob_stride
    n_slots = (L * E * 2) // 5 if T >= 64 else 96    # 40% of the experts; fewer for small calls
    # partial: pinned host store, slot pool of 40% of the experts
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    host.copy_(ctx["pool"])
    torch.cuda.synchronize()
    slot_pool = torch.empty(n_slots * stride, dtype=torch.uint8, device=DEV)
    cache = M.ExpertCache(n_slots, stride, slot_pool, host, L, E)
    hits, misses, evictions, distinct = _run_partial(ctx, cache, n_slots, slot_pool)
    assert hits + misses == distinct
    assert misses > 0 and evictions > 0 and hits > 0
    cache.close()


@pytest.mark.parametrize("direct", [False, True])
def test_partial_residency_from_file_store_bitwise_equals_resident(tmp_path, direct):
    """The same run with misses read from a container file of fixed-stride
    blobs (one positioned read per blob into pinned staging, then the copy):
    linlog.top article, core design 2; the output still equals the resident
    run bit for bit."""
    L, T, seed = 2, 64, 37
    ctx = _resident_reference(T, L, seed)
    geo = ctx["geo"]
    E, stride = geo.n_experts, geo.blob_stride
    path = str(tmp_path / "experts.store")
    store_w = M.ExpertStore.create(path, L, E, stride, geo.blob_bytes(geo.inter))
    host = ctx["pool"].cpu().numpy()
    for l in range(L):
        for e in range(E):
            store_w.write(l, e, host[(l * E + e) * stride:(l * E + e + 1) * stride])
    store_w.close()
    del host
    try:
        store = M.ExpertStore(path, direct=direct)
    except M.MoeError as err:
        if direct:
            pytest.skip(f"this file system refuses O_DIRECT: {err}")
        raise
    assert (store.n_layers, store.n_experts, store.stride) == (L, E, stride)
    n_slots = (L * E * 2) // 5
    n_staging = 4
    staging = torch.empty(n_staging * stride, dtype=torch.uint8, pin_memory=True)
    slot_pool = torch.empty(n_slots * stride, dtype=torch.uint8, device=DEV)
    cache = M.ExpertCache.from_store(n_slots, slot_pool, store, staging, n_staging)
    hits, misses, evictions, distinct = _run_partial(ctx, cache, n_slots, slot_pool)
    assert hits + misses == distinct
    assert misses > n_staging and evictions > 0 and hits > 0
    cache.close()
    store.close()


@pytest.mark.parametrize("keep_counts", [False, True])
def test_eviction_while_the_reader_is_in_flight(keep_counts):
    """Hazard ordering with no host wait on the compute: call i + 1's router
    runs on its own stream and its acquire evicts slots that call i's experts
    (held back on the compute stream behind a long matmul) have not read yet.
    The copies must wait for call i's compute_done event; every output must
    still equal the fully resident run bit for bit (explicit hazard
    management: Swiftlet README translation, "Relation to TurboFieldfare").
    Separate workspaces for the router and the experts; a pinned slot table
    per call, since the compute stream copies it after the host moved on."""
    L, T, seed = 4, 64, 43
    ctx = _resident_reference(T, L, seed)
    geo = ctx["geo"]
    E, k, H, stride = geo.n_experts, geo.top_k, geo.hidden, geo.blob_stride
    n_slots = 200
    host = torch.empty(L * E * stride, dtype=torch.uint8, pin_memory=True)
    host.copy_(ctx["pool"])
    torch.cuda.synchronize()
    slot_pool = torch.empty(n_slots * stride, dtype=torch.uint8, device=DEV)
    cache = M.ExpertCache(n_slots, stride, slot_pool, host, L, E)
    cache.set_policy(keep_counts)
    desc_p = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, "f32",
                        pool_bytes=n_slots * stride)
    ws_r = torch.zeros(M.workspace_bytes(desc_p, T), dtype=torch.uint8, device=DEV)
    ws_c = torch.zeros_like(ws_r)
    M.workspace_init(ws_r)
    M.workspace_init(ws_c)
    s_route, s_comp, s_copy = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn(3072, 3072, device=DEV)
    torch.cuda.synchronize()
    # both steps of a layer back to back (hits), then the next layer (evictions)
    order = [(s, l) for rep in range(2) for l in range(L) for s in range(2)]
    calls, in_flight_evictions = [], 0
    for i, (s, l) in enumerate(order):
        R, sh = _layer_args(ctx, l)
        c = dict(s=s, l=l, ids=torch.empty(T, k, dtype=torch.int32, device=DEV),
                 wts=torch.empty(T, k, dtype=torch.float32, device=DEV),
                 ids_h=torch.empty(T, k, dtype=torch.int32, pin_memory=True),
                 table_h=torch.zeros(E, dtype=torch.int64, pin_memory=True),
                 table_d=torch.empty(E, dtype=torch.int64, device=DEV),
                 out=torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV),
                 routed=torch.cuda.Event(), ready=torch.cuda.Event(), done=torch.cuda.Event())
        with torch.cuda.stream(s_route):
            M.router_topk(desc_p, T, _x_ptr(ctx, l, s), R, c["ids"], c["wts"], ws_r, stream=s_route)
            c["ids_h"].copy_(c["ids"], non_blocking=True)
            c["routed"].record(s_route)
        c["routed"].synchronize()                     # the host waits for the router only
        cache.acquire(l, c["ids_h"].numpy(), c["table_h"].numpy(), s_copy, c["ready"])
        if calls:
            p = calls[-1]
            if not p["done"].query():
                used = np.unique(p["ids_h"].numpy())
                in_flight_evictions += sum(cache.slot_of(p["l"], int(e)) * stride != int(p["table_h"][e])
                                           for e in used)
        with torch.cuda.stream(s_comp):
            s_comp.wait_event(c["routed"])
            s_comp.wait_event(c["ready"])
            torch.mm(a, a)                            # keeps this call's readers pending for a while
            c["table_d"].copy_(c["table_h"], non_blocking=True)
            M.experts_forward(desc_p, T, _x_ptr(ctx, l, s), c["ids"], c["wts"], c["table_d"], slot_pool, sh,
                              c["out"], ws_c, stream=s_comp)
            c["done"].record(s_comp)
        cache.release(l, c["done"])
        calls.append(c)
    torch.cuda.synchronize()
    M.status_check(ws_r)
    M.status_check(ws_c)
    for i, c in enumerate(calls):
        assert torch.equal(c["out"], ctx["ref"][(c["s"], c["l"])]), f"call {i} (step {c['s']}, layer {c['l']})"
    hits, misses, evictions = cache.stats()
    assert evictions > 0 and hits > 0
    assert in_flight_evictions > 0, "no slot was evicted while its reader was pending: the test did not test"
    cache.close()
