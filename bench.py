#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

Workloads (synthetic, seeded; pools filled in place by the device generator):

  80b_stack_decode (default)  80B-A3B-shaped stack decode: 48 layers, each with
      512 routed int4 g64 experts (bf16 scales/biases, 1,769,472-byte blobs)
      resident in one 43.5 GB HBM pool, top-10 routing with Zipf(1.1)-skewed
      popularity, a sigmoid-gated shared expert, T tokens per step (--tokens,
      default 1), float32 output.  One step = one token step through all 48
      layers in order, each layer one moe_layer_forward call.
  35b_rotation_decode  35B-A3B shape (256 experts, top-8) over 40 layers.
  80b_prefill  the 80B layer shape at T = 2048 tokens per call with near-uniform
      routing (about 40 tokens per expert, every expert used), bf16 output; one
      step = all 48 layers once.
  80b_gdn_decode  the gated-delta-rule recurrence of the 36 DeltaNet layers
      (16 q/k heads, 32 value heads, 128 x 128 fp32 state per head): one token
      of --sequences sequences through every layer's recurrence.

Steps are captured as HIP graphs and replayed (--eager launches directly).
Prints one JSON line: layer-tokens/s as `value`; the roofline of the dominant
kernel (algorithmic bytes or flops / its dispatch-stamped HIP-event duration);
the HBM traffic of that kernel from rocprofv3 counters when a summary under
profiles/ matches the current kernel sources; and the CPU oracle timed on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from int4_quantized_expert_amd.profiling import load_traffic, traffic_of  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0     # dense fp16/bf16 MFMA peak of MI355X
COPY_PROBE_BYTES = 256 << 20
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (% of 8 TB/s) at 80B-shape decode"

# name: (preset, layers, tokens per call (None = --tokens), routing, output dtype)
WORKLOADS = {
    "80b_stack_decode": ("80b", 48, None, "zipf", "f32"),
    "35b_rotation_decode": ("35b", 40, None, "zipf", "f32"),
    "80b_prefill": ("80b", 48, 2048, "normal", "bf16"),
    # experts streamed from a container file through a 40% HBM slot pool (not the headline metric)
    "35b_int8_store": ("35b_int8", 4, 64, "zipf", "f32"),
    # partial residency at full scale: 40 layers, 4,096 slots (40%), misses from pinned host memory
    "35b_int8_partial": ("35b_int8", 40, 64, "zipf", "f32"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed steps (each through every layer)")
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--tokens", type=int, default=1, help="tokens per call for the decode workloads")
    ap.add_argument("--workload", default="80b_stack_decode", choices=sorted(WORKLOADS) + ["80b_gdn_decode"])
    ap.add_argument("--sequences", type=int, default=64, help="80b_gdn_decode: sequences per call")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chain", action="store_true",
                    help="decode workloads: feed each layer x + y of the layer before (moe_layer_forward_chain), "
                         "layer 0 taking the step's tokens")
    ap.add_argument("--store-path", default="/tmp/moe_35b_int8.store",
                    help="35b_int8_store: container file written (or rewritten) before timing")
    ap.add_argument("--buffered", action="store_true",
                    help="35b_int8_store: read through the page cache instead of O_DIRECT")
    ap.add_argument("--no-extras", action="store_true",
                    help="80b_stack_decode at T = 1: skip the extra figures (chained, uniform routing, T = 8, "
                         "prefill) reported on the same line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first fill and copy a 256 MiB buffer once: the known-size reference that scales "
                         "HBM byte counters read by a profiler")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                          "(the multi-GPU expert-parallel layout is a design note only)"}))
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "launched with WORLD_SIZE > 1; this benchmark is single-GPU"}))
        sys.exit(2)

    import torch

    import int4_quantized_expert_amd as M
    import synth
    from synth import gpu as sgpu

    if args.workload == "35b_int8_store":
        return store_stream(args, torch, M, synth, sgpu)
    if args.workload == "35b_int8_partial":
        return partial_residency(args, torch, M, synth, sgpu)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)             # writes COPY_PROBE_BYTES
        dst.copy_(src)           # reads and writes COPY_PROBE_BYTES
        torch.cuda.synchronize()
        del src, dst
    ctx = Context(args, torch, M, synth, sgpu)
    if args.workload == "80b_gdn_decode":
        r = measure_gdn(ctx, args.sequences, args.steps, args.warmup)
        line = {"metric": "gated-delta-rule decode tokens/s + achieved HBM GB/s (% of 8 TB/s)",
                "value": r["value"], "unit": r["unit"], "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "f32", "data": "synthetic", "config": r["config"], "roofline": r["roofline"]}
        print(json.dumps(line), flush=True)
        return
    head = measure(ctx, args.workload, args.tokens, args.chain, None, args.steps, args.warmup)
    result = head["line"]
    if not args.no_extras and args.workload == "80b_stack_decode" and args.tokens == 1 and not args.chain:
        # further figures on the same line: the chained stack, near-uniform routing (fewer blobs served
        # again from the 256 MB last-level cache than under Zipf routing), T = 8 and the T = 2048 prefill
        extra = {}
        ke, we = min(args.steps, 16), 2
        for name, wl, T, chain, routing, kk in (("chained_t1", "80b_stack_decode", 1, True, None, ke),
                                                ("uniform_t1", "80b_stack_decode", 1, False, "normal", ke),
                                                ("t8", "80b_stack_decode", 8, False, None, ke),
                                                ("prefill_t2048", "80b_prefill", 2048, False, None, 2)):
            r = measure(ctx, wl, T, chain, routing, kk, we)["line"]
            extra[name] = {key: r[key] for key in ("value", "unit", "ms_per_step", "steps", "hbm", "roofline",
                                                   "kernels")}
            extra[name]["config"] = {key: r["config"][key] for key in ("workload", "tokens_per_call", "routing",
                                                                       "chained", "out_dtype")}
        # the gated-delta-rule recurrence of the 36 DeltaNet layers: one
        # sequence, and a batch of 64 sequences
        for B in (1, 64):
            extra[f"gdn_decode_b{B}"] = measure_gdn(ctx, B, ke, we)
        result["extra"] = extra
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(head["geo"], args, head["x_host"], head["r_host"], head["shared_host"],
                                              head["n_layers"], head["XS"], head["T"], head["geo"].shared_bytes,
                                              head["NX"])
    print(json.dumps(result), flush=True)


class Context:
    """Device state shared by the measured configurations: the 43.5 GB pool of
    the 80B stack (or the 35B one) and the per-layer shared-expert buffers."""

    def __init__(self, args, torch, M, synth, sgpu):
        self.args, self.torch, self.M, self.synth, self.sgpu = args, torch, M, synth, sgpu
        self.dev = torch.device("cuda:0")
        self.pools = {}

    def pool(self, preset, n_layers):
        key = (preset, n_layers)
        if key not in self.pools:
            torch, synth, geo = self.torch, self.synth, self.synth.PRESETS[preset]
            E, stride = geo.n_experts, geo.blob_stride
            stream = torch.cuda.current_stream(self.dev)
            self.pools.clear()
            torch.cuda.empty_cache()
            t0 = time.time()
            pool = torch.empty(n_layers * E * stride, dtype=torch.uint8, device=self.dev)
            for l in range(n_layers):
                self.sgpu.fill_blobs(geo, pool.data_ptr() + l * E * stride, E, self.args.seed, l, 0,
                                     stream=stream.cuda_stream)
            shared_host = np.concatenate([synth.make_shared(geo, self.args.seed, l) for l in range(n_layers)])
            shared = torch.from_numpy(shared_host).to(self.dev)
            torch.cuda.synchronize()
            log(f"pool filled in {time.time() - t0:.1f}s: {pool.numel() / 1e9:.2f} GB, {n_layers} layers")
            self.pools[key] = (pool, shared, shared_host)
        return self.pools[key]


def measure(ctx, workload, T_arg, chain_on, routing_over, K, W):
    """Times K steps (after W warm-up steps) of one workload configuration and
    returns the JSON line plus what the CPU baseline needs."""
    args, torch, M, synth = ctx.args, ctx.torch, ctx.M, ctx.synth
    preset, n_layers, T_fixed, routing, out_dt = WORKLOADS[workload]
    routing = routing_over or routing
    geo = synth.PRESETS[preset]
    T = T_fixed or T_arg
    prefill = T_fixed is not None
    S = K + W
    XS = 1 if prefill else S          # distinct token batches per layer
    H, E, k = geo.hidden, geo.n_experts, geo.top_k
    stride = geo.blob_stride
    dev = ctx.dev
    stream = torch.cuda.current_stream(dev)
    pool, shared, shared_host = ctx.pool(preset, n_layers)
    shared_bytes = geo.shared_bytes

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    # prefill: 8 distinct 2048-token batches cycle over the layers (each layer has its own router)
    NX = min(n_layers, 8) if prefill else n_layers
    x_host = np.empty((NX, XS * T, H), dtype=np.uint16)
    r_host = np.empty((n_layers, E, H), dtype=np.uint16)
    # a chain has no normalisation between its MoE layers, and with these synthetic weights a layer's
    # output grows about as |x|^2: from std 0.05 the 48-layer chain turns non-finite after about 10
    # layers, from 0.005 after about 36; from 0.002 every layer stays finite and x changes by about 0.5%
    # per layer (the run below is refused if any output or chained input is not finite)
    x_std = 0.002 if chain_on else 1.0
    for l in range(NX):
        x_host[l] = synth.tokens(geo, args.seed, l, XS * T, std=x_std)
    for l in range(n_layers):
        r_host[l] = (synth.router_zipf(geo, args.seed, l, x_host[l]) if routing == "zipf"
                     else synth.router_normal(geo, args.seed, l))
    x = torch.from_numpy(x_host.view(np.uint8)).to(dev)
    routers = torch.from_numpy(r_host.view(np.uint8)).to(dev)
    # one pool base for the whole stack: layer l's expert e at byte offset (l E + e) stride,
    # so the slot offsets of the deeper layers exceed 2^32 (up to 4.3e10 on the 80B stack)
    slots = (torch.arange(n_layers * E, dtype=torch.int64, device=dev) * stride).reshape(n_layers, E)
    out = torch.empty(n_layers, T, H, dtype=torch.float32 if out_dt == "f32" else torch.bfloat16, device=dev)
    ids = torch.full((XS, n_layers, T, k), -1, dtype=torch.int32, device=dev)
    desc = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, out_dt,
                      pool_bytes=pool.numel())
    ws = torch.zeros(M.workspace_bytes(desc, T), dtype=torch.uint8, device=dev)
    M.workspace_init(ws)
    torch.cuda.synchronize()
    log(f"{workload} T={T} routing={routing} chain={chain_on}: inputs ready in {time.time() - t0:.1f}s")

    act_sz = 2 if geo.act == "bf16" else 4
    r_bytes = E * H * act_sz
    xb = T * H * act_sz
    ob = T * H * out.element_size()
    chain = None
    if chain_on:
        assert not prefill, "--chain is for the decode workloads"
        chain = torch.empty(n_layers * xb, dtype=torch.uint8, device=dev)
    # one moe_stack_forward call per step, which runs all layers in one launch: T = 1, and T <= 8 unchained
    use_stack = not prefill and (T == 1 or (T <= 8 and not chain_on))

    def x_in(l, s):
        if chain is not None and l > 0:
            return chain.data_ptr() + (l - 1) * xb
        return x.data_ptr() + ((l % NX) * XS * T + (s % XS) * T) * H * act_sz

    def layer_call(l, s, strm):
        xs = s % XS
        args_l = (desc, T, x_in(l, s), routers.data_ptr() + l * r_bytes, slots[l], pool.data_ptr(),
                  shared.data_ptr() + l * shared_bytes, out[l])
        if chain is not None:
            M.layer_forward_chain(*args_l, chain.data_ptr() + l * xb, ws, ids[xs, l], None, stream=strm)
        else:
            M.layer_forward(*args_l, ws, ids[xs, l], None, stream=strm)

    def stack_call(s, strm):
        M.stack_forward(desc, n_layers, T, x.data_ptr() + (s % XS) * xb, XS * xb, routers, r_bytes, slots, E * 8,
                        pool, shared, shared_bytes, out, ob, ws, x_chain=chain,
                        chain_stride=xb if chain is not None else 0, topk_ids=ids[s % XS], stream=strm)

    def step(s, strm):
        if use_stack:
            stack_call(s, strm)
        else:
            for l in range(n_layers):
                layer_call(l, s, strm)

    # ---------------------------------------------------------------- timed run
    graphs = []
    if not args.eager:
        for s in range(S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(s, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(s):
        if args.eager:
            step(s, stream.cuda_stream)
        else:
            graphs[s].replay()

    for s in range(W):
        run_step(s)
    torch.cuda.synchronize()
    M.status_check(ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for s in range(W, S):
        run_step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = e0.elapsed_time(e1)
    M.status_check(ws)
    # a timing of inf or NaN activations (which take the top-k's slow tie path) measures nothing real
    if not bool(torch.isfinite(out.float()).all()) or (chain is not None and not bool(
            torch.isfinite(chain.view(torch.bfloat16 if geo.act == "bf16" else torch.float32).float()).all())):
        raise RuntimeError(f"{workload}: non-finite outputs or chained inputs; the timing would not be meaningful")
    ms_per_step = total_ms / K
    layer_tokens = K * n_layers * T
    value = layer_tokens / (total_ms * 1e-3)
    log(f"timed {K} steps: {total_ms:.2f} ms (wall {wall * 1e3:.2f} ms), {ms_per_step * 1e3 / n_layers:.2f} us/layer")
    del graphs

    # algorithmic bytes from the realised routing (distinct experts per layer call)
    ids_h = ids.cpu().numpy()
    steps_timed = [s % XS for s in range(W, S)]
    per_ls = np.array([[len(np.unique(ids_h[xs, l])) for xs in steps_timed] for l in range(n_layers)])
    blob = M.blob_bytes(desc, False)
    fixed = M.blob_bytes(desc, True) + r_bytes + H * act_sz + xb + ob
    bytes_total = float(per_ls.sum() * blob + fixed * per_ls.size)
    bytes_per_layer = bytes_total / per_ls.size
    stack_gbs = bytes_total / (total_ms * 1e-3) / 1e9

    # ---------------------------------------------------------------- per-kernel timing (eager, HIP events)
    # The library attaches a start/end event pair to each kernel dispatch of one call
    # (moe_set_launch_events); the runtime stamps them with that dispatch's execution.
    n_inst = min(8 if not prefill else 2, K)
    calls = []          # (step, layer or None for a whole-stack call)
    for s in range(W, W + n_inst):
        if use_stack:
            calls.append((s, None))
        else:
            calls += [(s, l) for l in range(n_layers)]
    timers = [M.LaunchTimer(16) for _ in calls]
    torch.cuda.synchronize()
    for tm, (s, l) in zip(timers, calls):
        tm.arm()
        if l is None:
            stack_call(s, stream.cuda_stream)
        else:
            layer_call(l, s, stream.cuda_stream)
    torch.cuda.synchronize()
    M.status_check(ws)
    n_k = {t.n_recorded // 2 for t in timers}
    if len(n_k) != 1:
        raise RuntimeError(f"calls launched differing kernel counts: {sorted(n_k)}")
    n_k = n_k.pop()
    durs = np.array([t.kernel_us() for t in timers])                       # [calls, kernels] us
    if use_stack:
        uniq_inst = [per_ls[:, s - W].astype(np.float64) for s, _ in calls]   # per call: one value per layer
    else:
        uniq_inst = [np.array([per_ls[l, s - W]], dtype=np.float64) for s, l in calls]
    kernels = kernel_work(desc, geo, T, n_k, uniq_inst, prefill, out.element_size(), use_stack, n_layers)
    table = []
    for j, (name, nbytes, flops) in enumerate(kernels):
        us = float(durs[:, j].mean())
        row = {"kernel": name, "avg_us": round(us, 3), "min_us": round(float(durs[:, j].min()), 3)}
        if nbytes is not None:
            row["bytes_per_launch"] = round(float(np.mean(nbytes)))
            row["gbs"] = round(float(np.mean(nbytes) / (us * 1e-6) / 1e9), 1)
        if flops is not None:
            row["tflops"] = round(float(np.mean(flops) / (us * 1e-6) / 1e12), 1)
            row["mfma_frac"] = round(row["tflops"] / MFMA_F16_PEAK_TFLOPS, 4)
        table.append(row)
    dom = max(range(n_k), key=lambda j: durs[:, j].mean())
    achieved = table[dom]["gbs"]
    traffic = traffic_of(load_traffic(os.path.join(ROOT, "profiles"), workload, T), table[dom]["kernel"])
    unit_us = float(durs.sum(axis=1).mean())

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if not prefill else "f16",
        "data": "synthetic",
        "config": {
            "workload": workload, "layers": n_layers, "tokens_per_call": T, "hidden": H,
            "experts": E, "top_k": k, "inter": geo.inter, "shared_inter": geo.shared_inter,
            "bits": geo.bits, "group": 64, "scale_dtype": geo.sb, "act_dtype": geo.act, "out_dtype": out_dt,
            "routing": routing, "pool_gb": round(pool.numel() / 1e9, 2), "pool_bases": 1,
            "max_slot_offset": int(slots.max().item()), "graphs": not args.eager,
            "chained": bool(chain_on), "launch": "one per step (all layers)" if use_stack else "per layer",
        },
        "hbm": {
            "algorithmic_bytes_per_layer": round(bytes_per_layer),
            "stack_gbs": round(stack_gbs, 1),
            "stack_frac_of_8tbs": round(stack_gbs / HBM_PEAK_GBS, 4),
            "mean_unique_experts": round(float(per_ls.mean()), 2),
        },
        "roofline": {
            "kernel": table[dom]["kernel"],
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_us": table[dom]["avg_us"],
            "bytes_per_launch": table[dom]["bytes_per_launch"],
        },
        "kernels": table,
        "kernels_sum_us": round(unit_us, 3),
    }
    if "tflops" in table[dom]:
        result["roofline"]["mfma"] = {"achieved": table[dom]["tflops"], "peak": MFMA_F16_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": table[dom]["mfma_frac"]}
    out_info = {"line": result, "geo": geo, "x_host": x_host, "r_host": r_host, "shared_host": shared_host,
                "n_layers": n_layers, "XS": XS, "T": T, "NX": NX}
    del x, routers, out, ws, chain
    torch.cuda.synchronize()
    return out_info


GDN_LAYERS = 36      # three quarters of the 48 layers


def measure_gdn(ctx, B, K, W):
    """One token of B sequences through the gated-delta-rule recurrence of 36
    layers (80B-shaped: 16 q/k heads, 32 value heads, 128 x 128 fp32 state per
    head), one gdn_recurrence_forward call per layer, captured in a HIP graph.
    Returns the figure with the roofline of the recurrence kernel."""
    torch, M = ctx.torch, ctx.M
    from synth.gdn import GDN_PRESETS, gdn_inputs
    p = GDN_PRESETS["80b"]
    nk, nv, dk, dv = p["n_k_heads"], p["n_v_heads"], p["d_k"], p["d_v"]
    desc = M.gdn_desc(nk, nv, dk, dv, act="bf16", out="bf16")
    q, k, v, al, be, st = gdn_inputs(nk, nv, dk, dv, B, 1, ctx.args.seed, "bf16")
    put = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(ctx.dev)
    qd, kd, vd, ad, bd = put(q), put(k), put(v), put(al), put(be)
    st1 = put(st)
    states = torch.empty((GDN_LAYERS,) + tuple(st1.shape), dtype=torch.float32, device=ctx.dev)
    states.copy_(st1.unsqueeze(0).expand_as(states))
    out = torch.empty((GDN_LAYERS, B, 1, nv, dv), dtype=torch.bfloat16, device=ctx.dev)
    stream = torch.cuda.Stream(ctx.dev)

    def step():
        for l in range(GDN_LAYERS):
            M.gdn_forward(desc, B, 1, qd, kd, vd, ad, bd, states[l], out[l], stream=stream)

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    graph = None
    if not ctx.args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
    run = graph.replay if graph is not None else step
    with torch.cuda.stream(stream):
        for _ in range(W):
            run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(K):
            run()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    per_launch_us = ms * 1e3 / GDN_LAYERS
    nbytes = (2 * B * nv * dv * dk * 4          # state read and written
              + 2 * B * nk * dk * 2 + B * nv * dv * 2   # q, k, v (bf16)
              + 2 * B * nv * 4 + B * nv * dv * 2)       # alpha, beta, out (bf16)
    gbs = nbytes / (per_launch_us * 1e-6) / 1e9
    log(f"gdn B={B}: {ms:.4f} ms per step of {GDN_LAYERS} layers, {per_launch_us:.2f} us per launch, {gbs:.0f} GB/s")
    del states, out
    return {
        "value": round(B / (ms * 1e-3), 1), "unit": "tokens/s (36 recurrences each)", "ms_per_step": round(ms, 4),
        "steps": K,
        "config": {"workload": "80b_gdn_decode", "sequences": B, "layers": GDN_LAYERS, "q_k_heads": nk,
                   "v_heads": nv, "d_k": dk, "d_v": dv, "state_dtype": "f32", "act_dtype": "bf16",
                   "out_dtype": "bf16", "graphs": graph is not None},
        "roofline": {"kernel": "k_gdn_recurrence", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_of(load_traffic(os.path.join(ROOT, "profiles"), "80b_gdn_decode", B),
                                           "k_gdn_recurrence"),
                     "avg_us": round(per_launch_us, 3), "bytes_per_launch": nbytes,
                     "timing": "graph of 36 back-to-back launches on one stream / 36"},
    }


def host_ram_gb():
    try:
        with open("/proc/meminfo") as fh:
            for line in fh:
                if line.startswith("MemTotal:"):
                    return round(int(line.split()[1]) / 1e6, 1)
    except OSError:
        pass
    return None


def partial_residency(args, torch, M, synth, sgpu):
    """The 35B int8 layer over 40 layers with an HBM slot pool of 40% of the
    experts (4,096 slots of 3,342,336 B): misses copied from a 34.2 GB pinned
    host store on a copy stream, the router of each call on its own stream,
    the experts on a compute stream, no host wait on the compute (the cache
    orders every slot overwrite after the last reader's event).  Timed for
    both eviction policies (use counts restarting at eviction, and kept), next
    to the same calls on the fully resident pool; sampled layers' outputs are
    compared with the resident run bit for bit."""
    preset, n_layers, T, _, out_dt = WORKLOADS[args.workload]
    geo = synth.PRESETS[preset]
    K, W = args.steps, args.warmup
    H, E, k = geo.hidden, geo.n_experts, geo.top_k
    stride = geo.blob_stride
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cur = torch.cuda.current_stream(dev)
    t0 = time.time()
    total = n_layers * E * stride
    pool = torch.empty(total, dtype=torch.uint8, device=dev)
    for l in range(n_layers):
        sgpu.fill_blobs(geo, pool.data_ptr() + l * E * stride, E, args.seed, l, 0, stream=cur.cuda_stream)
    host = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    host.copy_(pool)
    torch.cuda.synchronize()
    log(f"pool and pinned host store ready in {time.time() - t0:.1f}s: {total / 1e9:.2f} GB each")
    shared = torch.from_numpy(np.concatenate([synth.make_shared(geo, args.seed, l) for l in range(n_layers)])).to(dev)
    S = K + W
    xs = np.stack([synth.tokens(geo, args.seed, l, S * T) for l in range(n_layers)])
    rs = np.stack([synth.router_zipf(geo, args.seed, l, xs[l]) for l in range(n_layers)])
    x = torch.from_numpy(xs.view(np.uint8)).to(dev)
    routers = torch.from_numpy(rs.view(np.uint8)).to(dev)
    n_slots = (n_layers * E * 2) // 5
    slot_pool = torch.empty(n_slots * stride, dtype=torch.uint8, device=dev)
    desc_p = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, out_dt,
                        pool_bytes=n_slots * stride)
    desc_r = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, out_dt, pool_bytes=total)
    ws_r = torch.zeros(M.workspace_bytes(desc_p, T), dtype=torch.uint8, device=dev)
    ws_c = torch.zeros_like(ws_r)
    M.workspace_init(ws_r)
    M.workspace_init(ws_c)
    s_route, s_comp, s_copy = torch.cuda.Stream(dev), torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    sampled = {0, n_layers // 3, 2 * n_layers // 3, n_layers - 1}

    def xp(l, s):
        return x.data_ptr() + (l * S * T + s * T) * H * 2

    def rp(l):
        return routers.data_ptr() + l * E * H * 2

    def sp(l):
        return shared.data_ptr() + l * geo.shared_bytes

    # the fully resident run: timed, and the sampled layers' outputs kept
    ref = {}
    out_r = torch.empty(T, H, dtype=torch.float32, device=dev)
    res_slots = torch.arange(n_layers * E, dtype=torch.int64, device=dev).reshape(n_layers, E) * stride

    def step_resident(s, keep):
        for l in range(n_layers):
            M.layer_forward(desc_r, T, xp(l, s), rp(l), res_slots[l], pool, sp(l), out_r, ws_c)
            if keep and l in sampled:
                ref[(s, l)] = out_r.clone()

    for s in range(W):
        step_resident(s, False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(W, S):
        step_resident(s, True)
    torch.cuda.synchronize()
    dt_res = time.perf_counter() - t1
    M.status_check(ws_c)

    NR = 8      # ring of per-call buffers; an entry is reused after its call's compute_done
    ring = [dict(ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                 wts=torch.empty(T, k, dtype=torch.float32, device=dev),
                 ids_h=torch.empty(T, k, dtype=torch.int32, pin_memory=True),
                 table_h=torch.zeros(E, dtype=torch.int64, pin_memory=True),
                 table_d=torch.empty(E, dtype=torch.int64, device=dev),
                 out=torch.empty(T, H, dtype=torch.float32, device=dev),
                 routed=torch.cuda.Event(), ready=torch.cuda.Event(), done=torch.cuda.Event(), used=False)
            for _ in range(NR)]

    def run_policy(keep_counts):
        cache = M.ExpertCache(n_slots, stride, slot_pool, host, n_layers, E)
        cache.set_policy(keep_counts)
        n_call, checked, equal = 0, 0, 0
        pending = []

        def call(s, l, timed):
            nonlocal n_call
            c = ring[n_call % NR]
            n_call += 1
            if c["used"]:
                c["done"].synchronize()
            c["used"] = True
            with torch.cuda.stream(s_route):
                M.router_topk(desc_p, T, xp(l, s), rp(l), c["ids"], c["wts"], ws_r, stream=s_route)
                c["ids_h"].copy_(c["ids"], non_blocking=True)
                c["routed"].record(s_route)
            c["routed"].synchronize()
            cache.acquire(l, c["ids_h"].numpy(), c["table_h"].numpy(), s_copy, c["ready"])
            with torch.cuda.stream(s_comp):
                s_comp.wait_event(c["routed"])
                s_comp.wait_event(c["ready"])
                c["table_d"].copy_(c["table_h"], non_blocking=True)
                M.experts_forward(desc_p, T, xp(l, s), c["ids"], c["wts"], c["table_d"], slot_pool, sp(l), c["out"],
                                  ws_c, stream=s_comp)
                if timed and l in sampled:
                    pending.append(((s, l), c["out"].clone()))
                c["done"].record(s_comp)
            cache.release(l, c["done"])

        for s in range(W):
            for l in range(n_layers):
                call(s, l, False)
        torch.cuda.synchronize()
        h0, m0, e0 = cache.stats()
        t = time.perf_counter()
        for s in range(W, S):
            for l in range(n_layers):
                call(s, l, True)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        h1, m1, e1 = cache.stats()
        M.status_check(ws_r)
        M.status_check(ws_c)
        for key, o in pending:
            checked += 1
            equal += int(torch.equal(o, ref[key]))
        cache.close()
        hits, misses = h1 - h0, m1 - m0
        log(f"partial residency keep_counts={keep_counts}: {dt / K * 1e3:.1f} ms/step, hit rate "
            f"{hits / max(1, hits + misses):.3f}, {equal}/{checked} sampled calls bitwise equal")
        return {"value": round(K * n_layers * T / dt, 1), "ms_per_step": round(dt / K * 1e3, 3),
                "hits": hits, "misses": misses, "evictions": e1 - e0,
                "hit_rate": round(hits / max(1, hits + misses), 4),
                "miss_gbs": round(misses * stride / dt / 1e9, 2),
                "sampled_calls": checked, "sampled_bitwise_equal": equal}

    kept = run_policy(True)      # the cache's default policy: the headline figure
    lfu = run_policy(False)
    line = {
        "metric": "MoE-layer tokens/s with partial residency (35B int8, 40 layers, 40% of experts in HBM)",
        "value": kept["value"], "unit": "layer-tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": kept["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8 codes, f32 accumulate", "data": "synthetic",
        "config": {"workload": args.workload, "layers": n_layers, "tokens_per_call": T, "experts": E,
                   "top_k": k, "slots": n_slots, "slot_bytes": stride, "pinned_host_store_bytes": total,
                   "host_ram_gb": host_ram_gb(), "routing": "zipf",
                   "sampled_layers": sorted(sampled)},
        "policy_counts_kept": kept,
        "policy_counts_restart": lfu,
        "resident": {"value": round(K * n_layers * T / dt_res, 1), "ms_per_step": round(dt_res / K * 1e3, 3)},
        "timing": "host wall clock around K steps of 40 calls, synchronized on both sides; per call the host waits "
                  "for the router's ids only",
    }
    print(json.dumps(line), flush=True)


def store_stream(args, torch, M, synth, sgpu):
    """Layer calls whose experts come from a container file of fixed-stride
    blobs through a slot pool holding 40% of them: per layer, router + top-k,
    the ids to the host, one positioned read per missed blob into pinned
    staging and its copy into a slot (side stream), then the experts.  Timed
    as whole steps (every layer once), and beside it the same calls on a fully
    resident pool."""
    preset, n_layers, T, _, out_dt = WORKLOADS[args.workload]
    geo = synth.PRESETS[preset]
    K, W = args.steps, args.warmup
    H, E, k = geo.hidden, geo.n_experts, geo.top_k
    stride = geo.blob_stride
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cur = torch.cuda.current_stream(dev)
    t0 = time.time()
    pool = torch.empty(n_layers * E * stride, dtype=torch.uint8, device=dev)
    for l in range(n_layers):
        sgpu.fill_blobs(geo, pool.data_ptr() + l * E * stride, E, args.seed, l, 0, stream=cur.cuda_stream)
    torch.cuda.synchronize()
    st = M.ExpertStore.create(args.store_path, n_layers, E, stride, geo.blob_bytes(geo.inter))
    chunk = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
    host = chunk.numpy()
    for l in range(n_layers):
        chunk.copy_(pool[l * E * stride:(l + 1) * E * stride])
        for e in range(E):
            st.write(l, e, host[e * stride:(e + 1) * stride])
    st.close()
    del chunk, host
    os.sync()
    direct = not args.buffered
    try:
        store = M.ExpertStore(args.store_path, direct=direct)
    except M.MoeError as err:
        log(f"O_DIRECT refused ({err}); reading through the page cache")
        direct = False
        store = M.ExpertStore(args.store_path)
    log(f"store written in {time.time() - t0:.1f}s: {n_layers * E * stride / 1e9:.2f} GB, direct={direct}")
    shared = torch.from_numpy(np.concatenate([synth.make_shared(geo, args.seed, l) for l in range(n_layers)])).to(dev)
    S = K + W
    xs = np.stack([synth.tokens(geo, args.seed, l, S * T) for l in range(n_layers)])
    rs = np.stack([synth.router_zipf(geo, args.seed, l, xs[l]) for l in range(n_layers)])
    x = torch.from_numpy(xs.view(np.uint8)).to(dev)
    routers = torch.from_numpy(rs.view(np.uint8)).to(dev)
    n_slots = (n_layers * E * 2) // 5
    n_staging = 8
    staging = torch.empty(n_staging * stride, dtype=torch.uint8, pin_memory=True)
    slot_pool = torch.empty(n_slots * stride, dtype=torch.uint8, device=dev)
    desc_p = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, out_dt,
                        pool_bytes=n_slots * stride)
    desc_r = M.desc_for(H, E, k, geo.inter, geo.shared_inter, geo.bits, geo.act, geo.sb, out_dt,
                        pool_bytes=E * stride)
    ws = torch.zeros(M.workspace_bytes(desc_p, T), dtype=torch.uint8, device=dev)
    M.workspace_init(ws)
    cache = M.ExpertCache.from_store(n_slots, slot_pool, store, staging, n_staging)
    copy_stream = torch.cuda.Stream(dev)
    ready = torch.cuda.Event()
    done = [torch.cuda.Event() for _ in range(n_layers)]
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    table_h = np.zeros(E, dtype=np.int64)
    table_d = torch.zeros(E, dtype=torch.int64, device=dev)
    out = torch.empty(T, H, dtype=torch.float32, device=dev)
    res_slots = torch.arange(E, dtype=torch.int64, device=dev) * stride

    def xp(l, s):
        return x.data_ptr() + (l * S * T + s * T) * H * 2

    def rp(l):
        return routers.data_ptr() + l * E * H * 2

    def sp(l):
        return shared.data_ptr() + l * geo.shared_bytes

    def step_streamed(s):
        for l in range(n_layers):
            M.router_topk(desc_p, T, xp(l, s), rp(l), ids, wts, ws)
            ids_h = ids.cpu().numpy()
            cache.acquire(l, ids_h, table_h, copy_stream, ready)
            cur.wait_event(ready)
            table_d.copy_(torch.from_numpy(table_h))
            M.experts_forward(desc_p, T, xp(l, s), ids, wts, table_d, slot_pool, sp(l), out, ws)
            done[l].record(cur)
            cache.release(l, done[l])

    def step_resident(s):
        for l in range(n_layers):
            M.layer_forward(desc_r, T, xp(l, s), rp(l), res_slots, pool.data_ptr() + l * E * stride, sp(l), out, ws)

    for s in range(W):
        step_streamed(s)
    torch.cuda.synchronize()
    h0, m0, _ = cache.stats()
    t1 = time.perf_counter()
    for s in range(W, S):
        step_streamed(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    h1, m1, ev1 = cache.stats()
    M.status_check(ws)
    for s in range(W):
        step_resident(s)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for s in range(W, S):
        step_resident(s)
    torch.cuda.synchronize()
    dt_res = time.perf_counter() - t2
    cache.close()
    store.close()
    misses, hits = m1 - m0, h1 - h0
    value = K * n_layers * T / dt
    line = {
        "metric": "MoE-layer tokens/s with experts streamed from a container file (35B int8, 40% of experts in HBM)",
        "value": round(value, 1), "unit": "layer-tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(dt / K * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u8 codes, f32 accumulate", "data": "synthetic",
        "config": {"workload": args.workload, "layers": n_layers, "tokens_per_call": T, "experts": E,
                   "slots": n_slots, "staging_buffers": n_staging, "o_direct": direct,
                   "store_bytes": n_layers * E * stride},
        "stream": {"misses": misses, "hits": hits, "evictions": ev1, "hit_rate": round(hits / max(1, hits + misses), 4),
                   "miss_bytes": misses * stride, "miss_gbs": round(misses * stride / dt / 1e9, 3)},
        "resident": {"value": round(K * n_layers * T / dt_res, 1), "ms_per_step": round(dt_res / K * 1e3, 4)},
        "timing": "host wall clock around K steps, synchronized on both sides (each layer waits for its ids on the host)",
    }
    print(json.dumps(line), flush=True)


def kernel_work(desc, geo, T, n_kernels, uniq, prefill, out_bytes, stack=False, n_layers=1):
    """(name, algorithmic HBM bytes, MFMA flops) of each kernel of one call, per call (lists over calls;
    uniq[c] holds the distinct experts of each layer of call c).  A plane is one matrix of a blob: its
    codes, scales and biases.  Workspace traffic (logits, h, partial rows, exchanged words) is not counted."""
    H, E, I, SI, k = desc.hidden, desc.n_experts, desc.inter, desc.shared_inter, desc.top_k
    sb = 4 if geo.sb == "f32" else 2
    act = 4 if geo.act == "f32" else 2

    def plane(rows, cols):
        return rows * cols * geo.bits // 8 + 2 * rows * (cols // 64) * sb

    p_r, p_s = plane(I, H), plane(SI, H)       # a down plane [H, I] has the same size
    router = E * H * act + T * H * act
    gvec = H * act
    out = T * H * out_bytes
    u = np.array([float(np.sum(v)) for v in uniq])     # distinct experts summed over a call's layers
    nl = np.array([float(len(v)) for v in uniq])       # layers per call
    if prefill:
        pairs = T * k
        table = [
            ("k_pf_router", router * nl, 2.0 * T * E * H * nl),
            ("k_topk", None, None),
            ("k_pf_dispatch", None, None),
            ("k_pf_xprep", (gvec + T * H * act) * nl, None),   # also the shared-expert gates
            ("k_pf_gateup", 2 * p_s * nl + 2 * p_r * u, 4.0 * (pairs * I + T * SI) * H * nl),
            ("k_pf_down", p_s * nl + p_r * u, 2.0 * (pairs * I + T * SI) * H * nl),
            ("k_combine", out * nl, None),
        ]
        return table[:n_kernels]
    if stack:
        name = "k_decode_stack" if T == 1 else "k_decode_stack_t"
        return [(f"{name} (one launch: {n_layers} layers of router, top-k, gate/up, down, ordered combine)",
                 (router + gvec + 3 * p_s + out) * nl + 3 * p_r * u, None)]
    if n_kernels == 1:
        return [("k_decode_a (one launch: router, top-k, gate/up, down, ordered combine)",
                 (router + gvec + 3 * p_s + out) * nl + 3 * p_r * u, None)]
    if n_kernels == 2:
        return [("k_decode_a (router, shared gate/up, top-k, dispatch, routed gate/up)",
                 (router + gvec + 2 * p_s) * nl + 2 * p_r * u, None),
                ("k_decode_b (down projections, ordered combine)", (p_s + out) * nl + p_r * u, None)]
    names = ["k_router_logits", "k_topk", "k_dispatch", "k_gateup", "k_down", "k_combine"]
    nb = [router * nl, None, (gvec + T * H * act) * nl, 2 * p_s * nl + 2 * p_r * u, p_s * nl + p_r * u, out * nl]
    return [(n, b, None) for n, b in zip(names, nb)][:n_kernels]


def cpu_baseline(geo, args, x_host, r_host, shared_host, n_layers, XS, T, shared_bytes, NX):
    """The oracle (float64, unmodified) on a bounded sample: the tokens of the
    timed batches in order, each through every layer, until the time budget
    is spent.  BLAS threads are set explicitly to the cores this process may
    run on; a second, shorter pass with one thread gives the 1-thread figure."""
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        main_leg = _oracle_sample(geo, args, x_host, r_host, shared_host, n_layers, XS, T, shared_bytes, NX,
                                  args.cpu_seconds)
    with threadpool_limits(limits=1):
        one = _oracle_sample(geo, args, x_host, r_host, shared_host, n_layers, XS, T, shared_bytes, NX,
                             max(2.0, args.cpu_seconds / 3))
    done, spent, tokens = main_leg
    done1, spent1, _ = one
    return {
        "value": round(done / spent, 3),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} layer-tokens ({tokens} token(s) of the timed batches from the first, each through "
                  f"layers in order, the last pass possibly partial), {spent:.1f} s of float64 numpy with "
                  f"BLAS threads set to {cores}",
        "one_thread": {"value": round(done1 / spent1, 3), "unit": "tokens/s", "cores": 1,
                       "sample": f"{done1} layer-tokens, {spent1:.1f} s"},
    }


def _oracle_sample(geo, args, x_host, r_host, shared_host, n_layers, XS, T, shared_bytes, NX, budget):
    import synth
    from oracle import moe_oracle as O
    shape = O.LayerShape(geo.hidden, geo.n_experts, geo.top_k, geo.inter, geo.shared_inter, geo.bits,
                         geo.act, geo.sb)
    stride = geo.blob_stride
    pool = np.zeros(geo.n_experts * stride, dtype=np.uint8)
    slots = np.arange(geo.n_experts, dtype=np.int64) * stride
    q0 = (args.warmup % XS) * T          # first token of the first timed batch
    spent, done, tokens = 0.0, 0, 0
    for q in range(q0, XS * T):
        for l in range(n_layers):
            x1 = x_host[l % NX, q: q + 1]
            xs = O.decode_dense(x1, geo.act).reshape(1, -1)
            rs = O.decode_dense(r_host[l], geo.act).reshape(geo.n_experts, -1)
            for e in O.select_topk(O.router_logits(xs, rs)[0], geo.top_k):
                e = int(e)
                synth.fill_blob(geo, geo.inter, synth.blob_key(args.seed, l, e), pool[e * stride:(e + 1) * stride])
            sh = shared_host[l * shared_bytes:(l + 1) * shared_bytes]
            t0 = time.perf_counter()
            O.moe_layer(shape, 1, x1, r_host[l], slots, pool, sh)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget:
                break
        tokens += 1
        if spent >= budget:
            break
    return done, spent, tokens


if __name__ == "__main__":
    main()
