#!/usr/bin/env python3
"""Benchmark of the routed-MoE decode/verify layer on one MI355X.

One step = one ``moe_forward`` (router -> top-k -> union -> gate/up sweep ->
down sweep -> weighted sum + shared blend) over one batch of rows, inputs
resident in HBM.  Workload: the 256-expert shape (h=6144, E=256, top_k=8,
I=Is=2048, sigmoid + correction bias, routed_scaling_factor 2.5, NVFP4
experts), rows=8 independent N(0,1) rows.  Steps cycle over 16 seeded inputs
(so unions differ) and over several device copies of the layer (so no step
finds another step's weights in the 256 MB Infinity Cache).

Prints one JSON line: value = achieved HBM GB/s from algorithmic bytes (each
step's own union size) over the device time of K back-to-back steps, measured
by two HIP events on the launch stream with nothing else enqueued between the
steps.  A second pass of K steps launches every kernel with its own start and
stop events (hipExtLaunchKernel: the kernel's own execution, nothing
enqueued between kernels) and gives each stage's average kernel duration: the
dominant kernel's roofline figure.  Also reports, in the same line:
  staged_pass_per_step  p10 / median / p90 of each step's device time (first
                        kernel start to last kernel stop) and GB/s in that pass
                        (above us_per_step: its events widen the kernel gaps)
  sweep                 rows=1..8 at the same shape
  configs               every layer configuration at its own rows (also replayed
                        from a captured HIP graph: device time without launch cost)
  union_vs_token_major  the union sweep against moe_forward_token_major on the
                        same inputs (independent rows 1..8, correlated K=2..4)
  union_past_8_rows_vs_8_row_sub_chunks
                        12 and 16 rows in one union against 8-row sub-chunks
  ep_share              one GPU's expert-parallel share (8 ranges of 32 experts)
  read_ceiling_gbps     moe_read_probe's streaming-read rate over 4 GiB
  cpu_baseline          the CPU oracle timed on a bounded sample (a reference
                        point, not the target)
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

METRIC = "routed-MoE layer µs/step + achieved HBM GB/s (% peak), rows=1..8, NVFP4"

# HBM traffic of the gate/up sweep at rows=8 per algorithmic byte, measured with
# rocprofv3 --pmc over 119 dispatches (FETCH_SIZE x 2.000 + WRITE_SIZE; the factor comes
# from a plain 1 GiB copy, see profiles/gateup_sweep_e256_rows1_2_4_8_pmc.md).  Valid only
# for the kernel sources it was taken on; the roofline's traffic is this ratio times the
# launch's algorithmic bytes.
TRAFFIC_SOURCES = ('mixture_experts_decode_gate_amd/csrc/moe_gateup.h', 'mixture_experts_decode_gate_amd/csrc/moe_common.h',
                   'mixture_experts_decode_gate_amd/csrc/moe_device.h', 'mixture_experts_decode_gate_amd/csrc/moe_gateup_rows_5_8.hip')
TRAFFIC_MEASURED = {"sources_sha256_16": "93f46c421527a6ff", "rows": 8, "gate_up_traffic_per_byte": 1.0023}
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "c4_e256_prefill8"
N_INPUTS = 16


def measured_traffic(rows: int, bytes_per_launch: float):
    """Counter-measured HBM bytes per launch of the dominant kernel (the measured
    traffic per algorithmic byte times this launch's algorithmic bytes), or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != TRAFFIC_MEASURED["sources_sha256_16"] or rows != TRAFFIC_MEASURED["rows"]:
        return None
    return int(round(TRAFFIC_MEASURED["gate_up_traffic_per_byte"] * bytes_per_launch))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(n: int, k: int) -> int:
    return n * k // 2 + n * k // 16 + 4


def step_bytes(shape, rows: int, U: int) -> dict:
    """Algorithmic HBM bytes of one step, split by stage."""
    h, E, k, I, Is = shape.hidden, shape.num_experts, shape.top_k, shape.moe_inter, shape.shared_inter
    pairs = rows * k
    # route: router rows + gate vector + x, logits written and read back, bias, ids + weights out
    route = (4 * E * h + 4 * h + 2 * rows * h + 8 * rows * (E + 1) + (4 * E if shape.route_kind == 1 else 0)
             + 8 * pairs)
    gateup = 2 * U * expert_bytes(I, h) + 2 * expert_bytes(Is, h) + 2 * rows * h + 2 * (pairs * I + rows * Is)
    down = U * expert_bytes(h, I) + expert_bytes(h, Is) + 2 * (pairs * I + rows * Is) + 4 * (pairs + rows) * h
    blend = 4 * (pairs + rows) * h + 2 * rows * h + 8 * pairs
    # whole layer: weights + router + bias + gate vector + x in + out
    layer = (U * 3 * expert_bytes(I, h) + 3 * expert_bytes(Is, h) + 4 * E * h
             + (4 * E if shape.route_kind == 1 else 0) + 4 * h + 4 * rows * h)
    # down sweep and blend in one stage: weights, activations, out (plus the weights
    # and gates of the blend); the expert outputs are an intermediate of the two-kernel form
    down_blend = U * expert_bytes(h, I) + expert_bytes(Is, h) + 2 * (pairs * I + rows * Is) + 2 * rows * h + 8 * pairs
    return dict(layer=layer, route=route, gate_up_sweep=gateup, down_sweep=down, blend=blend,
                down_sweep_blend=down_blend)


def build_layers(shape, n_layers: int):
    import torch
    import mixture_experts_decode_gate_amd as moe
    from mixture_experts_decode_gate_amd.device import DeviceLayer
    import synth
    t0 = time.time()
    w = synth.layer_weights(shape, materialise=True, threads=16)
    log(f"[bench] generated {shape.name} weights in {time.time() - t0:.1f}s")
    cfg = moe.MoeConfig.from_shape(shape)
    base = DeviceLayer(cfg, w.router_w, w.bias, w.shared_gate_vec, w.shared, w.expert)
    w._experts.clear()
    layers = [base] + [base.clone() for _ in range(n_layers - 1)]
    torch.cuda.synchronize()
    log(f"[bench] {n_layers} device copies of {base.nbytes() / 1e9:.2f} GB ready after {time.time() - t0:.1f}s")
    return cfg, layers


def union_sizes(cfg, layers, xs, ws):
    """Union size of each input (one moe_forward per input; the inputs cycle
    over the layer copies so every copy has been run once before timing)."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    L = moe.moe_workspace_layout(cfg)
    out = torch.empty_like(xs[0])
    us = []
    for i in range(max(len(xs), len(layers))):
        moe.moe_forward(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], out, ws)
        torch.cuda.synchronize()
        if i < len(xs):
            us.append(int(ws[L.union_count:L.union_count + 4].cpu().numpy().view(np.int32)[0]))
    return us


def settle(cfg, layers, xs, ws, ms):
    """Untimed steps for ``ms`` milliseconds of host time, back to back.  After
    the setup (weight upload, one step per input with a host read-back each),
    the first few tens of steps run about 5% slower than the steady state
    while the device's clocks settle; a timed region of 20 steps started then
    would measure the transition, not the layer."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    out = torch.empty_like(xs[0])
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < ms / 1e3:
        moe.moe_forward(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], out, ws)
        i += 1
    torch.cuda.synchronize()
    return i


def timed_run(cfg, layers, xs, us, shape, rows, steps, warmup, ws, stage_events=False, token_major=False):
    """K back-to-back steps between two events on the launch stream.  With
    stage_events, every step is launched through moe_forward_timed, whose
    kernels each record a start and a stop event (their own execution): the
    per-stage kernel durations for the roofline.  With token_major, every step
    runs moe_forward_token_major (no union); its bytes are still counted with
    the union's U, so GB/s compares the two paths on the same useful work."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    from mixture_experts_decode_gate_amd.hip_events import HipEvent
    fwd = moe.moe_forward_token_major if token_major else moe.moe_forward
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)
    out = torch.empty_like(xs[0])
    nst = moe.moe_num_stages()
    traced = list(range(steps)) if stage_events else []
    events = {i: [HipEvent() for _ in range(2 * nst)] for i in traced}
    start, end = HipEvent(), HipEvent()
    # Barrier before the warm-up, then the warm-up steps and the timed steps
    # back to back: the start event is taken when the device finishes the last
    # warm-up step, so the device never idles before the timed steps (an idle
    # gap measurably slows the next steps while the clocks recover).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup):
        fwd(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], out, ws)
    start.record(sh)
    for i in range(steps):
        lay, xi = layers[i % len(layers)], i % len(xs)
        if i in events:
            moe.moe_forward_timed(cfg, lay.weights, xs[xi], out, ws, events[i])
        else:
            fwd(cfg, lay.weights, xs[xi], out, ws)
    end.record(sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_ms(end)
    sbytes = [step_bytes(shape, rows, us[i % len(xs)]) for i in range(steps)]
    res = dict(total_ms=total_ms, host_wall_ms=wall * 1e3, us_per_step=total_ms * 1e3 / steps,
               layer_bytes=sum(b["layer"] for b in sbytes),
               mean_union=float(np.mean([us[i % len(xs)] for i in range(steps)])))
    res["gbps"] = res["layer_bytes"] / (total_ms * 1e-3) / 1e9
    if traced:
        names = moe.moe_stage_names()
        stage = {}
        for s, name in enumerate(names):
            d = [events[i][2 * s].elapsed_ms(events[i][2 * s + 1]) for i in traced]
            b = sum(sbytes[i][name] for i in traced)
            stage[name] = dict(avg_us=float(np.mean(d)) * 1e3, gbps=b / (sum(d) * 1e-3) / 1e9,
                               bytes_per_launch=b / len(traced), launches=len(traced))
        res["stages"] = stage
        # Per step: the first kernel's start to the last kernel's stop (device
        # time of the whole step), and the GB/s of that step's own bytes.
        step_us = np.array([events[i][0].elapsed_ms(events[i][2 * nst - 1]) * 1e3 for i in traced])
        step_gbps = np.array([sbytes[i]["layer"] for i in traced]) / (step_us * 1e-6) / 1e9
        res["per_step"] = dict(us_p10_p50_p90=[round(float(v), 2) for v in np.percentile(step_us, [10, 50, 90])],
                               gbps_p10_p50_p90=[round(float(v), 1) for v in np.percentile(step_gbps, [10, 50, 90])],
                               steps=len(traced))
    return res


def union_vs_subchunks(cfg, layers, shape, K, steps, ws, settle_ms, sub_rows=8):
    """K rows as one moe_forward (one union over all K rows' experts) against
    the same rows as sub-chunks of ``sub_rows`` rows, one moe_forward each
    (each sub-chunk dedups only its own experts).  Same inputs, same layer
    copies; µs per K rows and the experts each form streams."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    import synth
    from mixture_experts_decode_gate_amd.hip_events import HipEvent
    L = moe.moe_workspace_layout(cfg)
    xs = [torch.from_numpy(synth.activations(shape, s, rows=K).view(np.int16)).cuda() for s in range(N_INPUTS)]
    out = torch.empty_like(xs[0])
    chunks = [(r0, min(K, r0 + sub_rows)) for r0 in range(0, K, sub_rows)]

    def u_of():
        torch.cuda.synchronize()
        return int(ws[L.union_count:L.union_count + 4].cpu().numpy().view(np.int32)[0])
    u_one, u_sub = [], []
    for i, x in enumerate(xs):
        moe.moe_forward(cfg, layers[i % len(layers)].weights, x, out, ws)
        u_one.append(u_of())
        tot = 0
        for a, b in chunks:
            moe.moe_forward(cfg, layers[i % len(layers)].weights, x[a:b], out[a:b], ws)
            tot += u_of()
        u_sub.append(tot)
    sh = int(torch.cuda.current_stream().cuda_stream)
    res = {}
    for mode in ("one_union", "sub_chunks"):
        settle(cfg, layers, xs, ws, settle_ms)
        for i in range(10):  # warm-up, back to back with the timed steps
            moe.moe_forward(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], out, ws)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sh)
        for i in range(steps):
            lay, x = layers[i % len(layers)], xs[i % len(xs)]
            if mode == "one_union":
                moe.moe_forward(cfg, lay.weights, x, out, ws)
            else:
                for a, b in chunks:
                    moe.moe_forward(cfg, lay.weights, x[a:b], out[a:b], ws)
        e1.record(sh)
        torch.cuda.synchronize()
        res[mode] = e0.elapsed_ms(e1) * 1e3 / steps
    return dict(workload=shape.name, rows=K, sub_chunk_rows=sub_rows, experts_one_union=float(np.mean(u_one)),
                experts_sub_chunks=float(np.mean(u_sub)), one_union_us=round(res["one_union"], 2),
                sub_chunks_us=round(res["sub_chunks"], 2), speedup=round(res["sub_chunks"] / res["one_union"], 4),
                expert_streams_saved=round(1 - np.mean(u_one) / np.mean(u_sub), 4))


def config_runs(steps, main_shape, main_layers, main_cfg, ws_main, settle_ms):
    """µs/step and GB/s of moe_forward on each configuration at its own rows.
    Every layer is copied on the device until a pass over the copies moves more
    than 1 GB of the bytes a step touches, so steps read HBM rather than the
    256 MB Infinity Cache.  The 256-expert configurations reuse the main
    layer's copies."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    import synth
    out = []
    for name in synth.CONFIG_ORDER:
        shape = synth.CONFIGS[name]
        same = (shape.hidden, shape.num_experts, shape.moe_inter) == (main_shape.hidden, main_shape.num_experts,
                                                                      main_shape.moe_inter)
        if same:
            cfg, layers, ws = main_cfg, main_layers, ws_main
        else:
            per_step = step_bytes(shape, shape.rows, min(shape.top_k * shape.rows, shape.num_experts))["layer"]
            n_copies = int(min(64, max(2, -(-(1 << 30) // per_step))))
            cfg, layers = build_layers(shape, n_copies)
            ws = torch.zeros(moe.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        xs = [torch.from_numpy(synth.activations(shape, s).view(np.int16)).cuda() for s in range(N_INPUTS)]
        us = union_sizes(cfg, layers, xs, ws)
        settle(cfg, layers, xs, ws, settle_ms)
        r = timed_run(cfg, layers, xs, us, shape, shape.rows, steps, 10, ws)
        g_us = graph_step_us(cfg, layers, xs, ws)
        out.append(dict(config=name, rows=shape.rows, mean_union=round(r["mean_union"], 3), layer_copies=len(layers),
                        us_per_step=round(r["us_per_step"], 2), gbps=round(r["gbps"], 1),
                        pct_peak=round(100 * r["gbps"] / HBM_PEAK_GBPS, 2), graph_us_per_step=round(g_us, 2)))
        log(f"[bench] config {name}: {r['us_per_step']:.1f} us/step, {r['gbps']:.0f} GB/s, U={r['mean_union']:.2f}; "
            f"graph replay {g_us:.1f} us/step")
        if not same:
            del layers, ws
            torch.cuda.empty_cache()
    return out


def graph_step_us(cfg, layers, xs, ws, n_steps=32, reps=10):
    """µs per step with n_steps moe_forward calls (cycling inputs and layer
    copies) captured once in a HIP graph and replayed: the device-side step time
    without per-call host launch cost."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    from mixture_experts_decode_gate_amd.hip_events import HipEvent
    outs = [torch.empty_like(xs[0]) for _ in range(2)]
    for i in range(4):  # warm-up outside capture
        moe.moe_forward(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], outs[i % 2], ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_steps):
            moe.moe_forward(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], outs[i % 2], ws)
    g.replay()
    torch.cuda.synchronize()
    sh = int(torch.cuda.current_stream().cuda_stream)
    e0, e1 = HipEvent(), HipEvent()
    e0.record(sh)
    for _ in range(reps):
        g.replay()
    e1.record(sh)
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) * 1e3 / (reps * n_steps)


def read_ceiling(nbytes=4 << 30, reps=5):
    """Streaming-read rate of moe_read_probe over a buffer larger than the
    Infinity Cache: the achievable ceiling for the weight sweeps' reads."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    from mixture_experts_decode_gate_amd.hip_events import HipEvent
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.zeros(moe.moe_read_probe_sink_words(), dtype=torch.int32, device="cuda")
    sh = int(torch.cuda.current_stream().cuda_stream)
    moe.moe_read_probe(src, sink)
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record(sh)
    for _ in range(reps):
        moe.moe_read_probe(src, sink)
    e1.record(sh)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    del src, sink
    return nbytes / (ms * 1e-3) / 1e9


def ep_shares(cfg, layers, xs, shape, rows, n_ranks, steps, ws, settle_ms):
    """Time moe_forward_ep_partial for each of n_ranks equal expert ranges."""
    import torch
    import mixture_experts_decode_gate_amd as moe
    from mixture_experts_decode_gate_amd.hip_events import HipEvent
    E = shape.num_experts
    L = moe.moe_workspace_layout(cfg)
    partial = torch.empty((rows, shape.hidden), dtype=torch.float32, device="cuda")
    sh = int(torch.cuda.current_stream().cuda_stream)
    out = []
    for g in range(n_ranks):
        lo, hi = g * E // n_ranks, (g + 1) * E // n_ranks
        us = []
        for x in xs:
            moe.moe_forward_ep_partial(cfg, layers[0].weights, x, partial, lo, hi, ws)
            torch.cuda.synchronize()
            us.append(int(ws[L.union_count:L.union_count + 4].cpu().numpy().view(np.int32)[0]))
        # settled clocks, then the warm-up back to back with the timed steps
        settle(cfg, layers, xs, ws, settle_ms)
        for i in range(10):
            moe.moe_forward_ep_partial(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], partial, lo, hi, ws)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sh)
        for i in range(steps):
            moe.moe_forward_ep_partial(cfg, layers[i % len(layers)].weights, xs[i % len(xs)], partial, lo, hi, ws)
        e1.record(sh)
        torch.cuda.synchronize()
        t_us = e0.elapsed_ms(e1) * 1e3 / steps
        mean_u = float(np.mean([us[i % len(xs)] for i in range(steps)]))
        nbytes = step_bytes(shape, rows, mean_u)["layer"]
        out.append(dict(lo=lo, hi=hi, mean_local_union=round(mean_u, 3), us_per_step=round(t_us, 2),
                        gbps=round(nbytes / (t_us * 1e-6) / 1e9, 1)))
    return dict(rows=rows, ranks=n_ranks, ranges=out, slowest_us=max(r["us_per_step"] for r in out),
                note="per-range time of moe_forward_ep_partial (local union + shared expert + fp32 partial); "
                     "all-reduce and combine not included")


def copy_reference(nbytes=2 << 30, reps=10):
    """Achieved bandwidth of a plain device copy (read + write), for context."""
    import torch
    from mixture_experts_decode_gate_amd.hip_events import HipEvent
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    sh = int(torch.cuda.current_stream().cuda_stream)
    e0, e1 = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    e0.record(sh)
    for _ in range(reps):
        b.copy_(a)
    e1.record(sh)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9, ms


def cpu_baseline(shape, steps=(0, 1, 2)):
    """The oracle as it stands, on a bounded sample of the workload: every row
    of the steps in ``steps`` (about 14 s on a 16-core host).  Rate = the
    sample's algorithmic bytes (each step's own union) / oracle time."""
    import synth
    from oracle.layer import moe_layer_from
    from oracle.route import route
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    w = synth.layer_weights(shape)
    dt, nbytes, unions = 0.0, 0, []
    for step in steps:
        x = synth.activations(shape, step)
        _, ids, _ = route(x, w.router_w, w.bias, shape.route_kind, shape.top_k, shape.norm_topk_prob,
                          shape.routed_scaling_factor)
        need = sorted(set(int(e) for e in ids.reshape(-1)))
        # weight generation is not timed: the oracle's input is the decoded layer's storage
        w._experts = {(e, p): synth.expert_tensor(shape, e, p) for e in need for p in range(3)}
        w.lazy = False
        t0 = time.perf_counter()
        moe_layer_from(w, x)
        dt += time.perf_counter() - t0
        nbytes += step_bytes(shape, shape.rows, len(need))["layer"]
        unions.append(len(need))
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
                sample=f"{shape.name} steps {list(steps)}, all {shape.rows} rows (unions {unions} + shared), "
                       f"float64 numpy oracle, {dt:.2f} s",
                seconds=dt, us_per_step=dt * 1e6 / len(steps))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rows", type=int, default=8)
    ap.add_argument("--layers", type=int, default=8, help="device copies of the layer cycled by the steps")
    ap.add_argument("--sweep-steps", type=int, default=100)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="untimed steps before the first timed region, in host milliseconds")
    ap.add_argument("--sweep-settle-ms", type=float, default=20.0,
                    help="untimed steps before each later timed pass (after its setup's read-backs)")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="configuration of the headline run (profiling other configurations)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true", help="short run for rocprofv3: no sweep, no CPU leg")
    ap.add_argument("--copy-calib", action="store_true", help="only run the plain copy kernel (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path in this library "
              "(an expert-parallel split would give each GPU E/N experts and one all-reduce of the output)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_decode_gate_amd as moe
    import synth
    moe.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calib:
        gbps, ms = copy_reference(1 << 30, reps=5)
        log(f"[bench] copy 1 GiB: {ms:.3f} ms, {gbps:.0f} GB/s (read+write)")
        return

    if args.profile:
        args.no_sweep, args.no_cpu = True, True

    base_shape = synth.CONFIGS[args.workload]
    shape = base_shape.with_rows(args.rows) if args.rows != base_shape.rows else base_shape
    cfg, layers = build_layers(base_shape, args.layers)
    ws = torch.zeros(moe.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")

    def inputs(rows):
        return [torch.from_numpy(synth.activations(base_shape, s, rows=rows).view(np.int16)).cuda()
                for s in range(N_INPUTS)]

    xs = inputs(args.rows)
    us = union_sizes(cfg, layers, xs, ws)
    log(f"[bench] unions over {N_INPUTS} inputs: {us}")
    settle_steps = settle(cfg, layers, xs, ws, args.settle_ms)
    log(f"[bench] {settle_steps} untimed settle steps ({args.settle_ms:.0f} ms)")
    res = timed_run(cfg, layers, xs, us, shape, args.rows, args.steps, args.warmup, ws)
    log(f"[bench] rows={args.rows}: {res['us_per_step']:.1f} us/step, {res['gbps']:.0f} GB/s")
    # the same K steps again, every kernel with its own start and stop events
    staged = timed_run(cfg, layers, xs, us, shape, args.rows, args.steps, args.warmup, ws, stage_events=True)
    log("[bench] kernel durations: " + ", ".join(f"{k} {v['avg_us']:.2f} us" for k, v in staged["stages"].items()))

    sweep = []
    if not args.no_sweep:
        for R in range(1, 9):
            xr = inputs(R)
            ur = union_sizes(cfg, layers, xr, ws)
            settle(cfg, layers, xr, ws, args.sweep_settle_ms)
            r = timed_run(cfg, layers, xr, ur, base_shape.with_rows(R), R, args.sweep_steps, 10, ws)
            sweep.append(dict(rows=R, us_per_step=round(r["us_per_step"], 2), gbps=round(r["gbps"], 1),
                              frac=round(r["gbps"] / HBM_PEAK_GBPS, 4), mean_union=r["mean_union"]))
            log(f"[bench] sweep rows={R}: {r['us_per_step']:.1f} us/step {r['gbps']:.0f} GB/s U={r['mean_union']:.2f}")

    # Union sweep vs token-major (every (row, expert) pair streamed on its own),
    # on the same inputs: independent rows at rows=1..8, and the correlated
    # rows=4 verify workload whose mean union is the pages' K=4 figure.
    ab = []
    if not args.no_sweep:
        c3 = synth.CONFIGS["c3_e256_verify4"]
        cases = [(base_shape.with_rows(R), R, "independent") for R in range(1, 9)] + [
            (c3.with_rows(K) if K != c3.rows else c3, K, "correlated a=0.58") for K in (2, 3, 4)]
        for shp, R, kind in cases:
            xr = [torch.from_numpy(synth.activations(shp, s, rows=R).view(np.int16)).cuda() for s in range(N_INPUTS)]
            ur = union_sizes(cfg, layers, xr, ws)
            settle(cfg, layers, xr, ws, args.sweep_settle_ms)
            a = timed_run(cfg, layers, xr, ur, shp, R, args.sweep_steps, 10, ws)
            settle(cfg, layers, xr, ws, args.sweep_settle_ms)
            b = timed_run(cfg, layers, xr, ur, shp, R, args.sweep_steps, 10, ws, token_major=True)
            ab.append(dict(rows=R, rows_kind=kind, mean_union=a["mean_union"], pairs=R * shp.top_k,
                           union_us=round(a["us_per_step"], 2), token_major_us=round(b["us_per_step"], 2),
                           speedup=round(b["us_per_step"] / a["us_per_step"], 4),
                           expert_streams_saved=round(1 - a["mean_union"] / (R * shp.top_k), 4)))
            log(f"[bench] A/B rows={R} ({kind}): union {a['us_per_step']:.1f} us (U={a['mean_union']:.2f}) vs "
                f"token-major {b['us_per_step']:.1f} us ({R * shp.top_k} streams): x{ab[-1]['speedup']:.3f}")

    # More than 8 rows in one call (the union over two 64-slot tiles) against
    # the pages' 8-row sub-chunks, on correlated verify rows: K = 12 at the
    # 256-expert shape (hidden 6144 stages at most 12 rows of x), K = 12 and 16
    # at the 128-expert shape (hidden 4096).
    wide = []
    if not args.no_sweep:
        c3 = synth.CONFIGS["c3_e256_verify4"]
        wide.append(union_vs_subchunks(cfg, layers, c3.with_rows(12), 12, args.sweep_steps, ws,
                                       args.sweep_settle_ms))
        log(f"[bench] rows>8: {wide[-1]}")
        c2 = synth.CONFIGS["c2_e128_verify2"]
        per_step = step_bytes(c2, 16, 16 * c2.top_k)["layer"]
        cfg2, layers2 = build_layers(c2, int(min(16, max(2, -(-(1 << 30) // per_step)))))
        ws2 = torch.zeros(moe.moe_workspace_bytes(cfg2), dtype=torch.uint8, device="cuda")
        for K in (12, 16):
            wide.append(union_vs_subchunks(cfg2, layers2, c2.with_rows(K), K, args.sweep_steps, ws2,
                                           args.sweep_settle_ms))
            log(f"[bench] rows>8: {wide[-1]}")
        del layers2, ws2
        torch.cuda.empty_cache()

    configs = [] if args.no_sweep else config_runs(args.sweep_steps, base_shape, layers, cfg, ws,
                                                   args.sweep_settle_ms)

    # One GPU's expert-parallel share at the real shape: the layer's 256
    # experts split over 8 GPUs, each sweeping its 32-expert range of the
    # union (plus the shared expert) and writing an fp32 partial.  Each range is
    # timed on its own; the slowest sets an 8-GPU step (the all-reduce is not
    # part of the library and not timed).
    ep = None
    if not args.no_sweep:
        ep = ep_shares(cfg, layers, xs, shape, args.rows, 8, args.sweep_steps, ws, args.sweep_settle_ms)
        log(f"[bench] EP share rows={args.rows}, 8 ranges of {shape.num_experts // 8} experts: "
            f"local unions {[r['mean_local_union'] for r in ep['ranges']]}, "
            f"us {[r['us_per_step'] for r in ep['ranges']]}")

    copy_gbps, _ = copy_reference()
    read_gbps = read_ceiling()
    log(f"[bench] streaming-read ceiling {read_gbps:.0f} GB/s; layer at {100 * res['gbps'] / read_gbps:.1f}% of it")
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(shape)
        log(f"[bench] cpu oracle: {cpu['sample']}: {cpu['value']:.3f} GB/s")

    dom = "gate_up_sweep"
    st = staged["stages"][dom]
    line = {
        "metric": METRIC,
        "value": round(res["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["us_per_step"] / 1e3, 5),
        "us_per_step": round(res["us_per_step"], 2),
        "pct_peak": round(100 * res["gbps"] / HBM_PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{base_shape.name}: h={base_shape.hidden} E={base_shape.num_experts} "
                               f"top_k={base_shape.top_k} I={base_shape.moe_inter} Is={base_shape.shared_inter} "
                               f"rows={args.rows} "
                               + ("sigmoid+bias rsf=%g" % base_shape.routed_scaling_factor
                                  if base_shape.route_kind == synth.ROUTE_SIGMOID_BIAS else "softmax")
                               + f" NVFP4 experts, {base_shape.x_kind} rows",
                   "rows": args.rows, "layer_copies": args.layers, "inputs": N_INPUTS,
                   "settle_steps": settle_steps,
                   "mean_union": res["mean_union"]},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(st["gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(st["gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.rows, st["bytes_per_launch"]),
                     "avg_launch_us": round(st["avg_us"], 2), "bytes_per_launch": int(st["bytes_per_launch"]),
                     "timed_launches": st["launches"],
                     "timing": "kernel start/stop events (hipExtLaunchKernel) in a second pass of the same steps"},
        "stages_us": {k: round(v["avg_us"], 2) for k, v in staged["stages"].items()},
        "stages_gbps": {k: round(v["gbps"], 1) for k, v in staged["stages"].items()},
        "staged_pass_us_per_step": round(staged["us_per_step"], 2),
        "staged_pass_per_step": dict(staged["per_step"],
                                     timing="first kernel start to last kernel stop of each step in the "
                                            "event-timed pass (its event records widen the gaps between "
                                            "kernels, so these read above us_per_step)"),
        "copy_gbps": round(copy_gbps, 1),
        "read_ceiling_gbps": round(read_gbps, 1),
        "pct_of_read_ceiling": round(100 * res["gbps"] / read_gbps, 2),
        "sweep": sweep,
        "union_vs_token_major": ab,
        "union_past_8_rows_vs_8_row_sub_chunks": wide,
        "configs": configs,
        "ep_share": ep,
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
