#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X: routed, block-quantized experts.

A step is one pass of the whole layer path over one batch of synthetic input:
moe_route_dispatch (moe_route + moe_dispatch; one launch for batches of up to
8 tokens) -> moe_expert_ffn -> moe_combine (for up to 4 tokens the last two as
moe_expert_ffn_combine, whose down kernel also merges), or with --separate-calls the four
calls moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine (for the
48-layer workloads: all 48 layers in sequence).  Inputs are resident in HBM before the
timed region.  The K timed steps (and the W warm-up steps) are captured into
one HIP graph each and replayed once, bracketed by stream synchronisation and
HIP events on the launch stream.  Per-call GPU durations come from one more
graph per call (back-to-back launches of that call over consecutive steps'
inputs), timed with HIP events on the same stream.

With no --workload the run covers the metric's three regimes: workload 1
(the headline line: value, roofline, cpu_baseline) and, under "regimes",
workloads 2 and 3, each with its own tokens/s, roofline and cpu_baseline,
timed the same way with the same --steps / --warmup.

Workloads:
  1  decode, T=1, d=2048, f=768, E=512, top-10 + shared, Q2 block-32, 1 layer
     (16 copies of the layer at distinct HBM addresses, cycled per step, and a
     fresh x per step, so the selected experts are not cache-resident)
  2  MTP verify, T=4 through 48 layers, Q3 block-32, Zipf(1.1) router bias
  3  prefill, T=8192, Q2, 1 layer           4  prefill, T=8192, Q3, 48 layers,
                                               Zipf(1.3) router bias
  5, 6  the "coder" variant (E=256 routed experts): decode T=1 as 1, prefill
        T=8192 as 3
--tail-skip RANK times the lossy route tail-skip variant (moe_dispatch_tail_skip)
and reports the pairs kept and the output's deviation from the full layer;
--overlap-shared runs the shared expert (moe_shared_ffn) on a second stream
beside moe_route_dispatch, then moe_routed_ffn, joining before moe_combine
(the fork and join are captured in the graph); --tokens T overrides the
workload's batch size.

Decode workloads report the expert FFN call against HBM bandwidth (bytes of
the distinct experts selected + activations); prefill workloads against the
dense fp16/bf16 matrix-core peak (2*M*N*K of the expert GEMMs).

Prints one JSON line on stdout.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FUSE_COMBINE_TMAX = 4          # moe_expert_ffn_combine merges inside the down kernel up to here
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix
METRIC = "MoE-layer tokens/s (decode T=1/4, prefill 8192); % HBM BW or % MFMA peak"

# HBM bytes per expert-FFN call of the step (moe_expert_ffn_combine for
# workloads 1 and 2, moe_expert_ffn for workloads 3 and 4), from two rocprofv3
# --pmc runs (FETCH_SIZE, WRITE_SIZE; each scaled by what it reads for a plain
# 1 GiB copy: 2.0 and 1.0), keyed by workload.  Each figure is tied to a hash of
# the kernel sources it was taken on and is reported as null once those
# sources change.
TRAFFIC = {
    1: (("common.h", "ffn_small.hip"), "0f3102109453b0af", 20210893),
    2: (("common.h", "ffn_small.hip"), "0f3102109453b0af", 49021881),
    3: (("common.h", "ffn_prefill.hip"), "9ef069ee536495f6", 2501741976),
    4: (("common.h", "ffn_prefill.hip"), "9ef069ee536495f6", 2202330775),
}


def traffic_for(wid):
    import hashlib
    if wid not in TRAFFIC:
        return None
    files, digest, nbytes = TRAFFIC[wid]
    m = hashlib.sha256()
    for fn in files:
        with open(os.path.join(ROOT, "quantized_moe_route_amd", "csrc", fn), "rb") as fh:
            m.update(fh.read())
    return float(nbytes) if m.hexdigest()[:16] == digest else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(w) -> int:
    """Packed bytes of one expert (gate + up + down)."""
    import synth
    s = sum(synth.plane_sizes(w.fmt, r, K)["lo"] + synth.plane_sizes(w.fmt, r, K)["hi"] +
            2 * (synth.plane_sizes(w.fmt, r, K)["scale"] + synth.plane_sizes(w.fmt, r, K)["min"])
            for r, K in ((w.d_ff, w.d_model), (w.d_ff, w.d_model), (w.d_model, w.d_ff)))
    return s


def clone_layer(dl):
    from quantized_moe_route_amd.layer import DeviceLayer
    planes = {n: tuple(None if t is None else t.clone() for t in p) for n, p in dl.planes.items()}
    return DeviceLayer(dl.fmt, dl.d_model, dl.d_ff, dl.n_experts, planes, dl.router.clone(),
                       None if dl.bias is None else dl.bias.clone())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, host_layer, router, bias, xs_host, seconds):
    """The oracle, as is, timed on a bounded sample of the same workload."""
    import oracle
    n = 0
    t0 = time.perf_counter()
    while True:
        x = xs_host[n % len(xs_host)]
        oracle.layer(host_layer, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k, x, wr=router, bias=bias)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return n, el


def oracle_spot_check(w, host_layer, x0, lg, ids_gpu, offsets_gpu, sp_gpu, w_gpu, out_gpu, rows, tf):
    """The CPU-baseline leg's parity sample: the oracle on the step's tokens
    `rows`, routed on the GPU's own logits; ids and the permutation checked
    in full.  Returns (ids_exact, max|err|/rms)."""
    import oracle
    ids_ref, _ = oracle.topk_softmax(lg, w.k)
    if tf is None:
        off_ref, sp_ref, _ = oracle.dispatch(ids_ref, w.n_experts)
    else:
        off_ref, sp_ref, _ = oracle.dispatch_tail_skip(ids_ref, w.n_experts, tf)
    n_kept = int(off_ref[w.n_experts])
    ids_ok = bool(np.array_equal(ids_gpu, ids_ref) and np.array_equal(offsets_gpu, off_ref)
                  and np.array_equal(sp_gpu[:n_kept], sp_ref[:n_kept]))
    if tf is None:
        _, _, out_ref = oracle.layer(host_layer, w.fmt, w.d_model, w.d_ff, w.n_experts, w.k,
                                     x0[rows], logits=lg[rows])
    else:
        # the kept set belongs to the whole batch: the sampled tokens' output
        # from their kept rows
        keep = oracle.tail_keep(ids_ref, w.n_experts, tf)
        idr = ids_ref[rows]
        re = np.concatenate([idr.ravel(), -np.ones(len(rows), np.int32)]).astype(np.int32)
        rt = np.concatenate([np.repeat(rows, w.k), rows]).astype(np.int32)
        yr = oracle.expert_rows(host_layer, w.fmt, w.d_model, w.d_ff, w.n_experts, x0, re, rt, f64=True)
        wk = w_gpu[rows].astype(np.float64) * keep[idr]
        out_ref = yr[len(rows) * w.k:] + np.einsum(
            "tj,tjd->td", wk, yr[:len(rows) * w.k].reshape(len(rows), w.k, w.d_model))
    rms = float(np.sqrt(np.mean(out_ref.astype(np.float64) ** 2)))
    err = float(np.max(np.abs(out_gpu[rows].astype(np.float64) - out_ref)) / rms)
    return ids_ok, err


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=None, choices=[1, 2, 3, 4, 5, 6],
                    help="one workload only (default: workload 1, plus 2 and 3 under \"regimes\")")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's T (tokens per layer), e.g. the mid-size batches")
    ap.add_argument("--tail-skip", type=int, default=None, metavar="RANK",
                    help="route tail-skip: experts the batch picked only at 0-based ranks >= RANK "
                         "are not computed (the pages' rule: 6 for a top-10); lossy, opt-in")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time moe_route and moe_dispatch as two calls (default: moe_route_dispatch)")
    ap.add_argument("--overlap-shared", action="store_true",
                    help="shared expert on a second stream beside routing (moe_shared_ffn), "
                         "routed experts after it (moe_routed_ffn)")
    ap.add_argument("--copies", type=int, default=None,
                    help="layer copies cycled, single-layer workloads (default 16 decode, 1 prefill)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference kernel "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def run_workload(wid, args):
    """Bench one workload; returns (result dict, ok)."""
    import torch

    import synth
    import synth.device as sdev
    import quantized_moe_route_amd as q
    from quantized_moe_route_amd import hip
    from quantized_moe_route_amd.layer import DeviceLayer, SideStream, alloc_buffers, run_layer

    w = synth.WORKLOADS[wid]
    if args.tokens is not None:
        import dataclasses
        import re
        w = dataclasses.replace(w, T=args.tokens, name=re.sub(r"T\d+", f"T{args.tokens}", w.name, count=1))
    prefill = w.T > 16   # the grouped matrix-core path
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if prefill:
        K = args.steps if args.steps is not None else (20 if w.layers == 1 else 3)
        W = args.warmup if args.warmup is not None else (3 if w.layers == 1 else 1)
        n_copies = 1 if args.copies is None else args.copies
    else:
        K = args.steps if args.steps is not None else (200 if w.layers == 1 else 20)
        W = args.warmup if args.warmup is not None else (20 if w.layers == 1 else 3)
        n_copies = 16 if args.copies is None else args.copies
    S = K + W
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream

    # ---------------------------------------------------------------- inputs
    t_setup = time.perf_counter()
    if w.layers == 1:
        L0 = synth.gen_layer(w, layer=0)
        dl0 = DeviceLayer.from_host(w.fmt, w.d_model, w.d_ff, w.n_experts, L0, L0.router, L0.bias,
                                    device=dev)
        layers = [dl0] + [clone_layer(dl0) for _ in range(n_copies - 1)]
        host_layer, host_router, host_bias = L0, L0.router, L0.bias
    else:
        layers = []
        for li in range(w.layers):
            planes = sdev.layer_planes(w, li, device=dev)
            wr, bias = sdev.router(w, li, device=dev)
            layers.append(DeviceLayer(w.fmt, w.d_model, w.d_ff, w.n_experts, planes, wr, bias))
        host_layer = sdev.to_host(layers[0].planes)
        host_router = layers[0].router.cpu().numpy()
        host_bias = None if layers[0].bias is None else layers[0].bias.cpu().numpy()
    n_lay = w.layers
    # x[step][layer]
    xs = [[sdev.x(w, li, s, device=dev) for li in range(n_lay)] for s in range(S)]
    with torch.cuda.stream(stream):
        buf = alloc_buffers(layers[0], w.T, w.k, device=dev, stream=stream)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f}s: {w.name}, {len(layers)} layer buffers, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    def layer_of(step, li):
        return layers[li] if n_lay > 1 else layers[step % len(layers)]

    tf = args.tail_skip
    if tf is not None and not 0 <= tf <= w.k:
        log(f"--tail-skip must lie in [0, {w.k}]")
        sys.exit(2)
    fused = not args.separate_calls
    ov = args.overlap_shared
    if ov and (not fused or tf is not None):
        log("--overlap-shared goes with the default calls (no --separate-calls / --tail-skip)")
        sys.exit(2)
    side = SideStream(device=dev) if ov else None
    fuse_cmb = not args.separate_calls and not ov and w.T <= FUSE_COMBINE_TMAX
    # step 0 once, eagerly: its outputs are the CPU-baseline leg's parity sample
    run_layer(layer_of(0, 0), xs[0][0], buf, stream=sh, tail_from=tf, fused=fused, side=side,
              fuse_combine=fuse_cmb)
    hip.stream_synchronize(sh)
    step0 = {"x": xs[0][0].cpu().numpy().view(np.uint16), "lg": buf.logits[:w.T].cpu().numpy(),
             "ids": buf.ids[:w.T].cpu().numpy(), "offsets": buf.offsets.cpu().numpy(),
             "sp": buf.sorted_pair[:w.T * w.k].cpu().numpy(), "w": buf.w[:w.T].cpu().numpy(),
             "out": buf.out[:w.T].cpu().numpy()}

    # deviation of the lossy tail-skip layer from the full layer (same input)
    tail_info = None
    if tf is not None:
        out_skip = buf.out[:w.T].clone()
        run_layer(layer_of(0, 0), xs[0][0], buf, stream=sh)
        hip.stream_synchronize(sh)
        full = buf.out[:w.T].double()
        dv = float((out_skip.double() - full).abs().max() / full.pow(2).mean().sqrt())
        tail_info = {"tail_from": tf, "pairs": w.T * w.k, "max_dev_from_full_layer_over_rms": dv}

    def dispatch():
        if tf is None:
            q.moe_dispatch(buf.ids, w.T, w.n_experts, w.k, buf.offsets, buf.sorted_pair,
                           buf.pair_pos, buf.ws, buf.ws_bytes, sh)
        else:
            q.moe_dispatch_tail_skip(buf.ids, w.T, w.n_experts, w.k, tf, buf.offsets,
                                     buf.sorted_pair, buf.pair_pos, buf.ws, buf.ws_bytes, sh)

    # ------------------------------------------------------------ capture
    ev_start, ev_end = hip.Event(), hip.Event()

    def call(c, s, li):
        L = layer_of(s, li)
        x = xs[s][li]
        if c == "route_dispatch" and tf is not None:
            q.moe_route_dispatch_tail_skip(x, L.router, L.bias, buf.logits, w.T, w.d_model, w.n_experts, w.k,
                                           tf, buf.ids, buf.w, buf.offsets, buf.sorted_pair, buf.pair_pos,
                                           buf.ws, buf.ws_bytes, sh)
        elif c == "shared_ffn":
            q.moe_shared_ffn(L.struct, x, w.T, buf.y_shared, buf.ws_sh, buf.ws_sh_bytes,
                             side.handle if side is not None else sh)
        elif c == "routed_ffn":
            q.moe_routed_ffn(L.struct, x, w.T, w.k, buf.offsets, buf.sorted_pair, buf.y_pairs,
                             buf.ws, buf.ws_bytes, sh)
        elif c == "route_dispatch":
            q.moe_route_dispatch(x, L.router, L.bias, buf.logits, w.T, w.d_model, w.n_experts, w.k,
                                 buf.ids, buf.w, buf.offsets, buf.sorted_pair, buf.pair_pos, buf.ws,
                                 buf.ws_bytes, sh)
        elif c == "route":
            q.moe_route(x, L.router, L.bias, buf.logits, w.T, w.d_model, w.n_experts, w.k,
                        buf.ids, buf.w, buf.ws, buf.ws_bytes, sh)
        elif c == "dispatch":
            dispatch()
        elif c == "expert_ffn_combine":
            q.moe_expert_ffn_combine(L.struct, x, w.T, w.k, buf.offsets, buf.sorted_pair, buf.pair_pos,
                                     buf.w, buf.y_pairs, buf.y_shared, buf.out, buf.ws, buf.ws_bytes, sh)
        elif c == "expert_ffn":
            q.moe_expert_ffn(L.struct, x, w.T, w.k, buf.offsets, buf.sorted_pair, buf.y_pairs,
                             buf.y_shared, buf.ws, buf.ws_bytes, sh)
        else:
            q.moe_combine(buf.y_pairs, buf.y_shared, buf.pair_pos, buf.w, w.T, w.k, w.d_model,
                          buf.out, sh)

    if ov:
        calls = ["shared_ffn", "route_dispatch", "routed_ffn", "combine"]
    elif fuse_cmb:
        calls = (["route_dispatch"] if fused else ["route", "dispatch"]) + ["expert_ffn_combine"]
    else:
        calls = (["route_dispatch"] if fused else ["route", "dispatch"]) + ["expert_ffn", "combine"]

    def enqueue(step0_, nsteps):
        for s in range(step0_, step0_ + nsteps):
            for li in range(n_lay):
                if ov:
                    # fork: the shared expert beside routing; join before the combine
                    side.fork.record(sh)
                    hip.stream_wait_event(side.handle, side.fork)
                    call("shared_ffn", s, li)
                    side.join.record(side.handle)
                    call("route_dispatch", s, li)
                    call("routed_ffn", s, li)
                    hip.stream_wait_event(sh, side.join)
                    call("combine", s, li)
                else:
                    for c in calls:
                        call(c, s, li)

    if args.eager:
        enqueue(K, W)
        hip.stream_synchronize(sh)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev_start.record(sh)
        enqueue(0, K)
        ev_end.record(sh)
        hip.stream_synchronize(sh)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        with hip.Graph(sh) as g_warm:
            enqueue(K, W)
        with hip.Graph(sh) as g_timed:
            enqueue(0, K)
        g_warm.launch()
        hip.stream_synchronize(sh)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev_start.record(sh)
        g_timed.launch()
        ev_end.record(sh)
        hip.stream_synchronize(sh)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3
    gpu_ms = ev_start.elapsed_ms(ev_end)
    out_graph = buf.out[:w.T].clone()

    # spread: the timed graph replayed four more times, each replay timed
    # with HIP events on the launch stream (per-step microseconds per replay)
    step_us = None
    if not args.eager:
        per_run = [1e3 * gpu_ms / K]
        for _ in range(4):
            ev_start.record(sh)
            g_timed.launch()
            ev_end.record(sh)
            hip.stream_synchronize(sh)
            per_run.append(1e3 * ev_start.elapsed_ms(ev_end) / K)
        pr = np.array(per_run)
        step_us = {"median": float(np.median(pr)), "p10": float(np.percentile(pr, 10)),
                   "p90": float(np.percentile(pr, 90)), "replays": len(per_run), "steps_each": K}
        del g_warm, g_timed

    # replay check: the last timed step again, eagerly; deterministic kernels
    enqueue(K - 1, 1)
    hip.stream_synchronize(sh)
    replay_ok = bool(torch.equal(out_graph, buf.out[:w.T]))

    # per-call GPU durations: a graph of G back-to-back launches of one call
    # (inputs of consecutive steps / layer copies), events around the graph
    G = min(K, 8 if prefill else 64)
    avg_us = {}
    side_saved, side = side, None   # per-call timing: every call on the main stream
    for c in calls + (["expert_ffn"] if "expert_ffn" not in calls else []):
        with hip.Graph(sh) as gc:
            for s in range(G):
                call(c, s, s % n_lay if n_lay > 1 else 0)
        gc.launch()
        e0, e1 = hip.Event(), hip.Event()
        e0.record(sh)
        gc.launch()
        e1.record(sh)
        hip.stream_synchronize(sh)
        avg_us[c] = 1e3 * e0.elapsed_ms(e1) / G
        del gc
    side = side_saved

    # algorithmic work of one moe_expert_ffn launch.
    #   decode: bytes = distinct experts used + shared, x rows in, y rows out
    #   prefill: flops = (P + T) rows x (gate + up + down) = rows * 6*d*f
    eb = expert_bytes(w)
    groups = []
    for s in range(min(K, 64)):
        for li in range(n_lay):
            L = layer_of(s, li)
            q.moe_route(xs[s][li], L.router, L.bias, buf.logits, w.T, w.d_model, w.n_experts,
                        w.k, buf.ids, buf.w, buf.ws, buf.ws_bytes, sh)
            dispatch()
            hip.stream_synchronize(sh)
            off = buf.offsets.cpu().numpy()
            groups.append(int(np.count_nonzero(np.diff(off))) + 1)
    rows_ffn = w.T * w.k + w.T
    act_bytes = rows_ffn * w.d_model * (2 + 4)             # x row in, y row out
    ffn_bytes = float(np.mean(groups)) * eb + act_bytes
    ffn_flops = float(rows_ffn) * 6.0 * w.d_model * w.d_ff
    ffn_call = "expert_ffn_combine" if "expert_ffn_combine" in calls else "expert_ffn"
    if ffn_call == "expert_ffn_combine":
        # + the merge: every y row read back, out written, pair positions and weights
        ffn_bytes += (rows_ffn * 4 + w.T * 4) * w.d_model + w.T * w.k * 8
    t_ffn = avg_us[ffn_call] * 1e-6
    # counters were taken at the workload's own T and calls only
    traffic = (traffic_for(wid) if args.tokens is None and tf is None and not ov and fused else None)
    if prefill:
        achieved = ffn_flops / t_ffn / 1e12
        roof = {"bound": "mfma", "kernel": "moe_expert_ffn (pf_gemm gate/up + down, "
                                           "routed + shared, item build, x to fp16)",
                "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic,
                "flops_per_launch": ffn_flops, "avg_groups": float(np.mean(groups)),
                "hbm_gbs_algorithmic": ffn_bytes / t_ffn / 1e9}
    else:
        achieved = ffn_bytes / t_ffn / 1e9
        roof = {"bound": "hbm",
                "kernel": ("moe_expert_ffn_combine call: gateup_small, down_small with the merge"
                           if ffn_call == "expert_ffn_combine" else
                           "moe_expert_ffn call: gateup_small, down_small"),
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "bytes_per_launch": ffn_bytes, "avg_groups": float(np.mean(groups))}
    layer_bytes = ffn_bytes + w.d_model * w.n_experts * 4  # + router weights

    ms_per_step = wall_ms / K
    tokens_per_s = w.T * K / (wall_ms / 1e3)

    # ------------------------------------------------------------ CPU oracle
    # The only oracle calls of the run: the parity sample of step 0 (decode:
    # every token; prefill: 16 seeded tokens, routed on the GPU's logits;
    # ids and the permutation in full), then the oracle's own throughput on
    # a bounded sample of the same workload.
    cpu = None
    parity = {"ids_exact": None, "max_err_over_rms": None, "tokens_checked": 0,
              "graph_replay_bitwise": replay_ok}
    if not args.no_cpu_baseline:
        import oracle as orc
        rows = (np.sort(np.random.default_rng(7).choice(w.T, size=16, replace=False))
                if prefill else np.arange(w.T))
        ids_ok, err = oracle_spot_check(w, host_layer, step0["x"], step0["lg"], step0["ids"],
                                        step0["offsets"], step0["sp"], step0["w"], step0["out"], rows, tf)
        parity.update(ids_exact=ids_ok, max_err_over_rms=err, tokens_checked=int(len(rows)))
        log(f"parity step 0 ({len(rows)} tokens): ids/permutation exact={ids_ok} max|err|/rms={err:.3e}")
        if prefill:
            # 256-token slices of the chunk, layer 0, until the time is up
            chunk = 256
            xs_host = [step0["x"][i:i + chunk] for i in range(0, w.T, chunk)]
        else:
            chunk = w.T
            xs_host = [xs[s][0].cpu().numpy().view(np.uint16) for s in range(min(S, 64))]
        n, el = cpu_baseline(w, host_layer, host_router, host_bias, xs_host, args.cpu_seconds)
        rate = n * chunk / el
        what = (f"{n} oracle layer evaluations of {chunk}-token slices of the T={w.T} chunk"
                if prefill else f"{n} oracle layer evaluations of T={w.T} token(s)")
        cpu = {"value": rate / n_lay,
               "unit": "tokens/s" + (" (through the 48-layer stack)" if n_lay > 1 else ""),
               "cores": orc.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"{what} on layer 0 ({el:.1f} s)" +
                         (f"; stack rate = per-layer rate / {n_lay}" if n_lay > 1 else "")}

    res = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s" + (" (through the 48-layer stack)" if n_lay > 1 else ""),
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16" if prefill else "bf16",
        "data": "synthetic (seeded generator; random weights of the stated shape)",
        "config": {"workload": w.name, "d_model": w.d_model, "d_ff": w.d_ff,
                   "n_experts": w.n_experts, "top_k": w.k, "shared_experts": 1, "T": w.T,
                   "layers": n_lay, "format": "Q2_B32" if w.fmt == 1 else "Q3_B32",
                   "layer_copies": len(layers) if n_lay == 1 else 1,
                   "mode": "eager" if args.eager else "hip-graph",
                   "calls": calls,
                   **({"shared_expert": "second stream, beside routing"} if ov else {}),
                   **({} if tf is None else {"route_tail_skip_from": tf})},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_ms_per_step": gpu_ms / K,
        "step_us": step_us,
        "per_call_us": avg_us,
        ("layer_mfma_frac" if prefill else "layer_hbm_frac"):
            (ffn_flops * n_lay / (gpu_ms / K * 1e-3) / 1e12 / BF16_PEAK_TFLOPS) if prefill else
            (layer_bytes * n_lay / (gpu_ms / K * 1e-3) / 1e9 / HBM_PEAK_GBS),
        "parity": parity,
        **({} if tail_info is None else {"tail_skip": tail_info}),
    }
    ok = replay_ok and (parity["ids_exact"] is None or (parity["ids_exact"] and parity["max_err_over_rms"] <= 2e-3))
    # release this workload's device memory before the next one
    del layers, xs, buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, ok


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library has "
              "no multi-GPU path (the expert-parallel sharding it would use is not implemented).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}))
        return

    single = (args.workload is not None or args.tokens is not None or args.tail_skip is not None
              or args.separate_calls or args.overlap_shared or args.copies is not None)
    wids = [args.workload or 1] if single else [1, 2, 3]
    results = []
    all_ok = True
    for wid in wids:
        log(f"--- workload {wid}")
        res, ok = run_workload(wid, args)
        results.append(res)
        all_ok = all_ok and ok
    head = results[0]
    if len(results) > 1:
        keep = ("value", "unit", "steps", "warmup", "ms_per_step", "dtype", "config", "roofline",
                "cpu_baseline", "gpu_ms_per_step", "step_us", "per_call_us", "layer_mfma_frac",
                "layer_hbm_frac", "parity")
        head["regimes"] = {r["config"]["workload"]: {k: r[k] for k in keep if k in r} for r in results[1:]}
    print(json.dumps(head))
    if not all_ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
