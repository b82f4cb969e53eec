#!/usr/bin/env python3
"""Throughput of the fp9 routed-expert MoE layer on one MI355X.

Workload: one DeepSeek-V3-shaped MoE layer (hidden 7168, intermediate 2048,
256 routed experts + 1 shared, top-8) with fp9 expert weights resident in HBM,
decode batch 1 (and 2, reported alongside).  A step is one full layer call
(gate/up + SwiGLU + down + combine) on a fresh seeded routing draw, so each
step streams the selected experts from HBM rather than from cache.

Prints one JSON line.  `value` is layer tokens/s at bsz 1 with inputs already
in HBM.  The roofline object is for the dominant kernel, k_gate_up (two thirds
of the bytes): its launches run back to back between two HIP events on the
stream they run on (each on a fresh routing draw), so the average is the
kernel's own duration plus the gap between two dispatches.  The CPU baseline
is the float64 oracle on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
H, I, E, K = 7168, 2048, 256, 8
SEED, WORKLOAD = 0, 3
METRIC = "MoE-layer tokens/s at bsz=1/2 and achieved HBM GB/s (% of MI355X peak)"

# HBM bytes per k_gate_up launch at bsz 1 from rocprofv3 FETCH_SIZE + WRITE_SIZE,
# each scaled by the same counter's reading for a 1 GiB device copy (profiles/
# moe_layer_hbm_counters.md).  Valid only for the kernel sources it was taken on.
MEASURED_TRAFFIC = {
    "sources_sha256": "580f596975f465ccc6f32c2615b7b280abd234600fd35204c1691dd88bada7d4",
    "bytes_per_launch": 297756021,
}
KERNEL_SOURCES = ("bit_moe_expert_fp9_amd/csrc/duckmoe.hip", "bit_moe_expert_fp9_amd/csrc/fp9_device.h",
                  "bit_moe_expert_fp9_amd/csrc/mfma_device.h", "bit_moe_expert_fp9_amd/csrc/host_util.h")


def measured_traffic():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != MEASURED_TRAFFIC["sources_sha256"]:
        return None  # the kernels changed since the counters were taken
    return MEASURED_TRAFFIC["bytes_per_launch"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=16,
                   help="tokens (bsz 1 steps) the oracle times for the CPU baseline")
    p.add_argument("--bsz2", type=int, default=1, help="also time bsz 2 (0 to skip)")
    p.add_argument("--more-bsz", type=str, default="4,8",
                   help="comma-separated further batch sizes (3..8, the matrix-core path) timed "
                        "on the same layer ('' to skip); results go under config.layer_bsz")
    p.add_argument("--stack", type=int, default=1,
                   help="time the 16-layer stack (about 204 GB of fp9 weights drawn on the "
                        "device) at bsz 1, 2, 4 and 8 (0 to skip); results go under 'stack'")
    p.add_argument("--stack-steps", type=int, default=20)
    p.add_argument("--dense", type=int, default=1,
                   help="also time the dense fp9 MLP 7168/18432 at bsz 1 and 2 (0 to skip)")
    p.add_argument("--prefill", type=str, default="2048",
                   help="comma-separated token counts for the prefill path on the same layer "
                        "('' to skip); results go under config.prefill")
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--extra", type=int, default=1,
                   help="also run the 256x512 GEMV, lane-overlap, single-expert and shard-partial "
                        "legs (0 to skip)")
    p.add_argument("--calib-copy-mb", type=int, default=0,
                   help="first run 3 plain device copies of this many MiB (a known-size "
                        "reference for HBM byte counters under rocprofv3 --pmc)")
    return p.parse_args()


def calib_copy(torch, mib):
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("calibration copies: 3 x %d bytes read + %d bytes written" % (n, n))
    del src, dst


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)

SETTLE_MS = 60.0


def settle(torch, fn, ms=SETTLE_MS):
    """Runs fn() untimed, synchronizing every few calls, until `ms` of wall time
    has passed.  After a pause (the host preparing the next measurement's
    inputs) the GPU's clocks take tens of milliseconds to come back up:
    measured on MI355X, bsz-2 layer calls right after a 50 ms pause ran about
    11% slower over the next 20 calls than after 50 ms of work, and needed
    some 30 ms of calls to recover.  Every timed region starts settled."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def back_to_back_us(torch, stream, steps, call, primer):
    """Mean microseconds per call of `call(k)`, k = 0 .. steps-1, launched back
    to back between two events on `stream`, after settle() with `primer`.
    `primer()`, an untimed call of the same kind, is queued just ahead of the
    start event: the GPU runs it while
    the host queues the first timed calls, so the start event does not wait on
    the host's first launch (some tens of microseconds of Python and launch
    work, which over 20 steps would add more than a microsecond per step)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, primer)
    primer()
    a.record(stream)
    for k in range(steps):
        call(k)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / steps



def graph_us(torch, call, n=64, replays=5):
    """Mean microseconds per call of `call(k, stream)`, k = 0 .. n-1, captured in
    one HIP graph and replayed back to back between two events: the GPU's own
    time per call, with no host work between launches (the calls launch
    kernels only).  One replay, queued ahead of the start event, is untimed."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0, side)  # each launch site's first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        for k in range(n):
            call(k, st)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settle(torch, g.replay)
    g.replay()
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (n * replays)
    del g
    return us


def time_layer(torch, dm, layer, T, steps, warmup, draws):
    """Times `steps` layer calls (after `warmup`): once back to back between two
    events (the throughput), once with an event before each call (the per-call
    percentiles)."""
    from bit_moe_expert_fp9_amd import synth
    n = steps + warmup
    xs, ids, ws_, uniq = [], [], [], []
    for s in range(n):
        d = s % draws
        x = synth.activations(SEED, WORKLOAD, 0, 10_000 + d, T, H)
        i, w = synth.routing(SEED, WORKLOAD, 0, 10_000 + d, T, E, K)
        xs.append(x)
        ids.append(i)
        ws_.append(w)
        uniq.append(len(np.unique(i)))
    X = torch.from_numpy(np.stack(xs)).cuda()
    IDS = torch.from_numpy(np.stack(ids)).cuda()
    W = torch.from_numpy(np.stack(ws_)).cuda()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = layer.workspace(T)
    stream = torch.cuda.current_stream()

    for s in range(warmup):
        dm.moe_layer(layer, X[s], IDS[s], W[s], out=out, ws=ws, stream=stream)
    torch.cuda.synchronize()

    # The timed region: `steps` calls back to back between two events, the
    # last warm-up draw queued ahead of the start event as the primer.
    def call(k):
        s = warmup + k
        dm.moe_layer(layer, X[s], IDS[s], W[s], out=out, ws=ws, stream=stream)

    def primer():
        s = max(warmup - 1, 0)
        dm.moe_layer(layer, X[s], IDS[s], W[s], out=out, ws=ws, stream=stream)

    t0 = time.perf_counter()
    total_ms = back_to_back_us(torch, stream, steps, call, primer) * steps / 1e3
    wall = time.perf_counter() - t0
    # The per-call distribution: the same calls again with an event before each
    # (an event between two calls adds its own gap, so this pass is not the
    # throughput figure).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for k in range(steps):
        s = warmup + k
        ev[k].record(stream)
        dm.moe_layer(layer, X[s], IDS[s], W[s], out=out, ws=ws, stream=stream)
    ev[steps].record(stream)
    torch.cuda.synchronize()
    t_call = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    u = np.array(uniq[warmup:], dtype=np.float64)
    eb = layer.expert_bytes()
    bytes_call = (u + 1) * eb + 2 * T * H * 4   # selected experts' fp9 planes + x + out
    return {
        "T": T,
        "total_ms": total_ms,
        "wall_s": wall,
        "ms_per_step": total_ms / steps,
        "tokens_per_s": T * steps / (total_ms / 1e3),
        "call_us": float(t_call.mean() * 1e3),
        "bytes_step": float(bytes_call.mean()),
        "mean_experts": float((u + 1).mean()),
        "p10_us": float(np.percentile(t_call, 10) * 1e3),
        "p50_us": float(np.percentile(t_call, 50) * 1e3),
        "p90_us": float(np.percentile(t_call, 90) * 1e3),
    }


def time_stages(torch, dm, layer, T, steps, warmup, draws):
    """Times the gate/up and down stages launched one by one (HIP events around each)."""
    from bit_moe_expert_fp9_amd import synth
    n = steps + warmup
    xs, ids, ws_, uniq = [], [], [], []
    for s in range(n):
        d = s % draws
        x = synth.activations(SEED, WORKLOAD, 0, 30_000 + d, T, H)
        i, w = synth.routing(SEED, WORKLOAD, 0, 30_000 + d, T, E, K)
        xs.append(x)
        ids.append(i)
        ws_.append(w)
        uniq.append(len(np.unique(i)))
    X = torch.from_numpy(np.stack(xs)).cuda()
    IDS = torch.from_numpy(np.stack(ids)).cuda()
    W = torch.from_numpy(np.stack(ws_)).cuda()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = layer.workspace(T)
    stream = torch.cuda.current_stream()
    def both(s):
        dm.moe_gate_up(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)
        dm.moe_down(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)

    for s in range(warmup):
        both(s)
    settle(torch, lambda: both(max(warmup - 1, 0)))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    for k in range(steps):
        s = warmup + k
        ev[3 * k].record(stream)
        dm.moe_gate_up(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)
        ev[3 * k + 1].record(stream)
        dm.moe_down(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)
        ev[3 * k + 2].record(stream)
    torch.cuda.synchronize()
    gu = np.array([ev[3 * k].elapsed_time(ev[3 * k + 1]) for k in range(steps)]) * 1e3
    dn = np.array([ev[3 * k + 1].elapsed_time(ev[3 * k + 2]) for k in range(steps)]) * 1e3
    slots = np.array(uniq[warmup:], dtype=np.float64) + 1
    eb = layer.expert_bytes()
    # algorithmic bytes: gate/up reads 2/3 of each selected expert's planes and x and
    # writes one h' row per slot and token; down reads the last 1/3 and the h' rows
    # and writes out
    gu_bytes = slots * (eb * 2 // 3) + T * H * 4 + slots * T * I * 4
    dn_bytes = slots * (eb // 3) + slots * T * I * 4 + T * H * 4
    return {
        "T": T,
        "gate_up_us": float(gu.mean()),
        "down_us": float(dn.mean()),
        "gate_up_bytes": float(gu_bytes.mean()),
        "down_bytes": float(dn_bytes.mean()),
        "gate_up_gbps": float(gu_bytes.mean() / (gu.mean() * 1e-6) / 1e9),
        "down_gbps": float(dn_bytes.mean() / (dn.mean() * 1e-6) / 1e9),
    }


def time_gate_up_back_to_back(torch, dm, layer, T, steps, warmup, draws):
    """The gate/up stage alone, `steps` launches back to back between two
    events on their stream, each on a fresh routing draw: the kernel's average
    duration plus one dispatch gap (no event between launches)."""
    from bit_moe_expert_fp9_amd import synth
    n = steps + warmup
    xs, ids, ws_, uniq = [], [], [], []
    for s in range(n):
        d = s % draws
        xs.append(synth.activations(SEED, WORKLOAD, 0, 70_000 + d, T, H))
        i, w = synth.routing(SEED, WORKLOAD, 0, 70_000 + d, T, E, K)
        ids.append(i)
        ws_.append(w)
        uniq.append(len(np.unique(i)))
    X = torch.from_numpy(np.stack(xs)).cuda()
    IDS = torch.from_numpy(np.stack(ids)).cuda()
    W = torch.from_numpy(np.stack(ws_)).cuda()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = layer.workspace(T)
    stream = torch.cuda.current_stream()
    for s in range(warmup):
        dm.moe_gate_up(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)
    def call(k):
        s = warmup + k
        dm.moe_gate_up(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)

    def primer():
        s = max(warmup - 1, 0)
        dm.moe_gate_up(layer, X[s], IDS[s], W[s], ws, out=out, stream=stream)

    us = back_to_back_us(torch, stream, steps, call, primer)
    slots = np.array(uniq[warmup:], dtype=np.float64) + 1
    eb = layer.expert_bytes()
    gu_bytes = slots * (eb * 2 // 3) + T * H * 4 + slots * T * I * 4
    return {"us": us, "bytes": float(gu_bytes.mean()),
            "gbps": float(gu_bytes.mean() / (us * 1e-6) / 1e9)}


def time_gemv_256x512(torch, dm, reps=2000):
    """One fp9 GEMV 256 x 512 (N(0, 0.02) weights, x ~ N(0, 1)) and
    the decode of all 512 fp9 codes, each as back-to-back launches between two
    events: launch-bound, reported in microseconds per call."""
    from bit_moe_expert_fp9_amd import synth
    Wt = synth.weights(SEED, 1, 0, 0, synth.GATE, (256, 512))
    body, sign = dm.quantize_fp9(Wt)
    bd, sd = torch.from_numpy(body).cuda(), torch.from_numpy(sign).cuda()
    x = torch.from_numpy(synth.activations(SEED, 1, 0, 0, 1, 512)[0]).cuda()
    y = torch.empty(256, dtype=torch.float32, device="cuda")
    codes = np.arange(512, dtype=np.uint16)
    cb = torch.from_numpy((codes & 0xFF).astype(np.uint8)).cuda()
    cs = torch.from_numpy(np.packbits(((codes >> 8) & 1).astype(np.uint8), bitorder="little")).cuda()
    dec = torch.empty(512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}

    def fn_st(name, st):
        if name == "gemv_us":
            dm.gemv_fp9(bd, sd, x, out=y, stream=st)
        else:
            dm.decode_fp9(cb, cs, out=dec, stream=st)

    for name, fn in (("gemv_us", lambda: dm.gemv_fp9(bd, sd, x, out=y, stream=stream)),
                     ("decode_512_codes_us", lambda: dm.decode_fp9(cb, cs, out=dec, stream=stream))):
        for _ in range(50):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        settle(torch, fn)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) * 1e3 / reps
        res[name.replace("_us", "_graph_us")] = graph_us(torch, lambda k, st: fn_st(name, st))
    res["what"] = ("256 x 512 fp9 GEMV (147,456 weight bytes) and a decode of all 512 codes: "
                   "back-to-back launches from the host (bound by the host's launch work), "
                   "and the same launches replayed from a HIP graph (*_graph_us)")
    log("gemv 256x512:", json.dumps(res))
    return res


def read_ceiling(torch, dm, sizes, reps=100):
    """Plain streaming-read time (duckmoe_read_probe) for each byte count, each
    launch on a fresh window of an 8-window buffer (no reuse from the cache)."""
    sizes = [s // 1024 * 1024 for s in sizes]
    win = max(sizes)
    buf = torch.empty(8 * win, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {}
    for nb in sizes:
        for i in range(10):
            dm.read_probe(buf[(i % 8) * win:], nb, sink, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        settle(torch, lambda: dm.read_probe(buf[5 * win:], nb, sink, stream=stream))
        for i in range(reps):
            ev[2 * i].record(stream)
            dm.read_probe(buf[((i * 3) % 8) * win:], nb, sink, stream=stream)
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)])) * 1e3
        out[nb] = (us, nb / (us * 1e-6) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return out


def time_pair(torch, dm, layer, steps, warmup, draws):
    """Two tokens per step, three ways: one bsz-2 call, two lanes on their own
    streams (duckmoe_lane_begin/finish), and two bsz-1 calls in turn."""
    from bit_moe_expert_fp9_amd import synth
    n = steps + warmup
    X = torch.from_numpy(np.stack([synth.activations(SEED, WORKLOAD, 0, 50_000 + s % draws, 2, H)
                                   for s in range(n)])).cuda()
    r = [synth.routing(SEED, WORKLOAD, 0, 50_000 + s % draws, 2, E, K) for s in range(n)]
    IDS = torch.from_numpy(np.stack([a for a, _ in r])).cuda()
    W = torch.from_numpy(np.stack([b for _, b in r])).cuda()
    stream = torch.cuda.current_stream()
    out2 = torch.empty((2, H), dtype=torch.float32, device="cuda")
    outs = [torch.empty((1, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    ws1, ws2 = layer.workspace(1), layer.workspace(2)
    lanes = []  # created after the two single-stream forms are timed

    def bsz2(s):
        dm.moe_layer(layer, X[s], IDS[s], W[s], out=out2, ws=ws2, stream=stream)

    def lanes2(s):
        for t in range(2):
            lanes[t].begin(layer, X[s][t:t + 1], IDS[s][t:t + 1], W[s][t:t + 1], outs[t],
                           producer=stream)
        for lane in lanes:
            lane.finish(consumer=stream)

    def serial(s):
        for t in range(2):
            dm.moe_layer(layer, X[s][t:t + 1], IDS[s][t:t + 1], W[s][t:t + 1], out=outs[t],
                         ws=ws1, stream=stream)

    res = {}
    n_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    for name, fn in (("bsz2_call", bsz2), ("two_serial_calls", serial), ("two_lanes", lanes2),
                     ("two_lanes_half_budget", lanes2)):
        for lane in lanes:
            lane.close()
        if name == "two_lanes":
            lanes[:] = [dm.Lane(layer), dm.Lane(layer)]
        elif name == "two_lanes_half_budget":
            lanes[:] = [dm.Lane(layer, cus=n_cus // 2) for _ in range(2)]
        for s in range(warmup):
            fn(s)
        us = back_to_back_us(torch, stream, steps, lambda k: fn(warmup + k),
                             lambda: fn(max(warmup - 1, 0)))
        res[name] = {"us_per_pair": us, "tokens_per_s": 2 / (us * 1e-6)}
    for lane in lanes:
        lane.close()
    log("pair:", json.dumps(res))
    return res


def time_lane_overlap(torch, dm, layer, steps, warmup, draws):
    """The pair runtime of the pages' dual-lane decode on one GPU: per decoder
    layer each of two lanes runs a GPU stage (a bf16 GEMM stands in for the
    attention part, 1024 x 7168 by 7168 x 4096) and then the MoE layer (bsz 1),
    the next stage of a lane waiting for its MoE.  Serial: everything on one
    stream.  Overlapped: the stages on a stream of their own and each lane's
    MoE on its lane stream, so one lane's MoE runs while the other lane's
    stage does; with lanes sized to half the CUs, and (for comparison) with
    lanes whose grids fill the device."""
    from bit_moe_expert_fp9_amd import synth
    n = steps + warmup
    X = torch.from_numpy(np.stack([synth.activations(SEED, WORKLOAD, 0, 80_000 + s % draws, 2, H)
                                   for s in range(n)])).cuda()
    r = [synth.routing(SEED, WORKLOAD, 0, 80_000 + s % draws, 2, E, K) for s in range(n)]
    IDS = torch.from_numpy(np.stack([a for a, _ in r])).cuda()
    W = torch.from_numpy(np.stack([b for _, b in r])).cuda()
    ga = torch.randn(1024, 7168, device="cuda", dtype=torch.bfloat16)
    gb = torch.randn(7168, 4096, device="cuda", dtype=torch.bfloat16)
    gc = [torch.empty(1024, 4096, device="cuda", dtype=torch.bfloat16) for _ in range(2)]
    outs = [torch.empty((1, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    stream = torch.cuda.current_stream()
    ws1 = layer.workspace(1)

    def stage(t, st):
        with torch.cuda.stream(st):
            torch.matmul(ga, gb, out=gc[t])

    # GPU stage and MoE alone, each back to back on the whole device
    for _ in range(5):
        stage(0, stream)
    stage_us = back_to_back_us(torch, stream, steps, lambda k: stage(0, stream),
                               lambda: stage(0, stream))

    def serial(s):
        for t in range(2):
            stage(t, stream)
            dm.moe_layer(layer, X[s][t:t + 1], IDS[s][t:t + 1], W[s][t:t + 1], out=outs[t],
                         ws=ws1, stream=stream)

    for s in range(warmup):
        serial(s)
    serial_us = back_to_back_us(torch, stream, steps, lambda k: serial(warmup + k),
                                lambda: serial(max(warmup - 1, 0)))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run_overlapped(sst, lanes):
        def overlapped(s):
            for t in range(2):
                lanes[t].finish(consumer=sst)   # this lane's previous MoE is done
                stage(t, sst)
                lanes[t].begin(layer, X[s][t:t + 1], IDS[s][t:t + 1], W[s][t:t + 1], outs[t],
                               producer=sst)

        torch.cuda.synchronize()
        for s in range(warmup):
            overlapped(s)
        settle(torch, lambda: overlapped(max(warmup - 1, 0)))
        for lane in lanes:
            lane.finish(consumer=sst)
        sst.synchronize()
        a.record(sst)
        for k in range(steps):
            overlapped(warmup + k)
        for lane in lanes:
            lane.finish(consumer=sst)
        b.record(sst)
        sst.synchronize()
        for lane in lanes:
            lane.close()
        return a.elapsed_time(b) * 1e3 / steps

    n_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    over_full_us = run_overlapped(torch.cuda.Stream(), [dm.Lane(layer), dm.Lane(layer)])
    over_us = run_overlapped(torch.cuda.Stream(),
                             [dm.Lane(layer, cus=n_cus // 2), dm.Lane(layer, cus=n_cus // 2)])
    res = {"what": "per decoder layer, two lanes: GPU stage (bf16 GEMM 1024x7168x4096) then "
                   "the bsz-1 MoE layer, the next stage of a lane after its MoE; serial = one "
                   "stream; overlapped = the stages on their own stream, each lane's MoE on "
                   "its lane stream with a CU budget of half the device, so one lane's MoE "
                   "runs while the other lane's stage does",
           "stage_us": stage_us, "serial_us_per_layer": serial_us,
           "overlapped_us_per_layer": over_us, "speedup": serial_us / over_us,
           "overlapped_full_grid_lanes_us_per_layer": over_full_us}
    log("lane overlap:", json.dumps(res))
    return res


def time_expert_and_partials(torch, dm, layer, steps, warmup):
    """One expert at bsz 1 (49.5 MB) and the bsz-2 layer in 32-shard partial mode."""
    from bit_moe_expert_fp9_amd import synth
    stream = torch.cuda.current_stream()
    res = {}
    x1 = torch.from_numpy(synth.activations(SEED, 2, 0, 0, 1, H)).cuda()
    out1 = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws1 = layer.workspace(1)
    e = 17
    for _ in range(warmup):
        dm.expert_ffn(layer, e, x1, out=out1, ws=ws1, stream=stream)

    def one(k):  # a different expert each call, so HBM is read
        dm.expert_ffn(layer, k % E, x1, out=out1, ws=ws1, stream=stream)

    us = back_to_back_us(torch, stream, steps, one, lambda: one(E - 1))
    t0 = time.perf_counter()  # the host's own time per call: the enqueue loop alone
    for k in range(steps):
        one(k)
    host_us = (time.perf_counter() - t0) * 1e6 / steps
    torch.cuda.synchronize()
    eb = layer.expert_bytes()
    # host_us_per_call: the host's time per call over the same loop; when it is
    # not below `us`, the loop is bound by the host's launches, not the GPU
    # the same calls from a HIP graph, and a plain read of the same byte count
    # from a graph: the GPU's time per call without the host's launch work
    g_us = graph_us(torch, lambda k, st: dm.expert_ffn(layer, k % E, x1, out=out1, ws=ws1,
                                                       stream=st))
    buf = torch.empty(16 * eb, dtype=torch.uint8, device="cuda")  # 16 windows, 790 MB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    r_us = graph_us(torch, lambda k, st: dm.read_probe(buf[(k % 16) * eb:], eb, sink, stream=st))
    del buf
    res["one_expert_bsz1"] = {"us": us, "hbm_gbps": eb / (us * 1e-6) / 1e9, "bytes": eb,
                              "host_us_per_call": host_us,
                              "graph_us": g_us, "graph_hbm_gbps": eb / (g_us * 1e-6) / 1e9,
                              "read_probe_graph_us": r_us,
                              "vs_read_probe": r_us / g_us}
    n = steps + warmup
    X = torch.from_numpy(np.stack([synth.activations(SEED, WORKLOAD, 0, 60_000 + s, 2, H)
                                   for s in range(n)])).cuda()
    r = [synth.routing(SEED, WORKLOAD, 0, 60_000 + s, 2, E, K) for s in range(n)]
    IDS = torch.from_numpy(np.stack([p for p, _ in r])).cuda()
    W = torch.from_numpy(np.stack([q for _, q in r])).cuda()
    by = float(np.mean([(len(np.unique(p)) + 1) * eb for p, _ in r[warmup:]]))
    outp = torch.empty((32, 2, H), dtype=torch.float32, device="cuda")
    wsp = layer.workspace(2, 32)
    def part(s):
        dm.moe_layer(layer, X[s], IDS[s], W[s], out=outp, n_shards=32, ws=wsp, stream=stream)

    for s in range(warmup):
        part(s)
    us = back_to_back_us(torch, stream, steps, lambda k: part(warmup + k),
                         lambda: part(max(warmup - 1, 0)))
    res["pair_32_partials_bsz2"] = {"us": us, "tokens_per_s": 2 / (us * 1e-6),
                                    "hbm_gbps": by / (us * 1e-6) / 1e9}
    log("expert / partials:", json.dumps(res))
    return res


MFMA_F16_PEAK_TFLOPS = 2500.0


def time_prefill(torch, dm, layer, T, steps, warmup, draws=4):
    """The prefill path (token lists + grouped GEMMs) on T tokens of the same
    layer: a few seeded draws, cycled, with HIP events around the call."""
    from bit_moe_expert_fp9_amd import synth
    stream = torch.cuda.current_stream()
    xs, ids, ws_, uniq = [], [], [], []
    for d in range(draws):
        xs.append(torch.from_numpy(synth.activations(SEED, 7, 0, d, T, H)).cuda())
        i, w = synth.routing(SEED, 7, 0, d, T, E, K)
        ids.append(torch.from_numpy(i).cuda())
        ws_.append(torch.from_numpy(w).cuda())
        uniq.append(len(np.unique(i)))
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = layer.prefill_workspace(T)
    def call(k):
        d = k % draws
        dm.moe_prefill(layer, xs[d], ids[d], ws_[d], out=out, ws=ws, stream=stream)

    for s in range(warmup):
        call(s)
    ms = back_to_back_us(torch, stream, steps, call, lambda: call(draws - 1)) / 1e3
    eb = layer.expert_bytes()
    wbytes = float(np.mean([(u + 1) * eb for u in uniq]))
    flops = 2.0 * 3 * H * I * T * (K + 1)     # every (token, expert) pair: gate, up, down
    res = {"T": T, "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
           "weight_bytes": wbytes, "weight_gbps": wbytes / (ms * 1e-3) / 1e9,
           "weight_hbm_frac": wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "useful_tflops": flops / (ms * 1e-3) / 1e12,
           "useful_mfma_frac": flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
           "mean_experts": float(np.mean(uniq)) + 1,
           "dtype": "fp16 weights (exact fp9 decode) times scaled fp16 hi/lo activation pairs "
                    "on the matrix cores, f32 accumulation"}
    log("prefill T=%d:" % T, json.dumps(res))
    return res


DENSE_I, DENSE_WORKLOAD = 18432, 6


def time_dense(torch, dm, steps, warmup):
    """Dense fp9 MLP 7168/18432 (DeepSeek-V3's dense FFN shape) at bsz 1 and 2."""
    from bit_moe_expert_fp9_amd import synth
    mlp = dm.Layer(H, DENSE_I, 0, 1).fill_synthetic_device(SEED, DENSE_WORKLOAD, 0)
    stream = torch.cuda.current_stream()
    res = {"shape": "7168/18432 SwiGLU MLP, fp9 planes (3 x 7168 x 18432 x 9/8 B)",
           "weight_bytes": mlp.expert_bytes()}
    for T in (1, 2):
        X = torch.from_numpy(np.stack([synth.activations(SEED, DENSE_WORKLOAD, 0, s, T, H)
                                       for s in range(8)])).cuda()
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws = mlp.workspace(T)
        def call(s):
            dm.expert_ffn(mlp, 0, X[s % 8], out=out, ws=ws, stream=stream)

        for s in range(warmup):
            call(s)
        us = back_to_back_us(torch, stream, steps, call, lambda: call(7))
        gbps = mlp.expert_bytes() / (us * 1e-6) / 1e9
        res["bsz%d" % T] = {"us": us, "tokens_per_s": T / (us * 1e-6), "hbm_gbps": gbps,
                            "hbm_frac": gbps / HBM_PEAK_GBPS}
        log("dense bsz%d:" % T, json.dumps(res["bsz%d" % T]))
    del mlp
    torch.cuda.empty_cache()
    return res


STACK_LAYERS, STACK_WORKLOAD = 16, 5


def time_stack(torch, dm, steps, warmup):
    """Stack passes (16 layers + RMS glue, one native call each) at bsz 1, 2, 4, 8."""
    from bit_moe_expert_fp9_amd import synth
    t0 = time.time()
    layers = [dm.Layer(H, I, E, K).fill_synthetic_device(SEED, STACK_WORKLOAD, l)
              for l in range(STACK_LAYERS)]
    torch.cuda.synchronize()
    log("stack of %d layers drawn on the device in %.1f s" % (STACK_LAYERS, time.time() - t0))
    stack = dm.Stack(layers)
    eb = layers[0].expert_bytes()
    stream = torch.cuda.current_stream()
    res = {}
    for T in (1, 2, 4, 8):
        n = steps + warmup
        X, IDS, W, by = [], [], [], []
        for s in range(n):
            X.append(synth.activations(SEED, STACK_WORKLOAD, 0, 40_000 + s, T, H))
            r = [synth.routing(SEED, STACK_WORKLOAD, l, 40_000 + s, T, E, K)
                 for l in range(STACK_LAYERS)]
            IDS.append(np.stack([a for a, _ in r]))
            W.append(np.stack([b for _, b in r]))
            by.append(sum((len(np.unique(a)) + 1) * eb for a, _ in r))
        X = torch.from_numpy(np.stack(X)).cuda()
        IDS = torch.from_numpy(np.stack(IDS).astype(np.int32)).cuda()
        W = torch.from_numpy(np.stack(W).astype(np.float32)).cuda()
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ws = stack.workspace(T)
        def call(s):
            dm.moe_stack(stack, X[s], IDS[s], W[s], out=out, ws=ws, stream=stream)

        for s in range(warmup):
            call(s)
        ms = back_to_back_us(torch, stream, steps, lambda k: call(warmup + k),
                             lambda: call(max(warmup - 1, 0))) / 1e3
        if not np.all(np.isfinite(out.cpu().numpy())):
            raise RuntimeError("non-finite stack output at bsz %d" % T)
        gb = float(np.mean(by[warmup:])) / 1e9
        res[str(T)] = {
            "ms_per_pass": ms,
            "tokens_per_s": T / (ms * 1e-3),
            "layer_tokens_per_s": T * STACK_LAYERS / (ms * 1e-3),
            "gb_per_pass": gb,
            "hbm_gbps": gb / (ms * 1e-3),
            "hbm_frac": gb / (ms * 1e-3) / HBM_PEAK_GBPS,
            "dtype": ("f32: fp9 weights decoded to fp16, f32 multiply-add" if T <= 2 else
                      "matrix-core path: fp16 weights (exact fp9 decode) times scaled fp16 "
                      "hi/lo activation pairs, f32 accumulation"),
        }
        log("stack bsz%d:" % T, json.dumps(res[str(T)]))
        del X, IDS, W, ws
    del stack, layers
    torch.cuda.empty_cache()
    return {"layers": STACK_LAYERS, "workload": "16 distinct fp9 layers (7168/2048, 256 routed + "
            "1 shared, top-8), RMS glue between layers, one native call per pass",
            "weights": "N(0, 0.02) drawn on the device, quantized by the device quantizer",
            "steps": steps, "by_bsz": res}


def cpu_baseline(n_tokens):
    """The float64 oracle on `n_tokens` bsz-1 steps of the same layer (1 thread)."""
    import oracle
    from bit_moe_expert_fp9_amd import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import OracleExperts
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ox = OracleExperts(SEED, WORKLOAD, 0, H, I)
    draws = [(synth.activations(SEED, WORKLOAD, 0, 20_000 + s, 1, H),
              *synth.routing(SEED, WORKLOAD, 0, 20_000 + s, 1, E, K)) for s in range(n_tokens)]
    need = set([E])
    for _, ids, _ in draws:
        need.update(int(i) for i in ids.ravel())
    log("cpu baseline: quantizing %d experts for the oracle (untimed)" % len(need))
    ox.prefetch(sorted(need))
    def timed(threads):
        ctx = threadpool_limits(threads) if threadpool_limits else None
        if ctx:
            ctx.__enter__()
        try:
            t0 = time.perf_counter()
            for x, ids, w in draws:
                oracle.moe_layer(ox, x, ids, w, E)
            return time.perf_counter() - t0
        finally:
            if ctx:
                ctx.__exit__(None, None, None)

    def timed_parallel(workers):
        """The same steps spread over `workers` threads, one BLAS thread each
        (numpy releases the GIL inside its array operations)."""
        from concurrent.futures import ThreadPoolExecutor
        ctx = threadpool_limits(1) if threadpool_limits else None
        if ctx:
            ctx.__enter__()
        try:
            t0 = time.perf_counter()
            with ThreadPoolExecutor(workers) as ex:
                list(ex.map(lambda d: oracle.moe_layer(ox, d[0], d[1], d[2], E), draws))
            return time.perf_counter() - t0
        finally:
            if ctx:
                ctx.__exit__(None, None, None)

    dt = timed(1)
    res = {"value": n_tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": "%d bsz-1 steps of the same 256+1-expert layer (fp9 decode + "
                     "float64 SwiGLU experts, %.1f s), numpy with 1 BLAS thread" % (n_tokens, dt)}
    # the same steps over the host's share of cores (at most 16): one step per
    # thread at a time, each with one BLAS thread
    cores = min(16, len(os.sched_getaffinity(0)))
    if cores > 1:
        dtn = timed_parallel(cores)
        res["all_cores"] = {"value": n_tokens / dtn, "cores": cores, "seconds": dtn,
                            "how": "the steps spread over %d threads, 1 BLAS thread each" % cores}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_moe_expert_fp9_amd as dm
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dm.lib()  # raises if the library is not built
    if args.calib_copy_mb:
        calib_copy(torch, args.calib_copy_mb)

    log("building layer: %d routed + 1 shared experts, fp9, %.2f GB" %
        (E, (E + 1) * 3 * H * I * 9 / 8 / 1e9))
    t0 = time.time()
    layer = dm.Layer(H, I, E, K).fill_synthetic(SEED, WORKLOAD, 0)
    log("layer ready in %.1f s" % (time.time() - t0))

    draws = 512
    r1 = time_layer(torch, dm, layer, 1, args.steps, args.warmup, draws)
    log("bsz1:", json.dumps(r1))
    r2 = None
    if args.bsz2:
        r2 = time_layer(torch, dm, layer, 2, args.steps, args.warmup, draws)
        log("bsz2:", json.dumps(r2))

    more = {}
    for T in [int(v) for v in args.more_bsz.split(",") if v.strip()]:
        r = time_layer(torch, dm, layer, T, min(args.steps, 300), min(args.warmup, 20), draws)
        more[str(T)] = {"us_per_layer": r["ms_per_step"] * 1e3,
                        "tokens_per_s": r["tokens_per_s"],
                        "mean_experts": r["mean_experts"],
                        "hbm_gbps": r["bytes_step"] / (r["ms_per_step"] * 1e-3) / 1e9,
                        "hbm_frac": r["bytes_step"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        log("bsz%d:" % T, json.dumps(more[str(T)]))

    st1 = time_stages(torch, dm, layer, 1, args.steps, args.warmup, draws)
    log("bsz1 stages:", json.dumps(st1))
    gu_b2b = time_gate_up_back_to_back(torch, dm, layer, 1, max(args.steps, 50), args.warmup, draws)
    log("bsz1 gate/up back to back:", json.dumps(gu_b2b))
    gemv = time_gemv_256x512(torch, dm) if args.extra else None

    dense = time_dense(torch, dm, min(args.steps, 300), 20) if args.dense else None
    pair = time_pair(torch, dm, layer, min(args.steps, 300), 20, draws) if args.bsz2 else None
    overlap = time_lane_overlap(torch, dm, layer, min(args.steps, 100), 10, draws) if args.extra else None
    extra = time_expert_and_partials(torch, dm, layer, min(args.steps, 300), 20) if args.extra else None
    prefill = {}
    for tok in [int(v) for v in args.prefill.split(",") if v.strip()]:
        prefill[str(tok)] = time_prefill(torch, dm, layer, tok, args.prefill_steps, 3)

    gbps = r1["bytes_step"] / (r1["ms_per_step"] * 1e-3) / 1e9
    ceil = read_ceiling(torch, dm, [int(r1["bytes_step"]), int(st1["gate_up_bytes"])])
    (lay_b, (lay_us, lay_gbps)), (gu_b, (gu_us, gu_gbps)) = sorted(ceil.items(), reverse=True)
    log("read ceiling: %d B in %.1f us (%.0f GB/s); %d B in %.1f us (%.0f GB/s)" %
        (lay_b, lay_us, lay_gbps, gu_b, gu_us, gu_gbps))
    res = {
        "metric": METRIC,
        "value": r1["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r1["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fp9 routed MoE layer, bsz 1 (7168/2048, 256 routed + 1 shared, top-8)",
            "hidden": H, "inter": I, "n_routed": E, "n_shared": 1, "top_k": K, "bsz": 1,
            "weights": "fp9 body+sign planes, resident in HBM",
            "layer_hbm_gbps": gbps,
            "layer_hbm_frac": gbps / HBM_PEAK_GBPS,
            "us_per_layer_p10_p50_p90": [r1["p10_us"], r1["p50_us"], r1["p90_us"]],
            "us_per_layer_with_events_mean": r1["call_us"],
            "bsz2_tokens_per_s": r2["tokens_per_s"] if r2 else None,
            "bsz2_hbm_gbps": (r2["bytes_step"] / (r2["ms_per_step"] * 1e-3) / 1e9) if r2 else None,
            "bsz2_ms_per_step": r2["ms_per_step"] if r2 else None,
            "layer_bsz": more or None,
            "layer_bsz_dtype": "matrix-core path: fp16 weights (exact fp9 decode) times "
                               "scaled fp16 hi/lo activation pairs, f32 accumulation",
            "gemv_256x512": gemv,
            "stages_us": {"k_gate_up": st1["gate_up_us"], "k_down": st1["down_us"]},
            "read_ceiling": {"what": "plain streaming read of the same byte count, one launch, "
                                     "fresh window, HIP events (duckmoe_read_probe)",
                             "layer_bytes": lay_b, "layer_us": lay_us, "layer_gbps": lay_gbps,
                             "gate_up_bytes": gu_b, "gate_up_us": gu_us, "gate_up_gbps": gu_gbps},
            "layer_frac_of_read_ceiling": gbps / lay_gbps,
            "dense_mlp": dense,
            "pair_two_tokens": pair,
            "lane_overlap": overlap,
            "expert_and_partials": extra,
            "prefill": prefill or None,
            "k_down_gbps": st1["down_gbps"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_gate_up (gate and up GEMVs + SwiGLU for every selected expert)",
            "achieved": gu_b2b["gbps"],
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gu_b2b["gbps"] / HBM_PEAK_GBPS,
            "avg_launch_us": gu_b2b["us"],
            "avg_launch_how": "launches back to back between two HIP events on their stream, "
                              "fresh routing each",
            "bytes_per_launch": gu_b2b["bytes"],
            "traffic": measured_traffic(),
            "read_ceiling_gbps": gu_gbps,
            "frac_of_read_ceiling": gu_b2b["gbps"] / gu_gbps,
            "with_events_us": st1["gate_up_us"],
        },
        "cpu_baseline": None,
    }
    if args.stack:
        res["stack"] = time_stack(torch, dm, args.stack_steps, 5)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
