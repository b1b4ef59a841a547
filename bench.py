"""Benchmark of the MoE layer on one MI355X.

Headline (`value`): one step = one full layer call (routing, grouped gate/up
GEMM + SwiGLU, down GEMM, combine) over the 4096-token prefill workload (two
chunks of 2048; H=2048, 256 experts top-8 + shared, I=512, 4-bit group-64
weights, Zipf(1.1) logit bias).  Inputs are resident in HBM before the timed
region.  Weight copies rotate every step (4 packed blobs, 1.8 GB, more than
the 256 MB Infinity Cache) so each step reads its weights from HBM, as
consecutive layers of a model would.  Each layer's workspace holds two chunk
areas, so the library runs the two chunks on two streams, both in flight.
`--warmup` steps, then exactly `--steps` timed steps with nothing else
enqueued and no kernel timing inside.

Run order (one process):
 1. one chunk at a time (the same layers over one chunk area), the pages' two
    ablations (host-synchronised routing, a separate dequant pass; both run
    one chunk at a time) and their tile-height ablation (fixed tiles of 16, 32
    or 64 rows) against the headline in alternating blocks of steps, each step
    stamped by events, so the legs share clock and thermal state; kept as raw
    samples, reported as p50 / p95 / mean per leg.  This also brings the
    device to the clocks it holds under this load;
 2. the headline: W warm-up steps, then K timed steps (the contract);
 3. the gate/up grouped GEMM event-stamped by its own dispatch over K more
    steps run one chunk at a time, so that no other kernel shares the device
    during a launch: its average duration for `roofline`;
 4. per-kernel averages, one extra pass per kernel, one chunk at a time;
 5. prefill of 512 tokens (near-uniform routing, every expert touched):
    tok/s and the share of 8 TB/s its algorithmic bytes reach;
 6. decode: cold (24 layer copies rotated, about 420 MB read between two
    calls on the same copy, so every call reads its weights from HBM) and warm
    (one copy, one token row, every byte cached) per-call latency; graph
    replay; the T = 1..8 sweep of both paths behind the row threshold and of
    the GEMV with the grouped GEMM's arithmetic (batch_invariant = 1); the
    decode `roofline` against 8 TB/s and against the streaming-read probe at
    the same byte count;
 7. probes: sustained 16-byte-per-lane streaming read over 4 GiB, and the
    MFMA-only rate and shader clock at the grouped GEMMs' occupancy;
 8. the CPU oracle on one pinned host core over a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
EXPERT_BYTES = 1769472      # packed gate + up + down of one expert at H=2048, I=512


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=4, help="packed weight blobs rotated per prefill step")
    p.add_argument("--decode-copies", type=int, default=24, help="layer copies rotated per cold decode call")
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--ablation-rounds", type=int, default=5)
    p.add_argument("--ablation-block", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--counter-pass", action="store_true",
                   help="short run for rocprofv3 --pmc passes: 4 prefill T=4096 steps, 8 prefill T=512 calls, "
                        "16 cold decode calls, then copies of known size that calibrate FETCH_SIZE/WRITE_SIZE; "
                        "prints no JSON line")
    return p.parse_args()


def source_digest(names=None):
    """First 16 hex digits of the SHA-256 of the library's sources (all of
    csrc/ in name order, or the listed files)."""
    d = os.path.join(ROOT, "bit_quantized_moe_router_amd", "csrc")
    h = hashlib.sha256()
    for name in (names or sorted(os.listdir(d))):
        h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()[:16]


def gemm_source_digest():
    """Digest of the sources that decide the grouped GEMM's memory traffic: the
    kernel file, the header of shared device helpers, and the routing kernels,
    which build the schedule that places its tiles on the XCDs."""
    return source_digest(["gemm.hip", "common.h", "route.hip"])


def traffic_from_profile():
    """HBM bytes per gate/up GEMM launch from the committed counter summary, if
    it was taken on the current GEMM source (else None)."""
    prof = os.path.join(ROOT, "profiles", "k_expert_gemm_traffic_prefill4096.md")
    try:
        fields = dict(l.split(":", 1) for l in open(prof).read().splitlines() if l.count(":") == 1 and " " not in l.split(":")[0])
        if fields.get("gemm_source_sha256_16", "").strip() != gemm_source_digest():
            return None
        return int(fields["gateup_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def stats(us):
    a = np.asarray(us, np.float64)
    return {"p50": round(float(np.percentile(a, 50)), 3), "p95": round(float(np.percentile(a, 95)), 3),
            "mean": round(float(a.mean()), 3), "n": int(a.size)}


def cpu_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


def cpu_baseline(case, budget_s):
    """The oracle as it stands, pinned to one host core: routing of one
    2048-token chunk, then the layer output of as many of its tokens as fit
    the time budget."""
    from oracle import oracle as orc

    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    try:
        x = case["x"][:2048]
        t0 = time.perf_counter()
        r = orc.route(x, case["w"]["router_w"], case["bias"], case["k"], 64)
        t_route = time.perf_counter() - t0
        n, t_ffn = 0, 0.0
        step = 4
        while t_ffn < max(1.0, budget_s - t_route) and n + step <= 2048:
            toks = np.arange(n, n + step, dtype=np.int32)
            t1 = time.perf_counter()
            orc.ffn_tokens(case["w"], case["k"], x, r["topk_ids"], r["topk_weights"], toks)
            t_ffn += time.perf_counter() - t1
            n += step
    finally:
        os.sched_setaffinity(0, set(allowed))
    per_tok = t_route / 2048 + t_ffn / n
    info = cpu_info()
    return {"value": round(1.0 / per_tok, 3), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"routing of one 2048-token chunk of the T=4096 workload ({t_route:.2f} s) + layer output "
                      f"of its first {n} tokens ({t_ffn:.2f} s), single-threaded C in float64, pinned to host "
                      f"core {core}; tok/s = 1 / (routing time per token + output time per token)",
            "nproc": info["nproc"], "cpu_model": info["model"]}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the layer has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_inputs as mi
    import bit_quantized_moe_router_amd as moe
    from bit_quantized_moe_router_amd.layer import MoELayer, to_dev

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(0)
    case = mi.make_case("prefill4096")
    w, k, T, H = case["w"], case["k"], case["T"], case["cfg"]["H"]
    I, Is, E = w["I"], w["Is"], w["E"]

    def clone_layer(src, max_tokens):
        lay = MoELayer.__new__(MoELayer)
        lay.__dict__.update(src.__dict__)
        lay.desc = moe.make_desc(src.H, src.E, src.k, src.I, src.Is)
        lay.packed = src.packed.clone()
        lay.router_w = src.router_w.clone()
        lay.max_tokens = max_tokens
        lay.ws = torch.empty(moe.moe_workspace_bytes(lay.desc, max_tokens), dtype=torch.uint8, device=dev)
        return lay

    # Workspaces sized for the whole 4096-token call: two chunk areas, so the
    # library keeps both 2048-token chunks in flight (one per stream).
    layers = [MoELayer(w, k, device=dev, max_tokens=T)]
    layers += [clone_layer(layers[0], T) for _ in range(a.copies - 1)]
    x = to_dev(case["x"], dev)
    bias = to_dev(case["bias"], dev)
    ys = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in layers]

    def step(i):
        lay = layers[i % len(layers)]
        lay.forward_prefill(x, bias, ys[i % len(layers)])

    def one_chunk_views():
        # The same layers over the first chunk area of their workspace only: the
        # library then runs the chunks one after the other on the caller's
        # stream (per-kernel timing of each kernel alone on the device).
        out = []
        for lay in layers:
            v = MoELayer.__new__(MoELayer)
            v.__dict__.update(lay.__dict__)
            v.desc = moe.make_desc(lay.H, lay.E, lay.k, lay.I, lay.Is)
            v.max_tokens = 2048
            v.ws = lay.ws[:moe.moe_workspace_bytes(v.desc, 2048)]
            out.append(v)
        return out

    serial = one_chunk_views()

    def step_serial(i):
        serial[i % len(serial)].forward_prefill(x, bias, ys[i % len(serial)])

    def set_all(**kw):
        for lay in layers:
            lay.set_desc(**kw)

    if a.counter_pass:
        # 4 prefill T=4096 steps (8 chunks), 8 prefill T=512 calls, 16 cold
        # decode T=1 calls, then copies of known size.
        for i in range(4):
            step_serial(i)
        x512 = to_dev(mi.make_case("prefill512")["x"], dev)
        for i in range(8):
            layers[i % len(layers)].forward_prefill(x512, None, ys[0][:512])
        dl = list(layers) + [clone_layer(layers[0], 8) for _ in range(16 - len(layers))]
        xd = to_dev(mi.gen_x(16, H, 4242), dev)
        for i in range(16):
            dl[i].forward_decode(xd[i:i + 1], None, ys[0][:1])
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.mul_(0).add_(src)  # mul_: reads and writes 256 MiB; add_: reads 512 MiB, writes 256 MiB
        torch.cuda.synchronize()
        print("counter pass done", flush=True)
        return

    # The separate-dequant and fixed-tile legs need larger workspaces: sized once here.
    set_all(dequant_pass=1)
    set_all(dequant_pass=0)
    set_all(tile_rows=16)
    set_all(tile_rows=0)
    serial = one_chunk_views()

    # ---- 1. ablations in alternating blocks, per-step samples ----
    # One chunk at a time (the workspace's first chunk area only) against two
    # in flight; host-synchronised routing and the separate dequant pass (both
    # one chunk at a time by construction, so also compared with that leg);
    # fixed tiles of 16, 32 or 64 rows against the default (128-row tiles whose
    # row fragments follow each expert's load, long ones cut): the pages' tile
    # height ablation.  All legs give the same bits.
    legs = [("headline", {}, step), ("serial_chunks", {}, step_serial),
            ("host_sync_routing", {"host_sync_routing": 1}, step), ("dequant_pass", {"dequant_pass": 1}, step),
            ("fixed_tiles_16", {"tile_rows": 16}, step), ("fixed_tiles_32", {"tile_rows": 32}, step),
            ("fixed_tiles_64", {"tile_rows": 64}, step)]
    samples = {name: [] for name, _, _ in legs}
    B = a.ablation_block
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(B + 1)]
    it = 0
    for rnd in range(a.ablation_rounds):
        for name, kw, fn in legs:
            set_all(**kw)
            for _ in range(2):  # untimed: the first step after a switch
                fn(it)
                it += 1
            torch.cuda.synchronize()
            evs[0].record(stream)
            for j in range(B):
                fn(it)
                it += 1
                evs[j + 1].record(stream)
            torch.cuda.synchronize()
            samples[name] += [1000.0 * evs[j].elapsed_time(evs[j + 1]) for j in range(B)]
            set_all(host_sync_routing=0, dequant_pass=0, tile_rows=0)
    leg_stats = {name: stats(v) for name, v in samples.items()}
    base50 = leg_stats["headline"]["p50"]
    serial50 = leg_stats["serial_chunks"]["p50"]

    # ---- 2. the headline: W warm-up steps, then exactly K timed steps ----
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t_wall = time.perf_counter()
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = e0.elapsed_time(e1) / a.steps

    # ---- 3. the gate/up grouped GEMM stamped by its own dispatch, alone on
    # the device (chunks one at a time, so no other kernel shares its time) ----
    moe.moe_profile_reset()
    moe.moe_profile_enable(1 << moe.K_GATEUP_GEMM)
    for i in range(a.steps):
        step_serial(i)
    torch.cuda.synchronize()
    moe.moe_profile_enable(0)
    tot, n = moe.moe_profile_read(moe.K_GATEUP_GEMM)
    kern = {"k_gateup_gemm": {"avg_us": round(1000.0 * tot / n, 3), "launches": n}}

    def breakdown(run, kids):
        """Per-kernel average durations, one extra pass per kernel (outside the timed region)."""
        out = {}
        for kid in kids:
            moe.moe_profile_reset()
            moe.moe_profile_enable(1 << kid)
            run()
            torch.cuda.synchronize()
            moe.moe_profile_enable(0)
            t, c = moe.moe_profile_read(kid)
            if c:
                out[moe.KERNEL_NAMES[kid]] = {"avg_us": round(1000.0 * t / c, 3), "launches": c}
        return out

    def prefill_pass():
        for i in range(a.steps):
            step_serial(i)

    kern_all = breakdown(prefill_pass, [moe.K_LOGITS, moe.K_TOPK, moe.K_META, moe.K_DOWN_GEMM, moe.K_COMBINE])
    set_all(dequant_pass=1)
    # (the separate dequant pass always runs one chunk at a time)
    kern_dq = breakdown(lambda: [step(i) for i in range(a.steps)], [moe.K_DEQUANT, moe.K_GATEUP_GEMM, moe.K_DOWN_GEMM])
    set_all(dequant_pass=0)

    Tc = 2048
    flop_gateup = 2.0 * (Tc * k + Tc) * H * (2 * I)
    g = kern["k_gateup_gemm"]
    achieved = flop_gateup / (g["avg_us"] * 1e-6) / 1e12
    flop_down = 2.0 * (Tc * k + Tc) * I * H
    down_tf = flop_down / (kern_all["k_down_gemm"]["avg_us"] * 1e-6) / 1e12

    # ---- 5. prefill of 512 tokens (near-uniform routing) ----
    c512 = mi.make_case("prefill512")
    x512 = to_dev(c512["x"], dev)
    y512 = torch.empty((512, H), dtype=torch.float32, device=dev)
    r512 = layers[0].route(x512, None)
    torch.cuda.synchronize()
    touched = int((r512["expert_counts"] > 0).sum().item())
    rows512 = 512 * k + 512
    bytes512 = ((touched + 1) * EXPERT_BYTES + 4 * E * H + 2 * 512 * H + 2 * 2 * rows512 * I + 4 * 512 * H)
    flop512 = 512 * (k + 1) * 6 * H * I + 2 * 512 * E * H

    def p512(i):
        layers[i % len(layers)].forward_prefill(x512, None, y512)

    for i in range(10):
        p512(i)
    torch.cuda.synchronize()
    ev5 = [torch.cuda.Event(enable_timing=True) for _ in range(101)]
    ev5[0].record(stream)
    for i in range(100):
        p512(i)
        ev5[i + 1].record(stream)
    torch.cuda.synchronize()
    us512 = [1000.0 * ev5[i].elapsed_time(ev5[i + 1]) for i in range(100)]
    s512 = stats(us512)
    prefill512 = {"us_per_call": s512, "tok_s": round(512 / (s512["p50"] * 1e-6), 1),
                  "experts_touched": touched, "algorithmic_bytes": bytes512, "flop": flop512,
                  "hbm_GBs": round(bytes512 / (s512["p50"] * 1e-6) / 1e9, 1),
                  "hbm_frac": round(bytes512 / (s512["p50"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                  "weight_copies_rotated": len(layers)}

    # ---- 6. decode ----
    dlayers = list(layers) + [clone_layer(layers[0], 8) for _ in range(max(0, a.decode_copies - len(layers)))]
    NC = len(dlayers)
    NX = 256
    xd_all = to_dev(mi.gen_x(NX, H, 4242), dev)
    yd = torch.empty((8, H), dtype=torch.float32, device=dev)

    def dcall(i, T=1, cold=True):
        lay = dlayers[i % NC] if cold else dlayers[0]
        j = i % NX if cold else 0
        lay.forward_decode(xd_all[j:j + T], None, yd[:T])

    def decode_b2b(T=1, cold=True, n=None):
        n = n or a.decode_steps
        for i in range(10):
            dcall(i, T, cold)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for i in range(n):
            dcall(10 + i, T, cold)
        d1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * d0.elapsed_time(d1) / n

    def decode_percall(T=1, cold=True, n=None):
        n = n or a.decode_steps
        for i in range(10):
            dcall(i, T, cold)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for i in range(n):
            dcall(10 + i, T, cold)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return stats([1000.0 * ev[i].elapsed_time(ev[i + 1]) for i in range(n)])

    for lay in dlayers:
        lay.set_desc(gemv_max_rows=-1)
    dec_us = decode_b2b(1, True)
    dec_cold = decode_percall(1, True)
    dec_warm_b2b = decode_b2b(1, False)
    dec_warm = decode_percall(1, False)

    def graph_decode_us(T=1, n=48, reps=20):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for i in range(n):
                dcall(i, T, True)
        gph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            gph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * g0.elapsed_time(g1) / (reps * n)

    dec_graph_us = graph_decode_us(1)
    dkern = breakdown(lambda: [dcall(i, 1, True) for i in range(a.decode_steps)],
                      [moe.K_LOGITS, moe.K_GATEUP_GEMV, moe.K_DOWN_GEMV])

    # Probe: the same byte counts streamed by the 16-byte-per-lane read
    # kernel, cold (rotating over more than the Infinity Cache).
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def probe_read(nbytes, nbuf, n=200, max_wgs=8192):
        nbytes = (nbytes + 15) // 16 * 16
        bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(nbuf)]
        for i in range(10):
            moe.moe_probe_stream_read(bufs[i % nbuf], nbytes, sink, max_wgs)
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(stream)
        for i in range(n):
            moe.moe_probe_stream_read(bufs[i % nbuf], nbytes, sink, max_wgs)
        p1.record(stream)
        torch.cuda.synchronize()
        b2b = 1000.0 * p0.elapsed_time(p1) / n
        moe.moe_profile_reset()
        moe.moe_profile_enable(1 << moe.K_PROBE_READ)
        for i in range(n):
            moe.moe_probe_stream_read(bufs[i % nbuf], nbytes, sink, max_wgs)
        torch.cuda.synchronize()
        moe.moe_profile_enable(0)
        t, c = moe.moe_profile_read(moe.K_PROBE_READ)
        del bufs
        return {"bytes": nbytes, "back_to_back_us": round(b2b, 3), "kernel_us": round(1000.0 * t / c, 3),
                "back_to_back_GBs": round(nbytes / b2b / 1e3, 1), "kernel_GBs": round(nbytes / (1000.0 * t / c) / 1e3, 1)}

    layer_bytes = 4 * E * H + (k + 1) * EXPERT_BYTES + 2 * H + 4 * H  # the layer's algorithmic bytes at T=1
    ex_bytes = (k + 1) * EXPERT_BYTES  # the experts kernel's weight stream
    pr_layer = probe_read(layer_bytes, max(2, (600 << 20) // layer_bytes))
    pr_ex = probe_read(ex_bytes, max(2, (600 << 20) // ex_bytes))
    gemv_ex = dkern.get("k_gemv_experts")
    layer_gbs = layer_bytes / (dec_us * 1e-6) / 1e9
    dec_roof = {"bound": "hbm", "achieved": round(layer_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(layer_gbs / PEAK_HBM_GBS, 4), "bytes_per_call": layer_bytes,
                "achievable_GBs": pr_layer["back_to_back_GBs"],
                "frac_of_achievable": round(layer_gbs / pr_layer["back_to_back_GBs"], 4),
                "achievable_probe": pr_layer,
                "experts_kernel": {"bytes": ex_bytes,
                                   "GBs": round(ex_bytes / (gemv_ex["avg_us"] * 1e-6) / 1e9, 1) if gemv_ex else None,
                                   "probe_kernel_GBs": pr_ex["kernel_GBs"],
                                   "frac_of_probe": round(ex_bytes / (gemv_ex["avg_us"] * 1e-6) / 1e9 /
                                                          pr_ex["kernel_GBs"], 4) if gemv_ex else None}}

    # Row-count sweep, cold: the GEMV forced, the grouped GEMM forced, and the
    # GEMV with the grouped GEMM's arithmetic (batch_invariant = 1) forced.
    sweep = {}
    for T_ in (1, 2, 3, 4, 5, 6, 7, 8):
        row = {}
        for name, r, bi in (("gemv", 8, 0), ("gemm", 0, 0), ("gemv_batch_invariant", 8, 1)):
            for lay in dlayers:
                lay.set_desc(gemv_max_rows=r, batch_invariant=bi)
            row[name] = round(decode_b2b(T_, True, 100), 2)
        sweep[str(T_)] = row
    for lay in dlayers:
        lay.set_desc(gemv_max_rows=-1, batch_invariant=0)
    del dlayers[len(layers):]

    # ---- 7. probes: sustained streaming read, MFMA-only rate and clock ----
    pr_big = probe_read(4 << 30, 1, n=5)
    cus = props.multi_processor_count
    wgs = cus * 2
    clocks = torch.zeros(2 * wgs, dtype=torch.int64, device=dev)
    iters = 20000
    for _ in range(3):
        moe.moe_probe_mfma_rate(iters, wgs, clocks, sink)
    torch.cuda.synchronize()
    moe.moe_profile_reset()
    moe.moe_profile_enable(1 << moe.K_PROBE_MFMA)
    for _ in range(5):
        moe.moe_probe_mfma_rate(iters, wgs, clocks, sink)
    torch.cuda.synchronize()
    moe.moe_profile_enable(0)
    t, c = moe.moe_profile_read(moe.K_PROBE_MFMA)
    mfma_us = 1000.0 * t / c
    ck = clocks.cpu().view(-1, 2).double()
    mfma_probe = {"TFLOPs": round(wgs * 4 * iters * 8 * 32768 / mfma_us / 1e6, 1),
                  "sclk_MHz_under_mfma_load": round(float((ck[:, 0] / ck[:, 1]).median()) * 100.0, 1),
                  "note": "v_mfma_f32_32x32x16_f16 only, 8 independent chains, two waves per SIMD"}

    rocm = ""
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    rec = {
        "metric": "MoE-layer tok/s @T=4096 prefill; µs/layer @T=1 decode; % HBM/MFMA roofline",
        "value": round(T / (ms_per_step / 1000.0), 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands, fp32 accumulation (bf16 activations and scales, 4-bit codes)",
        "data": "synthetic",
        "config": {"workload": "MoE layer prefill T=4096 in 2x2048-token chunks, H=2048, E=256 top-8 + 1 shared, "
                               "I=Is=512, SwiGLU, 4-bit codes g64 bf16 scale/bias, Zipf(1.1) logit bias",
                   "weight_copies_rotated": a.copies, "wall_s_timed": round(t_wall, 4)},
        "roofline": {"bound": "mfma", "kernel": "k_gateup_gemm", "achieved": round(achieved, 2),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": traffic_from_profile(), "flop_per_launch": flop_gateup, "avg_us": g["avg_us"],
                     "frac_of_mfma_probe": round(achieved / mfma_probe["TFLOPs"], 4)},
        "headline_samples_us_per_step": leg_stats["headline"],
        "kernels_us": dict(kern, **kern_all),
        "down_gemm_tflops": round(down_tf, 2),
        "ablation_serial_chunks": dict(leg_stats["serial_chunks"],
                                       slowdown_p50=round(leg_stats["serial_chunks"]["p50"] / base50, 4)),
        "ablation_host_sync_routing": dict(leg_stats["host_sync_routing"],
                                           slowdown_p50=round(leg_stats["host_sync_routing"]["p50"] / base50, 4),
                                           slowdown_vs_serial_chunks_p50=round(
                                               leg_stats["host_sync_routing"]["p50"] / serial50, 4)),
        "ablation_dequant_pass": dict(leg_stats["dequant_pass"],
                                      slowdown_p50=round(leg_stats["dequant_pass"]["p50"] / base50, 4),
                                      slowdown_vs_serial_chunks_p50=round(leg_stats["dequant_pass"]["p50"] / serial50, 4),
                                      kernels_us=kern_dq),
        "ablation_fixed_tiles": {str(bm): dict(leg_stats[f"fixed_tiles_{bm}"],
                                               slowdown_p50=round(leg_stats[f"fixed_tiles_{bm}"]["p50"] / base50, 4))
                                 for bm in (16, 32, 64)},
        "ablation_protocol": f"{a.ablation_rounds} rounds x {len(legs)} legs x {B} event-stamped steps, legs "
                             "alternating, 2 untimed steps after each switch; us per step",
        "prefill512": prefill512,
        "decode": {"us_per_layer": round(dec_us, 3), "T": 1, "cold_per_call_us": dec_cold,
                   "warm_us_per_layer": round(dec_warm_b2b, 3), "warm_per_call_us": dec_warm,
                   "graph_us_per_layer": round(dec_graph_us, 3), "kernels_us": dkern, "roofline": dec_roof,
                   "layer_copies_rotated": NC, "token_rows_rotated": NX,
                   "sweep_us_per_layer_cold": sweep,
                   "batch_invariant_us_per_layer": sweep["1"]["gemv_batch_invariant"], "default_gemv_max_rows": moe.moe_default_gemv_max_rows()},
        "probes": {"stream_read_4GiB": pr_big, "mfma": mfma_probe},
        "env": {"gpu": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": cus, "rocm": rocm,
                "torch": torch.__version__, "hip_runtime": torch.version.hip,
                "libmoe_source_sha256_16": source_digest(), "bench_sha256_16":
                    hashlib.sha256(open(os.path.abspath(__file__), "rb").read()).hexdigest()[:16]},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, a.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
