"""Benchmark of the MoE layer on one MI355X.

One step = one full layer call (routing, grouped gate/up GEMM + SwiGLU, down
GEMM + combine) over the 4096-token prefill workload (two chunks of 2048;
H=2048, 256 experts top-8 + shared, I=512, 4-bit group-64 weights, Zipf(1.1)
logit bias).  Inputs are resident in HBM before the timed region.  Weight
copies rotate every step (4 distinct packed blobs, 1.8 GB > the 256 MB
Infinity Cache) so each step reads its weights from HBM, as consecutive layers
of a model would.

The timed region runs with no kernel timing in it (the events that stamp a
kernel's own start and end cost about 6 us per stamped launch).  A second
timed pass of the same K steps, with the dominant kernel (the gate/up grouped
GEMM) event-stamped on its launch stream, gives that kernel's average
duration for the roofline.

Also reported on the same line: the T=1 decode layer (GEMV path) in
microseconds per layer, eager and replayed from a HIP graph, per-kernel
averages from extra passes, and the CPU oracle timed on a bounded sample on
this host.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=4, help="distinct weight blobs rotated per step")
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--counter-pass", action="store_true",
                   help="short run for rocprofv3 --pmc passes: 8 prefill steps, then copies of known size "
                        "that calibrate FETCH_SIZE/WRITE_SIZE; prints no JSON line")
    return p.parse_args()


def gemm_source_digest():
    """First 16 hex digits of the SHA-256 of the grouped GEMM's sources (the
    kernel file, then the header of shared device helpers)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("gemm.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "bit_quantized_moe_router_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per gate/up GEMM launch from the committed counter summary, if
    it was taken on the current GEMM source (else None)."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "k_expert_gemm_traffic_prefill4096.md")
    try:
        fields = dict(l.split(":", 1) for l in open(prof).read().splitlines() if l.count(":") == 1 and " " not in l.split(":")[0])
        digest = gemm_source_digest()
        if fields.get("gemm_source_sha256_16", "").strip() != digest:
            return None
        return int(fields["gateup_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(case, budget_s):
    """The oracle as it stands on one host core: routing of one 2048-token chunk,
    then the layer output of as many of its tokens as fit the time budget."""
    from oracle import oracle as orc

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
    per_tok = t_route / 2048 + t_ffn / n
    return {"value": round(1.0 / per_tok, 3), "unit": "tok/s", "cores": 1, "kind": "oracle",
            "sample": f"routing of one 2048-token chunk ({t_route:.2f} s) + layer output of its first {n} "
                      f"tokens ({t_ffn:.2f} s), single-threaded C, float64"}


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
    case = mi.make_case("prefill4096")
    w, k, T, H = case["w"], case["k"], case["T"], case["cfg"]["H"]
    I, Is, E = w["I"], w["Is"], w["E"]
    layers = [MoELayer(w, k, device=dev, max_tokens=2048)]
    for _ in range(a.copies - 1):
        lay = MoELayer.__new__(MoELayer)
        lay.__dict__.update(layers[0].__dict__)
        lay.packed = layers[0].packed.clone()
        lay.router_w = layers[0].router_w.clone()
        lay.ws = torch.empty_like(layers[0].ws)
        layers.append(lay)
    x = to_dev(case["x"], dev)
    bias = to_dev(case["bias"], dev)
    ys = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in layers]
    stream = torch.cuda.current_stream()

    def step(i):
        lay = layers[i % len(layers)]
        lay.forward_prefill(x, bias, ys[i % len(layers)])

    if a.counter_pass:
        for i in range(8):
            step(i)
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.mul_(0).add_(src)  # mul_: reads and writes 256 MiB; add_: reads 512 MiB, writes 256 MiB
        torch.cuda.synchronize()
        print("counter pass done", flush=True)
        return

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps, nothing else enqueued.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t_wall = time.perf_counter()
    for i in range(a.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / a.steps

    # The same K steps again, the gate/up grouped GEMM event-stamped by its
    # own dispatch on this stream: its average duration for the roofline.
    moe.moe_profile_reset()
    moe.moe_profile_enable(1 << moe.K_GATEUP_GEMM)
    for i in range(a.steps):
        step(i)
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
            step(i)

    kern_all = breakdown(prefill_pass, [moe.K_LOGITS, moe.K_TOPK, moe.K_META, moe.K_DOWN_GEMM, moe.K_COMBINE])

    # Measurement of the design the pages argue against: each chunk's routing
    # read back by the host before the GEMM launches (same kernels).
    for lay in layers:
        lay.set_desc(host_sync_routing=1)
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    h0, h1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0.record(stream)
    for i in range(a.steps):
        step(i)
    h1.record(stream)
    torch.cuda.synchronize()
    ms_sync = h0.elapsed_time(h1) / a.steps
    for lay in layers:
        lay.set_desc(host_sync_routing=0)

    # Measurement of the other design the pages argue against: the active
    # experts rebuilt as fp16 in HBM by a pass of their own, then the grouped
    # GEMMs read fp16 weights (same rounding, same results).
    for lay in layers:
        lay.set_desc(dequant_pass=1)
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    h0.record(stream)
    for i in range(a.steps):
        step(i)
    h1.record(stream)
    torch.cuda.synchronize()
    ms_dq = h0.elapsed_time(h1) / a.steps
    kern_dq = breakdown(prefill_pass, [moe.K_DEQUANT, moe.K_GATEUP_GEMM, moe.K_DOWN_GEMM])
    for lay in layers:
        lay.set_desc(dequant_pass=0)

    # Dominant kernel: gate/up grouped GEMM, one launch per 2048-token chunk.
    Tc = 2048
    flop_gateup = 2.0 * (Tc * k + Tc) * H * (2 * I)
    g = kern["k_gateup_gemm"]
    achieved = flop_gateup / (g["avg_us"] * 1e-6) / 1e12
    flop_down = 2.0 * (Tc * k + Tc) * I * H
    d = kern_all["k_down_gemm"]
    down_tf = flop_down / (d["avg_us"] * 1e-6) / 1e12

    # Decode (GEMV path at T=1) on the same layer copies.  Every call takes
    # another of 64 seeded token rows, so the experts change from call to call
    # and the weights come from HBM, not from the Infinity Cache.
    NX = 64
    xd_all = to_dev(mi.gen_x(NX, H, 4242), dev)
    xds = [xd_all[i:i + 1] for i in range(NX)]
    yd = torch.empty((8, H), dtype=torch.float32, device=dev)

    def decode_run(n, T=1):
        for i in range(n):
            j = (i * 8) % NX
            xin = xds[j] if T == 1 else xd_all[j:j + T]
            layers[i % len(layers)].forward_decode(xin, None, yd[:T])

    def timed_decode(T=1):
        decode_run(10, T)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        decode_run(a.decode_steps, T)
        d1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * d0.elapsed_time(d1) / a.decode_steps

    for lay in layers:
        lay.set_desc(gemv_max_rows=-1)
    dec_us = timed_decode(1)

    # The same decode calls captured in a HIP graph (64 calls over the rotated
    # layer copies and token rows), then replayed: the host-side launch cost
    # is gone, the kernels' own boundaries remain.
    def graph_decode_us(T=1, n=64, reps=20):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                j = (i * 8) % NX
                xin = xds[j] if T == 1 else xd_all[j:j + T]
                layers[i % len(layers)].forward_decode(xin, None, yd[:T])
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        return 1000.0 * g0.elapsed_time(g1) / (reps * n)

    dec_graph_us = graph_decode_us(1)
    dkern = breakdown(lambda: decode_run(a.decode_steps), [moe.K_LOGITS, moe.K_META, moe.K_GATEUP_GEMV,
                                                           moe.K_DOWN_GEMV])
    blk = 1152
    # The experts kernel streams gate/up and down of the 8 routed experts and
    # the shared one; the reduce kernel reads the partial output rows.
    ex_bytes = 9 * ((I // 32) * (H // 64) * 2 + (H // 32) * (I // 64)) * blk
    red_bytes = (k + 1) * (I // 32) * H * 4 + H * 4
    gemv_ex = dkern.get("k_gemv_experts")
    gemv_red = dkern.get("k_gemv_reduce")

    # Reference for "achievable" at these sizes: a device-to-device copy of the
    # same number of bytes (read + write counted), over rotating buffers.
    def copy_gbs(nbytes):
        n = nbytes // 2
        srcs = [torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1) for _ in range(16)]
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
        for i in range(8):
            dst.copy_(srcs[i % 16])
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(200):
            dst.copy_(srcs[i % 16])
        c1.record(stream)
        torch.cuda.synchronize()
        return round(2 * n * 2 / (c0.elapsed_time(c1) / 200 * 1e-3) / 1e9, 1)

    dec_roof = {
        "experts_gemv_bytes": ex_bytes,
        "experts_gemv_GBs": round(ex_bytes / (gemv_ex["avg_us"] * 1e-6) / 1e9, 1) if gemv_ex else None,
        "reduce_bytes": red_bytes,
        "reduce_GBs": round(red_bytes / (gemv_red["avg_us"] * 1e-6) / 1e9, 1) if gemv_red else None,
        "copy_GBs_same_bytes_experts": copy_gbs(ex_bytes),
        "layer_bytes": ex_bytes + 4 * E * H + red_bytes + 2 * H,
        "layer_GBs": round((ex_bytes + 4 * E * H + red_bytes + 2 * H) / (dec_us * 1e-6) / 1e9, 1),
        "peak_GBs": PEAK_HBM_GBS,
    }
    # Row-count sweep of both paths (GEMV forced, grouped GEMM forced): the
    # evidence behind the default row threshold.
    sweep = {}
    for T_ in (1, 2, 3, 4, 5, 6, 7, 8):
        row = {}
        for name, r in (("gemv", 8), ("gemm", 0)):
            for lay in layers:
                lay.set_desc(gemv_max_rows=r)
            row[name] = round(timed_decode(T_), 2)
        sweep[str(T_)] = row
    for lay in layers:
        lay.set_desc(gemv_max_rows=-1)

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "MoE layer prefill T=4096 in 2x2048-token chunks, H=2048, E=256 top-8 + 1 shared, "
                               "I=Is=512, SwiGLU, 4-bit codes g64 bf16 scale/bias, Zipf(1.1) logit bias",
                   "weight_copies_rotated": a.copies, "wall_s_timed": round(t_wall, 4)},
        "roofline": {"bound": "mfma", "kernel": "k_gateup_gemm", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile(), "flop_per_launch": flop_gateup, "avg_us": g["avg_us"]},
        "kernels_us": dict(kern, **kern_all),
        "down_gemm_tflops": round(down_tf, 2),
        "ablation_host_sync_routing": {"ms_per_step": round(ms_sync, 4), "tok_s": round(T / (ms_sync / 1000.0), 1),
                                       "slowdown_vs_value": round(ms_sync / ms_per_step, 4)},
        "ablation_dequant_pass": {"ms_per_step": round(ms_dq, 4), "tok_s": round(T / (ms_dq / 1000.0), 1),
                                  "slowdown_vs_value": round(ms_dq / ms_per_step, 4), "kernels_us": kern_dq},
        "decode": {"us_per_layer": round(dec_us, 3), "T": 1, "graph_us_per_layer": round(dec_graph_us, 3),
                   "kernels_us": dkern, "roofline": dec_roof,
                   "sweep_us_per_layer": sweep, "default_gemv_max_rows": moe.moe_default_gemv_max_rows()},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case, a.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
