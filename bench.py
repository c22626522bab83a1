#!/usr/bin/env python3
"""Benchmark: DeepSeek-V2-shaped absorbed-MLA decode on one MI355X.

One step = the whole decode path for one batch, one library call: the latent
attention kernel (which plans the batch's split over workers itself), then one
kernel that merges the rows cut over several workers (log-sum-exp combine) and
applies the W_UV up-projection
(B=64 sequences x 4096 cached positions, H=128, d_c=512, d_r=64, d_v=128,
bf16 storage, fp32 accumulation). Inputs are synthetic (seeded), resident in
HBM before timing, and rotated over several independent copies so the
256 MiB Infinity Cache cannot serve a step from a previous one.

Prints ONE JSON line. `value` is latent head-tokens attended per second
(B*H*seq per step). `roofline` is for the dominant kernel (the latent
attention kernel), timed with two HIP events passed with its launch on its own
stream (they take the start and end of its dispatch) on every n-th timed step
(--event-every, default 5); its algorithmic bytes are the cache read once, the
absorbed queries and the latent output.
`entry_points_ms` gives each entry point's own time (median and min over
blocks of back-to-back calls, run before the warm-up steps). `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workload on this host.
`workloads` holds the other measured workloads, each with its own roofline:
the ragged paged decode (B=128, lengths U[1, 32768], 64-position pages), the
causal prefill B=2 S=4096 H=128 in both forms (absorbed chain and expanded
per-head form), the fused cache append, full absorption, the gated MLA
layer, and the decode step with a logit spike that makes one segment redo
its softmax (--headline-only skips them; --skip-headline runs only them,
--only picks some).

    python bench.py [--steps K] [--warmup W] [--headline-only | --skip-headline] [--only a,b]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "head_latent_attention_09_amd", "csrc", "mla_attn.hip")
TRAFFIC_FILE = os.path.join(PROFILE_DIR, "latent_attention_decode_b64_h128_s4096_traffic.json")

B, H, S, D_C, D_R, D_V = 64, 128, 4096, 512, 64, 128
W = D_C + D_R
ESIZE = 2


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the attention kernel keeps speeding up for about 40 ms (some 350 steps)
    # of sustained load after idle (clock ramp): the default warm-up covers it
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=600)
    p.add_argument("--copies", type=int, default=3, help="rotated input copies")
    p.add_argument("--event-every", type=int, default=5,
                   help="record the attention kernel's timing events on every n-th timed step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    p.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    p.add_argument("--only", default="", help="comma-separated subset of the other workloads")
    p.add_argument("--skip-headline", action="store_true",
                   help="run only the other workloads (for profiling them without the headline's kernels)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    return p.parse_args()


def cpu_baseline(case, budget_s):
    """fp64 numpy oracle (latent definition + per-head up-projection) on whole
    sequences of the same workload until the time budget is spent."""
    import oracle as O
    import workloads as G
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = min(threads, len(os.sched_getaffinity(0)))
    wuv = G.to_f64(case.w_uv, G.BF16)
    done, t0 = 0, time.perf_counter()
    nseq = 0
    while True:
        b = nseq % case.B
        lat = G.to_f64(case.cache[b], G.BF16)
        q = G.to_f64(case.q[b], G.BF16)
        out, _ = O.latent_attention(q, lat, D_C, case.kq_scale, int(case.lens[b]))
        O.up_project(out[None], wuv)
        done += H * int(case.lens[b])
        nseq += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": done / el, "unit": "latent tokens/s (B*H*seq)", "cores": cores, "kind": "oracle",
            "sample": f"{nseq} whole sequences (H={H}, seq={S}) of the benchmark workload, "
                      f"fp64 numpy latent definition + up-projection, {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(decode would shard by sequence); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_latent_attention_09_amd as M
    import workloads as G

    assert torch.cuda.is_available(), "no HIP device"
    dev = torch.device("cuda:0")
    if args.skip_headline:
        import bench_workloads as BW
        line = {"headline": "skipped", "workloads": BW.run_all(M, G, torch, dev, args, time_entry)}
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps(line), flush=True)
        return
    case = G.config3_decode_bf16(0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q0, cache0, wuv = to_dev(case.q), to_dev(case.cache), to_dev(case.w_uv)
    lens = torch.from_numpy(case.lens).to(dev)
    sets = []
    for i in range(args.copies):
        q = q0 if i == 0 else q0.clone()
        cache = cache0 if i == 0 else cache0.clone()
        sets.append(dict(q=q, cache=cache, out=torch.empty((B, H, D_C), dtype=torch.bfloat16, device=dev),
                         lse=torch.empty((B, H), dtype=torch.float32, device=dev),
                         v=torch.empty((B, H, D_V), dtype=torch.bfloat16, device=dev)))
    G_workers = M.default_workers()
    ws = torch.empty(M.decode_up_v_workspace_bytes(B, H, D_C, G_workers), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        # one call: attention over the latent cache, then the split-row merge
        # fused with the W_UV up-projection
        s = sets[i % len(sets)]
        M.latent_decode_up_v(s["q"], s["cache"], lens, D_C, case.kq_scale, wuv, out=s["v"], lse=s["lse"],
                             workspace=ws, timing_events=ev)

    # Per entry point: blocks of back-to-back calls between two events (the
    # events' own cost is spread over the block); median and min over blocks.
    # These ~300 calls run before the warm-up steps and also carry the GPU
    # through most of its clock ramp after idle; the fused entry, the step's
    # own call, is timed last.
    ws_two = torch.empty(M.decode_workspace_bytes(B, H, D_C, G_workers), dtype=torch.uint8, device=dev)
    two_call = time_entry(
        torch, stream, lambda i: M.latent_decode(sets[i % len(sets)]["q"], sets[i % len(sets)]["cache"], lens,
                                                 D_C, case.kq_scale, out=sets[i % len(sets)]["out"],
                                                 lse=sets[i % len(sets)]["lse"], workspace=ws_two))
    upv = time_entry(torch, stream, lambda i: M.up_v(sets[i % len(sets)]["out"], wuv, out=sets[i % len(sets)]["v"]))
    fused = time_entry(
        torch, stream, lambda i: M.latent_decode_up_v(sets[i % len(sets)]["q"], sets[i % len(sets)]["cache"],
                                                      lens, D_C, case.kq_scale, wuv, out=sets[i % len(sets)]["v"],
                                                      lse=sets[i % len(sets)]["lse"], workspace=ws))
    entry = {"latent_decode_up_v (attention + merge fused with W_UV)": fused,
             "latent_decode (attention + combine)": two_call,
             "up_v (W_UV stays in the last-level cache between calls)": upv}

    # The attention kernel is timed on every n-th step of the timed region.
    # The dispatch start is taken when the dispatch is picked up, which can be
    # while the kernel before it still drains (a few us of it fall inside the
    # interval: the measured rate is a lower bound). The events are created
    # before the warm-up, so that the GPU does not sit idle between the
    # warm-up and the timed steps while the host makes them (an idle gap of
    # tens of ms was followed by slower steps: the chip's clock management).
    every = max(1, args.event_every)
    attn_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(0, args.steps, every)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    for a, b_ in attn_ev + [(t_start, t_end)]:  # create the events (lazily created on first record)
        a.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, attn_ev[i // every] if i % every == 0 else None)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = [a.elapsed_time(b_) for a, b_ in attn_ev]
    attn_avg = float(np.mean(attn_ms))

    if args.copy_calibration:
        copy_calibration(torch, dev)

    tokens = B * H * S
    value = tokens / (ms_step / 1e3)
    alg_bytes = B * S * W * ESIZE + B * H * W * ESIZE + B * H * D_C * ESIZE   # cache + queries + latent output
    alg_flop = B * S * H * (2 * W + 2 * D_C)                   # QK (576) + PV (512) per head-position
    achieved = alg_bytes / (attn_avg / 1e3) / 1e9
    import bench_workloads as BW
    traffic = BW.traffic_from_profile(TRAFFIC_FILE, ATTN_SRC)
    line = {
        "metric": "latent tokens attended/sec (B*H*seq), H=128 decode",
        "value": round(value, 1),
        "unit": "latent tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; RMS-normed latent, roped k_pe/q_pe, q_abs ~ N(0,1/512), W_UV ~ N(0,1/512))",
        "config": {"workload": "DeepSeek-V2-shaped absorbed decode + W_UV up-projection",
                   "batch": B, "heads": H, "seq_len": S, "d_c": D_C, "d_r": D_R, "d_v": D_V,
                   "cache": "dense", "workers": G_workers, "rotated_copies": args.copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "latent attention (mla::mf::attn_mfma_kernel<4, true, true>)",
                     "avg_launch_ms": round(attn_avg, 5), "median_launch_ms": round(float(np.median(attn_ms)), 5),
                     "min_launch_ms": round(float(np.min(attn_ms)), 5), "alg_bytes_per_launch": alg_bytes,
                     "timed_launches": len(attn_ev)},
        "roofline_mfma": {"achieved": round(alg_flop / (attn_avg / 1e3) / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(alg_flop / (attn_avg / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                          "alg_flop_per_launch": alg_flop},
        "wall_s_timed": round(wall, 3),
        "entry_points_ms": entry,
    }
    if not args.headline_only:
        line["hbm_reference"] = hbm_reference(torch, dev)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    if not args.headline_only:
        del sets, q0, cache0, ws, ws_two
        torch.cuda.empty_cache()
        import bench_workloads as BW
        line["workloads"] = BW.run_all(M, G, torch, dev, args, time_entry)
    print(json.dumps(line), flush=True)


def hbm_reference(torch, dev):
    """What plain library kernels reach on this part, as context for the HBM
    fractions (which are against the published 8 TB/s): a 1 GiB bf16 sum
    (reads only) and a 1 GiB device copy (reads + writes), medians of 10."""
    x = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    res = {}
    for name, fn, nbytes in (("sum_read", lambda: x.sum(dtype=torch.float32), 1 << 30),
                             ("copy_read_write", lambda: y.copy_(x), 2 << 30)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        res[name] = {"GB/s": round(nbytes / (ms / 1e3) / 1e9, 1), "ms": round(ms, 4), "bytes": nbytes}
    del x, y
    torch.cuda.empty_cache()
    return res


def copy_calibration(torch, dev):
    """Three plain 1 GiB device copies: their HBM counter readings scale the
    attention kernel's."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def time_entry(torch, stream, call, per_block=20, blocks=5):
    """Median and min over `blocks` of the mean time of `per_block` back-to-back
    calls (ms per call)."""
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    res = []
    for _ in range(blocks):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(per_block):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / per_block)
    return {"median": round(float(np.median(res)), 5), "min": round(float(np.min(res)), 5),
            "calls": per_block * blocks}


if __name__ == "__main__":
    main()
