"""The benchmark's other workloads (everything but the headline decode step).

Each function times one workload on the device and returns a dict with its
throughput, the time of each entry point (median and min over blocks of
back-to-back calls) and a roofline object for its dominant kernel or chain:
algorithmic bytes or FLOP (what the method must move or compute) over the
measured time, against MI355X's HBM (8 TB/s) or dense bf16 MFMA (2.5 PFLOP/s)
peak. Values of the large inputs are drawn on the device with the workloads'
distributions (the lengths and page tables come from the seeded host
generator); timing does not depend on the exact values.
"""
from __future__ import annotations

import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


PROFILE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
ATTN_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "head_latent_attention_09_amd", "csrc",
                        "mla_attn.hip")
RAGGED_TRAFFIC_FILE = os.path.join(PROFILE_DIR, "latent_attention_ragged_paged_b128_h128_traffic.json")


def src_hash(path):
    """SHA-256 prefix of a kernel source with its // comments and blank lines
    removed, so that counter results survive edits of the comments only."""
    import re
    with open(path) as f:
        lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in f]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profile(path, src=ATTN_SRC):
    """Measured HBM bytes per launch from a committed counter summary, valid
    only for the kernel source it was taken on (else None)."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != src_hash(src):
        return None
    return t.get("bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def roof(bound, amount, seconds):
    """bound 'hbm': amount in bytes; 'mfma': amount in FLOP."""
    if bound == "hbm":
        a = amount / seconds / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4)}
    a = amount / seconds / 1e12
    return {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(a / BF16_PEAK_TFLOPS, 4)}


def _latent_rows(torch, dev, n, d_c, d_r, gen):
    """n cache rows [RMS-normed N(0,1) | N(0,1)] in bf16 (a rotation keeps iid N(0,1) rows N(0,1))."""
    z = torch.randn((n, d_c + d_r), device=dev, generator=gen, dtype=torch.float32)
    z[:, :d_c] *= torch.rsqrt(torch.mean(z[:, :d_c] ** 2, dim=1, keepdim=True) + 1e-6)
    return z.to(torch.bfloat16)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_graph(torch, call, per_block=20, blocks=5):
    """Median and min (ms per call) of `per_block` calls captured in one HIP
    graph and replayed `blocks` times: for entries whose GPU time is shorter
    than the Python wrapper's own time per call, so that the figure is the
    device's. The calls launch kernels only (no memory set or copy nodes)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_block):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    res = []
    for _ in range(blocks):
        e0, e1 = _events(torch)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / per_block)
    del g
    return {"median": round(float(np.median(res)), 5), "min": round(float(np.min(res)), 5),
            "calls": per_block * blocks, "timing": "graph replay"}


def _cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    return min(threads, len(os.sched_getaffinity(0)))


# ----------------------------------------------------------------------------
# ragged paged decode: B=128, H=128, lengths U[1, 32768], 64-position pages
# ----------------------------------------------------------------------------
def bench_ragged_paged(M, G, torch, dev, args, time_entry):
    B, H, d_c, d_r, page = 128, 128, 512, 64, 64
    lens = G.config4_lengths(0)
    table, P = G.paged_layout(lens, page, seed=0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    pool = torch.empty((P, page, d_c + d_r), dtype=torch.bfloat16, device=dev)
    flat = pool.view(P * page, d_c + d_r)
    for r0 in range(0, P * page, 1 << 20):
        n = min(1 << 20, P * page - r0)
        flat[r0:r0 + n] = _latent_rows(torch, dev, n, d_c, d_r, gen)
    q = torch.randn((B, H, d_c + d_r), device=dev, generator=gen)
    q[:, :, :d_c] /= math.sqrt(d_c)
    q = q.to(torch.bfloat16)
    lens_d = torch.from_numpy(lens).to(dev)
    table_d = torch.from_numpy(table).to(dev)
    out = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(M.decode_workspace_bytes(B, H, d_c), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(192.0)

    def call(i, ev=None):
        M.latent_decode(q, pool, lens_d, d_c, scale, block_table=table_d, out=out, lse=lse, workspace=ws,
                        timing_events=ev)

    for i in range(5):
        call(i)
    torch.cuda.synchronize()
    entry = time_entry(torch, torch.cuda.current_stream(), call, per_block=10, blocks=5)
    # the attention kernel alone: events around every 4th of 80 back-to-back
    # calls, so that the figure spans the chip's clock swings over ~60 ms
    evs = [_events(torch) for _ in range(20)]
    for i in range(80):
        call(i, evs[i // 4] if i % 4 == 0 else None)
    torch.cuda.synchronize()
    attn = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    tokens = int(lens.sum())
    alg_bytes = tokens * (d_c + d_r) * 2 + B * H * (d_c + d_r) * 2 + B * H * d_c * 2
    res = {"workload": "ragged paged decode B=128 H=128 d_c=512 d_r=64, lengths U[1,32768] (seed 0), "
                       "64-position pages in a shuffled pool",
           "metric": "latent tokens attended/sec (sum of H*len)",
           "value": round(H * tokens / (entry["median"] / 1e3), 1), "unit": "latent tokens/s",
           "tokens": tokens, "pages": int(P), "ms_per_call": entry["median"],
           "entry_points_ms": {"latent_decode (attention + combine)": entry},
           "roofline": dict(roof("hbm", alg_bytes, attn / 1e3),
                            kernel="latent attention (mla::mf::attn_mfma_kernel<4, true, true>)",
                            avg_launch_ms=round(attn, 5), alg_bytes_per_launch=alg_bytes,
                            traffic=traffic_from_profile(RAGGED_TRAFFIC_FILE)),
           "roofline_mfma": roof("mfma", tokens * H * (2 * 576 + 2 * 512), attn / 1e3)}
    if not args.no_cpu_baseline:
        # the oracle on whole sequences drawn with the first lengths of the workload
        import oracle as O
        budget, el, done, nseq = 6.0, 0.0, 0, 0
        while el < budget and nseq < 16:
            n = int(lens[nseq])
            c = G.decode_case(1, H, d_c, d_r, [n], G.BF16, seed=100 + nseq, poison=False)
            qh, lat = G.to_f64(c.q[0], G.BF16), G.to_f64(c.cache[0], G.BF16)
            t1 = time.perf_counter()
            O.latent_attention(qh, lat, d_c, scale, n)
            el += time.perf_counter() - t1
            done += H * n
            nseq += 1
        res["cpu_baseline"] = {"value": done / el, "unit": "latent tokens/s", "cores": _cpu_cores(), "kind": "oracle",
                               "sample": f"{nseq} sequences of the workload's first lengths "
                                         f"({int(lens[:nseq].sum())} positions), fp64 latent definition, {el:.1f} s"}
    return res


# ----------------------------------------------------------------------------
# causal prefill B=2 S=4096 H=128, absorbed chain and expanded form
# ----------------------------------------------------------------------------
def bench_prefill(M, G, torch, dev, args, time_entry):
    c = G.config5_prefill_bf16(0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    Bp, Sp, Hp = c.B, c.S_q, c.H
    qn4, qp4 = to_dev(c.q_nope), to_dev(c.q_pe)
    qn, qp = qn4.reshape(Bp * Sp, Hp, -1), qp4.reshape(Bp * Sp, Hp, -1)
    wuk, wuv, cache = to_dev(c.w_uk), to_dev(c.w_uv), to_dev(c.cache)
    q = torch.empty((Bp * Sp, Hp, c.W), dtype=torch.bfloat16, device=dev)
    out = torch.empty((Bp, Sp, Hp, c.d_c), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((Bp, Sp, Hp), dtype=torch.float32, device=dev)
    v = torch.empty((Bp * Sp, Hp, c.d_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.prefill_workspace_bytes(Bp, Sp, Hp, c.d_c, 0), dtype=torch.uint8, device=dev)
    vu = torch.empty((Bp, Sp, Hp, c.d_v), dtype=torch.bfloat16, device=dev)
    wsu = torch.empty(M.prefill_unabsorbed_workspace_bytes(Bp, Sp, Hp), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def attn(i, e=None):
        M.latent_prefill_causal(q.view(Bp, Sp, Hp, -1), cache, c.d_c, c.kq_scale, out=out, lse=lse, workspace=ws,
                                timing_events=e)

    def unabs(i):
        M.prefill_unabsorbed(qn4, qp4, cache, wuk, wuv, c.kq_scale, out=vu, lse=lse, workspace=wsu)

    M.absorb_q(qn, qp, wuk, out=q)
    for _ in range(2):
        attn(0)
        unabs(0)
    torch.cuda.synchronize()
    entry = {
        "absorb_q": time_entry(torch, stream, lambda i: M.absorb_q(qn, qp, wuk, out=q), per_block=5, blocks=3),
        "latent_prefill_causal": time_entry(torch, stream, attn, per_block=3, blocks=3),
        "up_v": time_entry(torch, stream, lambda i: M.up_v(out.view(Bp * Sp, Hp, -1), wuv, out=v), per_block=5,
                           blocks=3),
        "prefill_unabsorbed (K/V expansion + per-head attention)": time_entry(torch, stream, unabs, per_block=3,
                                                                              blocks=3),
    }
    evs = [_events(torch) for _ in range(5)]
    for e in evs:
        attn(0, e)
    torch.cuda.synchronize()
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    pairs = Bp * Hp * Sp * (Sp + 1) // 2
    flop_abs = pairs * (2 * c.W + 2 * c.d_c)
    absorbed_ms = entry["absorb_q"]["median"] + entry["latent_prefill_causal"]["median"] + entry["up_v"]["median"]
    unabs_ms = entry["prefill_unabsorbed (K/V expansion + per-head attention)"]["median"]
    dk, dv = c.d_nope + c.d_r, c.d_v
    flop_expand = 2 * Bp * Sp * Hp * (c.d_nope + c.d_v) * c.d_c
    flop_unabs = flop_expand + pairs * (2 * dk + 2 * dv)
    return {"workload": "causal prefill B=2 S=4096 H=128 d_nope=128 d_c=512 d_r=64 d_v=128",
            "metric": "latent tokens attended/sec (B*H*S(S+1)/2)",
            "value": round(pairs / (min(absorbed_ms, unabs_ms) / 1e3), 1), "unit": "latent tokens/s",
            "absorbed_chain": {"ms": round(absorbed_ms, 4), "tokens_per_s": round(pairs / (absorbed_ms / 1e3), 1),
                               "attention": dict(roof("mfma", flop_abs, attn_ms / 1e3), avg_launch_ms=round(attn_ms, 4),
                                                 flop_per_launch=flop_abs, flop_per_pair=2 * c.W + 2 * c.d_c)},
            "expanded_form": {"ms": round(unabs_ms, 4), "tokens_per_s": round(pairs / (unabs_ms / 1e3), 1),
                              "roofline": dict(roof("mfma", flop_unabs, unabs_ms / 1e3), flop_per_call=flop_unabs,
                                               flop_per_pair=2 * dk + 2 * dv, flop_expansion=flop_expand)},
            "entry_points_ms": entry}


# ----------------------------------------------------------------------------
# fused cache append: decode (64 tokens) and a prefill chunk (8192 tokens)
# ----------------------------------------------------------------------------
def bench_append(M, G, torch, dev, args, time_entry):
    d_model, d_c, d_r, page = 5120, 512, 64, 64
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    w_c = (torch.randn((d_c, d_model), device=dev, generator=gen) / math.sqrt(d_model)).to(torch.bfloat16)
    w_kr = (torch.randn((d_r, d_model), device=dev, generator=gen) / math.sqrt(d_model)).to(torch.bfloat16)
    res = {"workload": "fused cache append d_model=5120 -> [RMSNorm(W_c x) (512) | RoPE(W_kr x) (64)] into a "
                       "paged cache (64-position pages)"}
    stream = torch.cuda.current_stream()
    for name, N, seqs in (("decode_64_tokens", 64, 64), ("prefill_8192_tokens", 8192, 2)):
        x = torch.randn((N, d_model), device=dev, generator=gen).to(torch.bfloat16)
        per = N // seqs
        seq = torch.arange(N, device=dev, dtype=torch.int32) // per
        pos = (torch.arange(N, device=dev, dtype=torch.int32) % per) + (4095 if N == 64 else 0)
        npg = (4096 + per + page - 1) // page
        table = torch.arange(seqs * npg, device=dev, dtype=torch.int32).reshape(seqs, npg)
        pool = torch.zeros((seqs * npg, page, d_c + d_r), dtype=torch.bfloat16, device=dev)
        wsa = torch.empty(M.lib.mla_cache_append_workspace(N, d_model, d_c, d_r, M.MLA_BF16) + 256,
                          dtype=torch.uint8, device=dev)
        call = lambda i: M.cache_append(x, w_c, w_kr, seq, pos, pool, block_table=table, workspace=wsa)
        call(0)
        torch.cuda.synchronize()
        e = time_graph(torch, call, per_block=20, blocks=5)
        t = e["median"] / 1e3
        flop = 2 * N * d_model * (d_c + d_r)
        nbytes = (N * d_model + (d_c + d_r) * d_model + N * (d_c + d_r)) * 2
        # the binding roofline of the two
        r_h, r_m = roof("hbm", nbytes, t), roof("mfma", flop, t)
        res[name] = {"tokens": N, "ms_per_call": e["median"], "entry_ms": e,
                     "roofline": dict(r_h if nbytes / 8e12 >= flop / 2.5e15 else r_m, alg_bytes=nbytes, alg_flop=flop),
                     "tokens_per_s": round(N / t, 1)}
        del x, pool
    return res


# ----------------------------------------------------------------------------
# full absorption: decode B=64 through absorbed query and output weights
# ----------------------------------------------------------------------------
def bench_full_absorption(M, G, torch, dev, args, time_entry):
    B, H, S, d_cq, d_c, d_r, d_nope, d_v, d_model = 64, 128, 4096, 1536, 512, 64, 128, 128, 5120
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    bf = torch.bfloat16
    rn = lambda shape, sc: (torch.randn(shape, device=dev, generator=gen) * sc).to(bf)
    a_qk = rn((H, d_c, d_cq), 1 / math.sqrt(d_cq))
    a_vo = rn((d_model, H * d_c), 1 / math.sqrt(H * d_c))
    c_q = rn((B, d_cq), 1.0)
    q_pe = rn((B, H, d_r), 1.0)
    caches = []
    for _ in range(2):
        cache = torch.empty((B, S, d_c + d_r), dtype=bf, device=dev)
        for b in range(B):
            cache[b] = _latent_rows(torch, dev, S, d_c, d_r, gen)
        caches.append(cache)
    lens = torch.full((B,), S, dtype=torch.int32, device=dev)
    q = torch.empty((B, H, d_c + d_r), dtype=bf, device=dev)
    lat = torch.empty((B, H, d_c), dtype=bf, device=dev)
    out = torch.empty((B, d_model), dtype=bf, device=dev)
    ws = torch.empty(M.decode_workspace_bytes(B, H, d_c), dtype=torch.uint8, device=dev)
    wso = torch.empty(M.lib.mla_out_absorbed_workspace(B, H, d_c, d_model, M.MLA_BF16) + 256, dtype=torch.uint8,
                      device=dev)
    scale = 1.0 / math.sqrt(d_nope + d_r)
    stream = torch.cuda.current_stream()
    e_q = time_graph(torch, lambda i: M.absorb_q_full(c_q, q_pe, a_qk, out=q), per_block=20, blocks=5)
    e_a = time_entry(torch, stream, lambda i: M.latent_decode(q, caches[i % 2], lens, d_c, scale, out=lat,
                                                              workspace=ws), per_block=10, blocks=5)
    e_o = time_entry(torch, stream, lambda i: M.out_absorbed(lat, a_vo, out=out, workspace=wso), per_block=10,
                     blocks=5)
    total = e_q["median"] + e_a["median"] + e_o["median"]
    b_q = (H * d_c * d_cq + B * d_cq + B * H * (d_c + d_r)) * 2
    b_o = (d_model * H * d_c + B * H * d_c + B * d_model) * 2
    return {"workload": "fully absorbed decode B=64 H=128 S=4096: q_abs = a_qk c' (d_cq=1536), latent decode, "
                        "out = a_vo concat_h(out_lat) (d_model=5120)",
            "ms_per_step": round(total, 4), "tokens_per_s": round(B * H * S / (total / 1e3), 1),
            "entry_points_ms": {"absorb_q_full": e_q, "latent_decode": e_a, "out_absorbed": e_o},
            "absorb_q_full_roofline": dict(roof("hbm", b_q, e_q["median"] / 1e3), alg_bytes=b_q),
            "out_absorbed_roofline": dict(roof("hbm", b_o, e_o["median"] / 1e3), alg_bytes=b_o)}


# ----------------------------------------------------------------------------
# gated MLA layer
# ----------------------------------------------------------------------------
def bench_gated(M, G, torch, dev, args, time_entry):
    B, S, D, L, H = 2, 4096, 2048, 512, 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    bf = torch.bfloat16
    rn = lambda shape, sc: (torch.randn(shape, device=dev, generator=gen) * sc).to(bf)
    x = rn((B, S, D), 1.0)
    w = [rn((D, D), D ** -0.5), rn((L, D), D ** -0.5), rn((D, L), L ** -0.5), rn((D, L), L ** -0.5),
         rn((D, D), D ** -0.5), rn((D, D), D ** -0.5)]
    out = torch.empty((B, S, D), dtype=bf, device=dev)
    lc = torch.empty((B, S, L), dtype=bf, device=dev)
    ws = torch.empty(M.lib.mla_gated_mla_workspace(B, S, D, L, H, M.MLA_BF16, M.default_workers()) + 256,
                     dtype=torch.uint8, device=dev)
    call = lambda i: M.gated_mla(x, *w, H, True, out=out, latent_cache=lc, workspace=ws)
    call(0)
    torch.cuda.synchronize()
    e = time_entry(torch, torch.cuda.current_stream(), call, per_block=5, blocks=3)
    n = B * S
    Dh = D // H
    pairs = B * H * S * (S + 1) // 2
    flop = 2 * n * D * D * 3 + 2 * n * D * L + 2 * 2 * n * L * D + pairs * (2 * Dh + 2 * Dh)
    return {"workload": f"gated MLA layer B={B} S={S} D={D} H={H} (D_h={Dh}) L={L}, causal",
            "ms_per_call": e["median"], "entry_ms": e, "tokens_per_s": round(n / (e["median"] / 1e3), 1),
            "roofline": dict(roof("mfma", flop, e["median"] / 1e3), alg_flop=flop)}


# ----------------------------------------------------------------------------
# softmax reference overflow: the decode step with and without a logit spike
# ----------------------------------------------------------------------------
def bench_overflow_redo(M, G, torch, dev, args, time_entry):
    """The long-context decode step (B=64, H=128, S=4096, one call: attention
    plus the merge fused with W_UV), first on N(0,1) inputs, then with one
    row's scores rising by about 70 nats at position 2500 (a segment past its
    first tile: its fixed reference overflows and the segment is redone with
    its exact maxima)."""
    B, H, S, d_c, d_r, d_v = 64, 128, 4096, 512, 64, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    bf = torch.bfloat16
    cache = torch.empty((B, S, d_c + d_r), dtype=bf, device=dev)
    for b in range(B):
        cache[b] = _latent_rows(torch, dev, S, d_c, d_r, gen)
    q = torch.randn((B, H, d_c + d_r), device=dev, generator=gen)
    q[:, :, :d_c] /= math.sqrt(d_c)
    q = q.to(bf)
    wuv = (torch.randn((H, d_v, d_c), device=dev, generator=gen) / math.sqrt(d_c)).to(bf)
    lens = torch.full((B,), S, dtype=torch.int32, device=dev)
    v = torch.empty((B, H, d_v), dtype=bf, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(M.decode_up_v_workspace_bytes(B, H, d_c, M.default_workers()), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d_c // 4 + d_r)
    stream = torch.cuda.current_stream()

    def call(i):
        M.latent_decode_up_v(q, cache, lens, d_c, scale, wuv, out=v, lse=lse, workspace=ws)

    normal = time_entry(torch, stream, call, per_block=10, blocks=5)
    q[7, :, d_c] = 40.0
    cache[7, 2500, d_c] = 24.0  # 40 * 24 / sqrt(192) ~ 69 nats above the row's other scores
    torch.cuda.synchronize()
    spiked = time_entry(torch, stream, call, per_block=10, blocks=5)
    return {"workload": "decode B=64 H=128 S=4096 (fused up-projection), normal vs one row with a ~69-nat "
                        "logit spike at position 2500",
            "normal_ms": normal, "spiked_ms": spiked,
            "ratio": round(spiked["median"] / normal["median"], 3)}


WORKLOADS = [("ragged_paged_decode", bench_ragged_paged), ("causal_prefill", bench_prefill),
             ("cache_append", bench_append), ("full_absorption", bench_full_absorption),
             ("gated_mla", bench_gated), ("overflow_redo", bench_overflow_redo)]


def run_all(M, G, torch, dev, args, time_entry):
    only = [s for s in args.only.split(",") if s]
    res = {}
    for name, fn in WORKLOADS:
        if only and name not in only:
            continue
        t0 = time.perf_counter()
        log(f"{name} ...")
        res[name] = fn(M, G, torch, dev, args, time_entry)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        log(f"{name} done in {time.perf_counter() - t0:.1f} s")
    return res
