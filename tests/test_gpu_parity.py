"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Same seeded inputs on both sides; small cases are compared element by element,
full-size workloads on sampled outputs the oracle computes one by one.
Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32) or 2e-2 (bf16 inputs,
fp32 accumulation); lse within the same bound in absolute terms.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as G
from gpu_util import LSE_TOL, TOL, dtype_torch, elem_rel_err, lse_err, rel_err, to_dev, to_host64

pytestmark = pytest.mark.gpu

M = None


def setup_module(module):
    global M
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import head_latent_attention_09_amd as lib_mod
    M = lib_mod


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def run_decode(case, num_workers=0):
    q = to_dev(case.q, case.dtype)
    lens = torch.from_numpy(case.lens.astype(np.int32)).cuda()
    if case.page_size is None:
        cache = to_dev(case.cache, case.dtype)
        out, lse = M.latent_decode(q, cache, lens, case.d_c, case.kq_scale, num_workers=num_workers)
    else:
        cache = to_dev(case.pages, case.dtype)
        table = torch.from_numpy(case.block_table).cuda()
        out, lse = M.latent_decode(q, cache, lens, case.d_c, case.kq_scale, block_table=table,
                                   num_workers=num_workers)
    torch.cuda.synchronize()
    return to_host64(out), lse.cpu().numpy().astype(np.float64)


def oracle_decode(case, rows=None, heads=None):
    rows = range(case.B) if rows is None else rows
    outs, lses = [], []
    for b in rows:
        lat = G.to_f64(G.seq_rows(case, b), case.dtype)
        q = G.to_f64(case.q[b], case.dtype)
        o, l = O.latent_attention(q, lat, case.d_c, case.kq_scale, int(case.lens[b]), heads)
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)


def check_decode(case, num_workers=0, label=""):
    say(f"decode {label}: dtype={case.dtype} B={case.B} H={case.H} d_c={case.d_c} d_r={case.d_r} "
        f"lens={list(case.lens)[:8]} paged={case.page_size} workers={num_workers}")
    got, glse = run_decode(case, num_workers)
    ref, rlse = oracle_decode(case)
    e, le = rel_err(got, ref), lse_err(glse, rlse)
    say(f"  out rel err {e:.3e}  lse abs err {le:.3e}")
    assert e <= TOL[case.dtype] and le <= LSE_TOL[case.dtype]
    return got, glse


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
@pytest.mark.parametrize("H", [128, 96, 64, 32, 16])
def test_decode_dense_small(dtype, H):
    lens = [1, 45, 100, 0, 257]
    case = G.decode_case(5, H, 512, 64, lens, dtype, seed=100 + H, cache_rows=300)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, label="dense small")


@pytest.mark.parametrize("workers", [1, 3, 7, 64, 0])
def test_decode_split_count_invariance(workers):
    case = G.decode_case(3, 128, 512, 64, [700, 33, 1000], G.BF16, seed=7)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, num_workers=workers, label="split invariance")


@pytest.mark.parametrize("H,page_size,workers", [(128, None, 1), (128, None, 5), (128, 16, 9), (64, None, 13),
                                                  (128, 16, 23)])
def test_decode_short_segments(H, page_size, workers):
    """Segments of 1 to 6 tiles, shorter than, equal to and just past the
    tile pipeline's depth, where the last steps load and score stand-in tiles
    past the segment's end (rows past each length, and unused page slots,
    hold NaN, so a read of them would show)."""
    lens = [16, 32, 48, 64, 80, 96, 15, 47]
    case = G.decode_case(len(lens), H, 512, 64, lens, G.BF16, seed=90 + workers, page_size=page_size)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, num_workers=workers, label="short segments")


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
def test_decode_timing_events(dtype):
    """Timing events passed with the attention launch: the results equal those
    of a launch without them, and the events take a positive interval."""
    case = G.decode_case(3, 128, 512, 64, [700, 33, 1000], dtype, seed=8)
    case.kq_scale = 1.0 / math.sqrt(192)
    say(f"decode timing events: dtype={dtype}")
    q = to_dev(case.q, dtype)
    cache = to_dev(case.cache, dtype)
    lens = torch.from_numpy(case.lens.astype(np.int32)).cuda()
    out0, lse0 = M.latent_decode(q, cache, lens, case.d_c, case.kq_scale)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    out1, lse1 = M.latent_decode(q, cache, lens, case.d_c, case.kq_scale, timing_events=ev)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    assert ev[0].elapsed_time(ev[1]) > 0


def run_decode_up_v(case, num_workers=0):
    q = to_dev(case.q, case.dtype)
    lens = torch.from_numpy(case.lens.astype(np.int32)).cuda()
    w = to_dev(case.w_uv, case.dtype)
    if case.page_size is None:
        v, lse = M.latent_decode_up_v(q, to_dev(case.cache, case.dtype), lens, case.d_c, case.kq_scale, w,
                                      num_workers=num_workers)
    else:
        v, lse = M.latent_decode_up_v(q, to_dev(case.pages, case.dtype), lens, case.d_c, case.kq_scale, w,
                                      block_table=torch.from_numpy(case.block_table).cuda(), num_workers=num_workers)
    torch.cuda.synchronize()
    return to_host64(v), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype,H,d_v,lens,paged,workers", [
    (G.BF16, 128, 128, [700, 33, 1000], False, 7),      # merge fused with the up-projection, cut rows
    (G.BF16, 128, 128, [1, 0, 300, 65, 0], False, 0),   # empty and one-position rows
    (G.BF16, 64, 128, [130, 500, 64], True, 5),         # paged, 64 heads
    (G.BF16, 128, 64, [200, 40], False, 3),             # d_v outside the fused kernel: decode, combine, up_v
    (G.F32, 16, 24, [50, 7, 0], False, 4),              # fp32: the generic kernels
])
def test_decode_up_v(dtype, H, d_v, lens, paged, workers):
    case = G.decode_case(len(lens), H, 512, 64, lens, dtype, seed=120 + H + d_v, d_v=d_v,
                         page_size=64 if paged else None)
    case.kq_scale = 1.0 / math.sqrt(192)
    say(f"decode + up_v: dtype={dtype} H={H} d_v={d_v} lens={lens} paged={paged} workers={workers}")
    got, glse = run_decode_up_v(case, workers)
    lat, rlse = oracle_decode(case)
    ref = O.up_project(lat, G.to_f64(case.w_uv, dtype))
    e, le = rel_err(got, ref), lse_err(glse, rlse)
    say(f"  v rel err {e:.3e}  lse abs err {le:.3e}")
    assert e <= TOL[dtype] and le <= LSE_TOL[dtype]
    # the same as the two calls it replaces, up to the rounding of the merge
    lat_gpu, _ = run_decode(case, workers)
    two = O.up_project(lat_gpu, G.to_f64(case.w_uv, dtype))
    assert rel_err(got, two) <= TOL[dtype]


def test_decode_up_v_events_and_no_lse():
    """The combined call with timing events and without an lse output gives
    the same v as the plain call, bit for bit (the same kernels run; only the
    lse stores are skipped), and the events take a positive interval."""
    case = G.decode_case(3, 128, 512, 64, [700, 0, 1000], G.BF16, seed=9, d_v=128)
    case.kq_scale = 1.0 / math.sqrt(192)
    q, cache, w = to_dev(case.q, G.BF16), to_dev(case.cache, G.BF16), to_dev(case.w_uv, G.BF16)
    lens = torch.from_numpy(case.lens.astype(np.int32)).cuda()
    v0, lse0 = M.latent_decode_up_v(q, cache, lens, 512, case.kq_scale, w, num_workers=6)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    v1, lse1 = M.latent_decode_up_v(q, cache, lens, 512, case.kq_scale, w, num_workers=6, want_lse=False,
                                    timing_events=ev)
    torch.cuda.synchronize()
    assert lse1 is None and torch.equal(v0, v1)
    assert ev[0].elapsed_time(ev[1]) > 0
    assert torch.all(v0[1] == 0) and torch.all(torch.isneginf(lse0[1]))  # the empty row


@pytest.mark.parametrize("workers", [4, 1])
def test_decode_up_v_large_logits(workers):
    """Segments redone after a softmax reference overflow, under the fused merge."""
    case = G.decode_case(2, 128, 512, 64, [600, 300], G.BF16, seed=13, d_v=128)
    case.kq_scale = 1.0 / math.sqrt(192)
    cache = G.to_f64(case.cache, G.BF16)
    cache[:, :, 512] = np.linspace(0.0, 60.0, cache.shape[1])[None, :]
    case.cache = G.storage(cache, G.BF16)
    q = G.to_f64(case.q, G.BF16)
    q[:, :, 512] = 40.0
    case.q = G.storage(q, G.BF16)
    got, glse = run_decode_up_v(case, workers)
    lat, rlse = oracle_decode(case)
    ref = O.up_project(lat, G.to_f64(case.w_uv, G.BF16))
    assert rel_err(got, ref) <= TOL[G.BF16] and lse_err(glse, rlse) <= LSE_TOL[G.BF16]


@pytest.mark.parametrize("rows,workers", [(300, 0), (1, 200)])
def test_decode_up_v_plan_kernel_and_many_parts(rows, workers):
    """The fused merge after the planning kernel (more than 256 rows), and a
    row cut into about 190 parts."""
    if rows == 1:
        case = G.decode_case(1, 128, 512, 64, [3000], G.BF16, seed=42, d_v=128)
    else:
        lens = np.random.default_rng(6).integers(0, 41, rows)
        case = G.decode_case(rows, 32, 512, 64, lens, G.BF16, seed=56, d_v=128)
    case.kq_scale = 1.0 / math.sqrt(192)
    say(f"decode + up_v: rows={rows} workers={workers}")
    got, glse = run_decode_up_v(case, workers)
    lat, rlse = oracle_decode(case)
    ref = O.up_project(lat, G.to_f64(case.w_uv, G.BF16))
    assert rel_err(got, ref) <= TOL[G.BF16] and lse_err(glse, rlse) <= LSE_TOL[G.BF16]


def test_decode_batch_planned_by_kernel():
    """More rows than the attention kernel plans for itself (256): the MFMA
    kernel then reads the planning kernel's results."""
    lens = np.random.default_rng(5).integers(0, 41, 300)
    case = G.decode_case(300, 32, 512, 64, lens, G.BF16, seed=55)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, label="300 rows")


@pytest.mark.parametrize("workers", [200, 0])
def test_decode_row_over_many_workers(workers):
    """One long row cut into one or two tiles per worker: the combine merges
    about 190 partial results per row (its multi-pass path)."""
    case = G.decode_case(1, 128, 512, 64, [3000], G.BF16, seed=41)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, num_workers=workers, label="many parts")


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
def test_decode_paged_small(dtype):
    lens = [64, 1, 130, 0, 200, 65]
    case = G.decode_case(6, 128, 512, 64, lens, dtype, seed=31, page_size=64)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, num_workers=16, label="paged small")


@pytest.mark.parametrize("page_size", [1, 24, 16])
def test_decode_paged_page_sizes(page_size):
    """Pages smaller than a tile or not a multiple of it (generic kernel), and
    the smallest page the MFMA kernel takes (16 positions)."""
    lens = [40, 0, 17, 1, 33]
    case = G.decode_case(5, 128, 512, 64, lens, G.BF16, seed=60 + page_size, page_size=page_size)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, num_workers=7, label=f"page size {page_size}")


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
def test_decode_largest_dims_generic(dtype):
    """d_c = 1024 and d_c + d_r = 1152, the largest the generic kernel takes."""
    case = G.decode_case(2, 3, 1024, 128, [70, 9], dtype, seed=71)
    case.kq_scale = 1.0 / math.sqrt(1024 + 128)
    check_decode(case, num_workers=4, label="largest dims")


@pytest.mark.parametrize("H", [160, 40])
def test_decode_heads_outside_mfma(H):
    """bf16 with d_c=512, d_r=64 but a head count the MFMA kernel does not take."""
    case = G.decode_case(2, H, 512, 64, [100, 31], G.BF16, seed=80 + H)
    case.kq_scale = 1.0 / math.sqrt(192)
    check_decode(case, num_workers=9, label=f"H={H}")


def test_decode_all_rows_empty():
    """Every sequence empty: zeros and lse = -inf, no attention work."""
    case = G.decode_case(4, 128, 512, 64, [0, 0, 0, 0], G.BF16, seed=90, cache_rows=16)
    case.kq_scale = 1.0 / math.sqrt(192)
    got, glse = run_decode(case)
    assert np.all(got == 0) and np.all(np.isneginf(glse))


def test_decode_batch_zero():
    """An empty batch is accepted and launches nothing."""
    q = torch.zeros((0, 128, 576), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((0, 16, 576), dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out, lse = M.latent_decode(q, cache, lens, 512, 0.1)
    torch.cuda.synchronize()
    assert out.shape == (0, 128, 512) and lse.shape == (0, 128)


def test_decode_odd_shapes_generic():
    """d_c, d_r, H outside the MFMA specialisation (generic kernel), bf16 and fp32."""
    for dtype in (G.BF16, G.F32):
        case = G.decode_case(3, 5, 96, 32, [17, 50, 3], dtype, seed=5)
        case.kq_scale = 0.2
        check_decode(case, num_workers=5, label="odd shapes")


def test_decode_single_position_is_latent_row():
    """One visible position: softmax weight 1, output = c_0 exactly (bf16)."""
    case = G.decode_case(4, 128, 512, 64, [1, 1, 1, 1], G.BF16, seed=9)
    case.kq_scale = 1.0 / math.sqrt(192)
    got, glse = run_decode(case)
    for b in range(4):
        c0 = G.to_f64(G.seq_rows(case, b), G.BF16)[0, :512]
        assert np.array_equal(got[b], np.broadcast_to(c0, got[b].shape))


def test_decode_zero_query_is_mean():
    case = G.decode_case(2, 128, 512, 64, [300, 77], G.BF16, seed=12)
    case.q[:] = 0
    case.kq_scale = 1.0 / math.sqrt(192)
    got, glse = run_decode(case)
    for b in range(2):
        lat = G.to_f64(G.seq_rows(case, b), G.BF16)
        mean = lat[:, :512].mean(axis=0)
        assert rel_err(got[b], np.broadcast_to(mean, got[b].shape)) <= 2e-2
        assert np.allclose(glse[b], math.log(case.lens[b]), atol=1e-3)


@pytest.mark.parametrize("workers", [4, 1])
def test_decode_large_logits_fixup(workers):
    """Scores that rise steadily by far more than 2^64 along a sequence
    (segments whose first-tile softmax reference overflows are redone with
    their exact maxima): rows cut over several workers (4) and rows finished
    by one worker (1)."""
    case = G.decode_case(2, 128, 512, 64, [600, 300], G.BF16, seed=13)
    case.kq_scale = 1.0 / math.sqrt(192)
    cache = G.to_f64(case.cache, G.BF16)
    ramp = np.linspace(0.0, 60.0, cache.shape[1])
    cache[:, :, 512] = ramp[None, :]          # one rope coordinate grows along the sequence
    case.cache = G.storage(cache, G.BF16)
    q = G.to_f64(case.q, G.BF16)
    q[:, :, 512] = 40.0
    case.q = G.storage(q, G.BF16)
    check_decode(case, num_workers=workers, label="large logits")


def _spike(case, b, pos, value, coord=512):
    """Set rope coordinate `coord` of cache row (b, pos) to `value` (dense or paged)."""
    if case.page_size is None:
        x = G.to_f64(case.cache[b, pos], case.dtype)
        x[coord] = value
        case.cache[b, pos] = G.storage(x, case.dtype)
    else:
        pg = int(case.block_table[b, pos // case.page_size])
        x = G.to_f64(case.pages[pg, pos % case.page_size], case.dtype)
        x[coord] = value
        case.pages[pg, pos % case.page_size] = G.storage(x, case.dtype)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("workers", [16, 1])
def test_decode_overflow_redo_later_segment(workers, paged):
    """Isolated logit spikes in the middle of long rows, against the oracle on
    every head: row 0 rises by about 60 nats over the rest (sum of weights
    past 2^64 but finite), row 1 by about 150 nats (weights overflow to inf),
    row 2 has its spike in the first tile (no redo), row 3 none. With 16
    workers the rows are cut across workers, so the redone segments are parts
    of split rows; with 1 worker each row is one segment."""
    case = G.decode_case(4, 128, 512, 64, [2000, 1500, 1000, 700], G.BF16, seed=21,
                         page_size=64 if paged else None)
    case.kq_scale = 1.0 / math.sqrt(192)
    q = G.to_f64(case.q, G.BF16)
    q[:, :, 512] = 40.0
    case.q = G.storage(q, G.BF16)
    for b, pos, val in [(0, 1517, 24.0), (0, 1701, 24.0), (1, 1211, 52.0), (2, 5, 24.0)]:
        _spike(case, b, pos, val)
    check_decode(case, num_workers=workers, label="overflow redo")


# ----------------------------------------------------------------------------
# full-size workloads
# ----------------------------------------------------------------------------
def test_config2_full_fp32():
    case = G.config2_decode_f32(0)
    check_decode(case, label="config 2")


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_config3_sampled():
    case = G.config3_decode_bf16(0)
    say("config 3: generating done; running decode + up_v")
    q = to_dev(case.q, G.BF16)
    cache = to_dev(case.cache, G.BF16)
    lens = torch.from_numpy(case.lens).cuda()
    w_uv = to_dev(case.w_uv, G.BF16)
    out_lat, lse = M.latent_decode(q, cache, lens, 512, case.kq_scale)
    v = M.up_v(out_lat, w_uv)
    # the benchmark's call: attention, then the merge fused with the up-projection
    vf, lsef = M.latent_decode_up_v(q, cache, lens, 512, case.kq_scale, w_uv)
    torch.cuda.synchronize()
    out_lat, v, lse = to_host64(out_lat), to_host64(v), lse.cpu().numpy()
    vf, lsef = to_host64(vf), lsef.cpu().numpy()
    say(f"  fused vs two calls: v {rel_err(vf, v):.2e}  lse {np.max(np.abs(lsef - lse)):.2e}")
    assert rel_err(vf, v) <= 1e-2 and np.max(np.abs(lsef - lse)) <= 1e-4
    wuv = G.to_f64(case.w_uv, G.BF16)
    # every head of 8 rows (first, last, both sides of the middle, two drawn)
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, 31, 32, 62, 63} | set(int(r) for r in rng.integers(2, 62, 2)))
    for b in rows:
        lat = G.to_f64(case.cache[b], G.BF16)
        qb = G.to_f64(case.q[b], G.BF16)
        ro, rl = O.latent_attention(qb, lat, 512, case.kq_scale, 4096)
        rv = O.up_project(ro, wuv)   # equals the per-head expanded values (value-side associativity pin)
        e1, e2, e3 = rel_err(out_lat[b], ro), rel_err(v[b], rv), float(np.max(np.abs(lse[b] - rl)))
        e4, e5 = rel_err(vf[b], rv), float(np.max(np.abs(lsef[b] - rl)))
        el = elem_rel_err(out_lat[b], ro)
        say(f"  row {b}, all heads: out_lat {e1:.2e} (elementwise, floored {el:.2e}) v {e2:.2e} lse {e3:.2e} "
            f"fused v {e4:.2e} lse {e5:.2e}")
        assert e1 <= 2e-2 and e2 <= 2e-2 and e3 <= 2e-2 and e4 <= 2e-2 and e5 <= 2e-2
    # and two heads against values expanded per head before the weighted sum
    for b, h in ((0, 0), (63, 127)):
        lat = G.to_f64(case.cache[b], G.BF16)
        rv, _ = O.latent_attention_expanded_v(G.to_f64(case.q[b], G.BF16), lat, 512, wuv, case.kq_scale, 4096, [h])
        e = rel_err(vf[b, h], rv[0])
        say(f"  (b={b}, h={h}) fused v vs expanded values {e:.2e}")
        assert e <= 2e-2


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_config4_sampled():
    case = G.config4_paged_bf16(0)
    say(f"config 4: {int(case.lens.sum())} tokens in {case.pages.shape[0]} pages")
    got, glse = run_decode(case)
    order = np.argsort(case.lens)
    # every head of 16 rows: the shortest and longest, quantiles of the length mix, and fixed picks
    rows = sorted(set([int(order[k]) for k in (0, 1, 32, 64, 96, 126, 127)] + list(range(0, 128, 8))))
    ref, rlse = oracle_decode(case, rows=rows)
    for i, b in enumerate(rows):
        e, le = rel_err(got[b], ref[i]), lse_err(glse[b], rlse[i])
        say(f"  seq {b} len {case.lens[b]}: out {e:.2e} (elementwise, floored {elem_rel_err(got[b], ref[i]):.2e}) "
            f"lse {le:.2e}")
        assert e <= 2e-2 and le <= 2e-2
    assert len(rows) >= 16


# ----------------------------------------------------------------------------
# causal prefill, absorb, up_v
# ----------------------------------------------------------------------------
def run_prefill_chain(case, num_workers=0):
    qn, qp = to_dev(case.q_nope, case.dtype), to_dev(case.q_pe, case.dtype)
    wuk, wuv = to_dev(case.w_uk, case.dtype), to_dev(case.w_uv, case.dtype)
    cache = to_dev(case.cache, case.dtype)
    B, S, H = case.B, case.S_q, case.H
    q = M.absorb_q(qn.reshape(B * S, H, -1), qp.reshape(B * S, H, -1), wuk)
    out_lat, lse = M.latent_prefill_causal(q.reshape(B, S, H, -1), cache, case.d_c, case.kq_scale,
                                           num_workers=num_workers)
    v = M.up_v(out_lat.reshape(B * S, H, -1), wuv)
    torch.cuda.synchronize()
    return (to_host64(q).reshape(B, S, H, -1), to_host64(out_lat), lse.cpu().numpy(),
            to_host64(v).reshape(B, S, H, -1))


@pytest.mark.parametrize("dtype,H,d_c,d_r,d_nope,d_v,S_q,S_kv", [
    (G.BF16, 128, 512, 64, 128, 128, 70, 70),     # MFMA path, several tiles, ragged tail
    (G.BF16, 128, 512, 64, 128, 128, 40, 100),    # chunk at the end of a longer cache
    (G.F32, 8, 64, 16, 32, 24, 33, 33),           # generic path
    (G.BF16, 32, 512, 64, 128, 128, 50, 20),      # more queries than cache rows
])
def test_prefill_chain_small(dtype, H, d_c, d_r, d_nope, d_v, S_q, S_kv):
    say(f"prefill chain: {dtype} H={H} d_c={d_c} S_q={S_q} S_kv={S_kv}")
    case = G.prefill_case(2, S_q, S_kv, H, d_nope, d_c, d_r, d_v, dtype, seed=21)
    gq, gout, glse, gv = run_prefill_chain(case, num_workers=13)
    tol = TOL[dtype]
    for b in range(case.B):
        qn, qp = G.to_f64(case.q_nope[b], dtype), G.to_f64(case.q_pe[b], dtype)
        wuk, wuv = G.to_f64(case.w_uk, dtype), G.to_f64(case.w_uv, dtype)
        rq = O.absorb_query(qn, qp, wuk)
        assert rel_err(gq[b], rq) <= tol
        lat = G.to_f64(case.cache[b], dtype)
        ro, rl = O.latent_prefill_causal(rq, lat, d_c, case.kq_scale)
        e, le = rel_err(gout[b], ro), lse_err(glse[b], rl)
        # end to end against the unabsorbed definition (per-head expanded K and V)
        ev = 0.0
        for i in range(0, S_q, max(1, S_q // 7)):
            n = O.causal_visible(i, S_q, S_kv)
            rv, _ = O.mla_unabsorbed(qn[i], qp[i], lat, d_c, wuk, wuv, case.kq_scale, n)
            ev = max(ev, rel_err(gv[b, i], rv))
        say(f"  b={b}: out {e:.2e} lse {le:.2e} v(unabsorbed) {ev:.2e}")
        assert e <= tol and le <= LSE_TOL[dtype] and ev <= tol


@pytest.mark.parametrize("workers", [1, 4, 64, 0])
def test_prefill_split_count_invariance(workers):
    """Causal prefill with many short rows per worker (the plan charges each
    row a fixed cost) and rows cut across workers, at several worker counts."""
    say(f"prefill split invariance: workers={workers}")
    case = G.prefill_case(2, 160, 160, 32, 128, 512, 64, 128, G.BF16, seed=23)
    rng = np.random.default_rng(23)   # absorbed queries drawn directly: [q_abs ~ N(0, 1/512) | q_pe ~ N(0, 1)]
    qa = np.concatenate([rng.standard_normal((2, 160, 32, 512)) / math.sqrt(512),
                         rng.standard_normal((2, 160, 32, 64))], axis=-1)
    q = to_dev(G.storage(qa, G.BF16), G.BF16)
    cache = to_dev(case.cache, G.BF16)
    out, lse = M.latent_prefill_causal(q, cache, 512, case.kq_scale, num_workers=workers)
    torch.cuda.synchronize()
    got, glse = to_host64(out), lse.cpu().numpy().astype(np.float64)
    qh = to_host64(q)
    for b in range(2):
        ro, rl = O.latent_prefill_causal(qh[b], G.to_f64(case.cache[b], G.BF16), 512, case.kq_scale)
        e, le = rel_err(got[b], ro), lse_err(glse[b], rl)
        say(f"  b={b}: out {e:.2e} lse {le:.2e}")
        assert e <= TOL[G.BF16] and le <= LSE_TOL[G.BF16]


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_config5_sampled():
    case = G.config5_prefill_bf16(0)
    say("config 5 generated; running absorb + prefill + up_v")
    gq, gout, glse, gv = run_prefill_chain(case)
    wuk, wuv = G.to_f64(case.w_uk, G.BF16), G.to_f64(case.w_uv, G.BF16)
    for b in range(2):
        lat = G.to_f64(case.cache[b], G.BF16)
        for i in [0, 1, 31, 32, 1000, 4095]:
            qn, qp = G.to_f64(case.q_nope[b, i], G.BF16), G.to_f64(case.q_pe[b, i], G.BF16)
            rq = O.absorb_query(qn, qp, wuk)
            eq = rel_err(gq[b, i], rq)
            ro, rl = O.latent_attention(rq, lat, 512, case.kq_scale, i + 1)
            e, le = rel_err(gout[b, i], ro), lse_err(glse[b, i], rl)
            hs = [0, 77, 127]
            rv = np.array([O.mla_unabsorbed(qn[[h]], qp[[h]], lat, 512, wuk[[h]], wuv[[h]], case.kq_scale,
                                            i + 1)[0][0] for h in hs])
            ev = rel_err(gv[b, i, hs], rv)
            say(f"  b={b} i={i}: q {eq:.2e} out {e:.2e} lse {le:.2e} v {ev:.2e}")
            assert eq <= 2e-2 and e <= 2e-2 and le <= 2e-2 and ev <= 2e-2


@pytest.mark.parametrize("dtype,N,H,d_in,d_out", [
    (G.BF16, 300, 4, 512, 128), (G.BF16, 64, 128, 512, 128), (G.F32, 5, 3, 20, 20), (G.BF16, 7, 2, 40, 24),
    (G.BF16, 1100, 64, 512, 128),   # 128x128 tiles, 8 K slices, ragged last row block
    (G.BF16, 260, 4, 256, 256)])
def test_up_v(dtype, N, H, d_in, d_out):
    say(f"up_v {dtype} N={N} H={H} {d_in}->{d_out}")
    c = G.gemm_case(N, H, d_in, d_out, dtype, seed=N, transpose_w=True)
    got = to_host64(M.up_v(to_dev(c.x, dtype), to_dev(c.w, dtype)))
    ref = O.up_project(G.to_f64(c.x, dtype), G.to_f64(c.w, dtype))
    assert rel_err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype,N,H,d_nope,d_c,d_r", [
    (G.BF16, 300, 4, 128, 512, 64), (G.BF16, 129, 2, 64, 256, 0), (G.F32, 3, 3, 20, 20, 0), (G.F32, 9, 2, 4, 6, 2),
    (G.BF16, 700, 8, 256, 512, 64),    # 128x128 tiles, 4 K slices (buffers refilled), ragged last row block
    (G.BF16, 700, 8, 128, 512, 64),    # streaming kernel: W_UK resident, row blocks split over workgroups
    (G.BF16, 1000, 3, 64, 128, 16)])   # streaming kernel, one K slice, one column block
def test_absorb(dtype, N, H, d_nope, d_c, d_r):
    say(f"absorb {dtype} N={N} H={H} {d_nope}->{d_c} + {d_r}")
    c = G.gemm_case(N, H, d_nope, d_c, dtype, seed=N + 1, transpose_w=False)
    qp = G.storage(np.random.default_rng(N).standard_normal((N, H, d_r)), dtype)
    got = to_host64(M.absorb_q(to_dev(c.x, dtype), to_dev(qp, dtype) if d_r else None, to_dev(c.w, dtype)))
    ref = O.absorb_query(G.to_f64(c.x, dtype), G.to_f64(qp, dtype), G.to_f64(c.w, dtype))
    assert rel_err(got[..., :d_c], ref[..., :d_c]) <= TOL[dtype]
    assert np.array_equal(got[..., d_c:], ref[..., d_c:])   # q_pe copied bit-exactly


# ----------------------------------------------------------------------------
# the pages' own small workloads end to end
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [G.F32, G.BF16])
def test_ferrox_shape_chain(dtype):
    """The ferrox-core unit-test shape: absorb -> latent decode -> up_v equals the
    unabsorbed attention over per-head expanded K and V."""
    c = G.p2_tiny_case()
    st = lambda a: G.storage(a, dtype)
    scale = 1.0 / math.sqrt(c.d_nope + c.d_r)
    q = M.absorb_q(to_dev(st(c.q_nope[None]), dtype), to_dev(st(c.q_pe[None]), dtype), to_dev(st(c.w_uk), dtype))
    lens = torch.tensor([c.seq], dtype=torch.int32).cuda()
    lat, lse = M.latent_decode(q, to_dev(st(c.latent[None]), dtype), lens, c.d_c, scale)
    v = to_host64(M.up_v(lat, to_dev(st(c.w_uv), dtype)))[0]
    f = lambda a: G.to_f64(st(a), dtype)
    ref, _ = O.mla_unabsorbed(f(c.q_nope), f(c.q_pe), f(c.latent), c.d_c, f(c.w_uk), f(c.w_uv), scale, c.seq)
    e = rel_err(v, ref)
    say(f"ferrox chain {dtype}: rel err {e:.2e}")
    assert e <= TOL[dtype]
    if dtype == G.F32:
        assert np.max(np.abs(v - ref)) < 1e-5   # the page's own absolute bound


def test_config1_notebook_chain():
    d = G.config1_notebook(0)
    scale = 1.0 / math.sqrt(d.d_h)
    H, dh = d.H, d.d_h
    # head s owns columns s*d_h .. (s+1)*d_h - 1 of the up-projections and the
    # same rows of W_O (sliced here, independently of the oracle)
    blk = lambda W: np.stack([W[:, s * dh:(s + 1) * dh] for s in range(H)])   # [H, d_c, d_h]
    uK, uV = blk(d.W_uK), blk(d.W_uV)
    Ow = np.stack([d.W_O[s * dh:(s + 1) * dh] for s in range(H)])            # [H, d_h, d_model]
    cache = np.vstack([d.C_KV, d.X @ d.W_dKV])                 # host-side append of the new latent
    q_nope = np.einsum("i,hij->hj", (d.X @ d.W_dQ)[0], blk(d.W_uQ))          # [H, d_h]
    st = lambda a: G.storage(a, G.F32)
    q = M.absorb_q(to_dev(st(q_nope[None]), G.F32), None, to_dev(st(uK.transpose(0, 2, 1)), G.F32))
    lens = torch.tensor([cache.shape[0]], dtype=torch.int32).cuda()
    lat, _ = M.latent_decode(q, to_dev(st(cache[None]), G.F32), lens, d.d_c, scale)
    v = to_host64(M.up_v(lat, to_dev(st(uV.transpose(0, 2, 1)), G.F32)))[0]
    final = np.einsum("hi,hio->o", v, Ow)
    v_ref, final_ref = O.notebook_softmax_unabsorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O,
                                                     d.C_KV, d.H, scale)
    say(f"config 1: v {rel_err(v, v_ref):.2e} final {rel_err(final, final_ref):.2e}")
    assert rel_err(v, v_ref) <= 1e-4 and rel_err(final, final_ref) <= 1e-4


# ----------------------------------------------------------------------------
# the log-sum-exp combine on its own
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [G.F32, G.BF16])
def test_lse_combine(dtype):
    rng = np.random.default_rng(17)
    P, R, H, d = 5, 3, 4, 512
    o = rng.standard_normal((P, R, H, d)).astype(np.float32)
    l = (rng.standard_normal((P, R, H)) * 20).astype(np.float32)
    l[1] = -np.inf                      # an empty part everywhere
    l[:, 2, 3] = -np.inf                # a row/head with nothing at all
    o[1] = np.nan                       # never read
    got, glse = M.lse_combine(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), dtype=dtype_torch(dtype))
    ref, rlse = O.lse_merge(o.astype(np.float64), l.astype(np.float64))
    assert rel_err(to_host64(got), ref) <= TOL[dtype]
    assert lse_err(glse.cpu().numpy(), rlse) <= 1e-4
