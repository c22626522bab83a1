"""Parity of the steps around the core path (through the C ABI) with the fp64
oracle: the fused cache append and the query rope, the unabsorbed causal
prefill, full absorption, and the gated MLA variant (including the page's own
worked example on the GPU).

Bar: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32) or 2e-2 (bf16 inputs,
fp32 accumulation) per output tensor; placement in the cache bit-exact."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as G
from gpu_util import LSE_TOL, TOL, lse_err, rel_err, to_dev, to_host64

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


def rnd(rng, shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def stored(a, dtype):
    """(device tensor, exact float64 copy of the stored values)"""
    st = G.storage(a, dtype)
    return to_dev(st, dtype), G.to_f64(st, dtype)


# ----------------------------------------------------------------------------
# fused cache append
# ----------------------------------------------------------------------------
def _append_case(dtype, N, d_model, d_c, d_r, paged, seed, n_seqs=4, page=64, bad=()):
    # paged: positions up to 40000 (large rotation angles), pool pages only for
    # the logical pages written (other table entries -1); dense: 2000 rows
    cap = 40000 if paged else 2000
    rng = np.random.default_rng(seed)
    x_d, x = stored(rnd(rng, (N, d_model)), dtype)
    wc_d, wc = stored(rnd(rng, (d_c, d_model), 1 / math.sqrt(d_model)), dtype)
    wk_d, wk = stored(rnd(rng, (d_r, d_model), 1 / math.sqrt(d_model)), dtype)
    seq = rng.integers(0, n_seqs, N).astype(np.int32)
    pos = rng.integers(0, cap, N).astype(np.int32)
    pos[0] = 0
    pos[-1] = cap - 1
    # distinct (sequence, position) pairs so every addressed slot has one writer
    pairs = {}
    for n in range(N):
        while (int(seq[n]), int(pos[n])) in pairs:
            pos[n] = (pos[n] + 1) % cap
        pairs[(int(seq[n]), int(pos[n]))] = n
    for n in bad:                     # tokens the cache cannot hold: skipped
        pos[n] = cap + 5
    W = d_c + d_r
    sentinel = 7.0
    if paged:
        npg = (cap + page - 1) // page
        used = sorted({(int(seq[n]), int(pos[n]) // page) for n in range(N) if n not in bad})
        table = np.full((n_seqs, npg), -1, dtype=np.int32)
        perm = rng.permutation(len(used))
        for k, (b_, j) in enumerate(used):
            table[b_, j] = perm[k]
        cache0 = np.full((len(used), page, W), sentinel)
    else:
        table = None
        cache0 = np.full((n_seqs, cap, W), sentinel)
    return dict(x_d=x_d, x=x, wc_d=wc_d, wc=wc, wk_d=wk_d, wk=wk, seq=seq, pos=pos, table=table,
                cache0=cache0, dtype=dtype, d_c=d_c, d_r=d_r, bad=set(bad))


@pytest.mark.parametrize("dtype,N,d_model,d_c,d_r,paged", [
    (G.BF16, 64, 5120, 512, 64, True),      # one decode token per sequence, DeepSeek-V2 widths (split-K MFMA)
    (G.BF16, 37, 2048, 512, 64, False),     # ragged token count, 16 K splits of two 64-wide slices
    (G.BF16, 300, 1024, 512, 64, False),    # a prefill chunk, dense cache
    (G.F32, 9, 100, 20, 4, True),           # fp32, widths off the MFMA tiles (generic product)
    (G.F32, 1100, 96, 20, 4, False),        # enough tokens for the wave-per-token row epilogue
    (G.BF16, 1536, 1024, 512, 64, True),    # the same epilogue at DeepSeek-V2 row widths, paged
])
def test_cache_append(dtype, N, d_model, d_c, d_r, paged):
    say(f"cache append: {dtype} N={N} d_model={d_model} d_c={d_c} d_r={d_r} paged={paged}")
    c = _append_case(dtype, N, d_model, d_c, d_r, paged, seed=N + d_model, bad=(1,))
    cache = to_dev(G.storage(c["cache0"], dtype), dtype)
    seq_d = torch.from_numpy(c["seq"]).cuda()
    pos_d = torch.from_numpy(c["pos"]).cuda()
    table_d = None if c["table"] is None else torch.from_numpy(c["table"]).cuda()
    M.cache_append(c["x_d"], c["wc_d"], c["wk_d"], seq_d, pos_d, cache, block_table=table_d, eps=1e-6)
    torch.cuda.synchronize()
    got = to_host64(cache)
    rows = O.latent_cache_rows(c["x"], c["wc"], c["wk"], c["pos"], 1e-6, 10000.0)
    keep = [n for n in range(N) if n not in c["bad"]]
    want = O.append_rows(c["cache0"], rows[keep], c["seq"][keep], c["pos"][keep], c["table"])
    written = np.any(want != c["cache0"], axis=-1)
    changed = np.any(got != c["cache0"], axis=-1)
    assert np.array_equal(written, changed), "rows written at the wrong slots (or a skipped token written)"
    e = rel_err(got[written], want[written])
    say(f"  rows rel err {e:.2e}, {int(written.sum())} rows placed")
    assert e <= TOL[dtype]


def test_append_then_decode_sees_itself():
    """The notebook's order: the new row is appended before the query attends,
    so a decode over len+1 positions includes the token's own row."""
    rng = np.random.default_rng(77)
    B, H, d_model, d_c, d_r, L0 = 3, 128, 1024, 512, 64, 100
    case = G.decode_case(B, H, d_c, d_r, [L0] * B, G.BF16, seed=78, cache_rows=L0 + 1, poison=False)
    case.kq_scale = 1.0 / math.sqrt(192)
    x_d, x = stored(rnd(rng, (B, d_model)), G.BF16)
    wc_d, wc = stored(rnd(rng, (d_c, d_model), 1 / math.sqrt(d_model)), G.BF16)
    wk_d, wk = stored(rnd(rng, (d_r, d_model), 1 / math.sqrt(d_model)), G.BF16)
    cache = to_dev(case.cache, G.BF16)
    seq = torch.arange(B, dtype=torch.int32).cuda()
    pos = torch.full((B,), L0, dtype=torch.int32).cuda()
    M.cache_append(x_d, wc_d, wk_d, seq, pos, cache)
    lens = torch.full((B,), L0 + 1, dtype=torch.int32).cuda()
    out, lse = M.latent_decode(to_dev(case.q, G.BF16), cache, lens, d_c, case.kq_scale)
    torch.cuda.synchronize()
    got = to_host64(out)
    new = O.latent_cache_rows(x, wc, wk, np.full(B, L0), 1e-6, 10000.0)
    for b in range(B):
        lat = np.vstack([G.to_f64(case.cache[b, :L0], G.BF16), G.to_f64(G.storage(new[b:b + 1], G.BF16), G.BF16)])
        ref, _ = O.latent_attention(G.to_f64(case.q[b], G.BF16), lat, d_c, case.kq_scale, L0 + 1)
        e = rel_err(got[b], ref)
        say(f"  seq {b}: rel err {e:.2e}")
        assert e <= TOL[G.BF16]


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
def test_absorb_q_rope(dtype):
    rng = np.random.default_rng(5)
    N, H, dn, dc, dr = 50, 8, 128, 512, 64
    qn_d, qn = stored(rnd(rng, (N, H, dn)), dtype)
    qp_d, qp = stored(rnd(rng, (N, H, dr)), dtype)
    w_d, w = stored(rnd(rng, (H, dn, dc), 1 / math.sqrt(dc)), dtype)
    pos = rng.integers(0, 40000, N).astype(np.int32)
    got = to_host64(M.absorb_q_rope(qn_d, qp_d, w_d, torch.from_numpy(pos).cuda()))
    ref = O.absorb_query(qn, O.rope(qp, pos[:, None], 10000.0), w)
    e1, e2 = rel_err(got[..., :dc], ref[..., :dc]), rel_err(got[..., dc:], ref[..., dc:])
    say(f"absorb + rope {dtype}: absorbed {e1:.2e} rope {e2:.2e}")
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype]


# ----------------------------------------------------------------------------
# unabsorbed causal prefill
# ----------------------------------------------------------------------------
def _unabsorbed_ref(case, b):
    lat = G.to_f64(case.cache[b], case.dtype)
    wuk, wuv = G.to_f64(case.w_uk, case.dtype), G.to_f64(case.w_uv, case.dtype)
    K, V = O.expand_per_head(lat, case.d_c, wuk, wuv)
    q = np.concatenate([G.to_f64(case.q_nope[b], case.dtype), G.to_f64(case.q_pe[b], case.dtype)], axis=2)
    return O.mha_attention(q, K, V, case.kq_scale, True)


@pytest.mark.parametrize("H,d_r,S_q,S_kv", [
    (4, 64, 150, 150),     # ragged query and key blocks
    (2, 64, 70, 200),      # a chunk at the end of a longer cache
    (2, 64, 200, 70),      # more queries than cache rows: the first see nothing
    (3, 0, 130, 130),      # no rope part
])
def test_prefill_unabsorbed_small(H, d_r, S_q, S_kv):
    say(f"unabsorbed prefill: H={H} d_r={d_r} S_q={S_q} S_kv={S_kv}")
    case = G.prefill_case(2, S_q, S_kv, H, 128, 512, d_r, 128, G.BF16, seed=40 + H + S_q)
    qn, qp = to_dev(case.q_nope, G.BF16), to_dev(case.q_pe, G.BF16) if d_r else None
    out, lse = M.prefill_unabsorbed(qn, qp, to_dev(case.cache, G.BF16), to_dev(case.w_uk, G.BF16),
                                    to_dev(case.w_uv, G.BF16), case.kq_scale)
    torch.cuda.synchronize()
    got, glse = to_host64(out), lse.cpu().numpy().astype(np.float64)
    for b in range(2):
        ro, rl = _unabsorbed_ref(case, b)
        e, le = rel_err(got[b], ro), lse_err(glse[b], rl)
        say(f"  b={b}: out {e:.2e} lse {le:.2e}")
        assert e <= TOL[G.BF16] and le <= LSE_TOL[G.BF16]
        if S_q > S_kv:
            assert np.all(got[b, :S_q - S_kv] == 0) and np.all(np.isneginf(glse[b, :S_q - S_kv]))


def test_prefill_unabsorbed_matches_absorbed_chain():
    """Both forms of the same causal prefill: expanded per head, and absorbed
    (mla_absorb_q -> mla_latent_prefill_causal -> mla_up_v)."""
    case = G.prefill_case(1, 257, 257, 128, 128, 512, 64, 128, G.BF16, seed=9)
    qn, qp = to_dev(case.q_nope, G.BF16), to_dev(case.q_pe, G.BF16)
    cache, wuk, wuv = to_dev(case.cache, G.BF16), to_dev(case.w_uk, G.BF16), to_dev(case.w_uv, G.BF16)
    out_u, lse_u = M.prefill_unabsorbed(qn, qp, cache, wuk, wuv, case.kq_scale)
    q = M.absorb_q(qn.reshape(257, 128, -1), qp.reshape(257, 128, -1), wuk)
    lat, lse_a = M.latent_prefill_causal(q.reshape(1, 257, 128, -1), cache, 512, case.kq_scale)
    v = M.up_v(lat.reshape(257, 128, -1), wuv)
    torch.cuda.synchronize()
    e = rel_err(to_host64(out_u).reshape(257, 128, -1), to_host64(v))
    le = float(torch.max(torch.abs(lse_u - lse_a)))
    say(f"unabsorbed vs absorbed chain: out {e:.2e} lse {le:.2e}")
    assert e <= TOL[G.BF16] and le <= LSE_TOL[G.BF16]
    # and against the oracle on sampled rows
    lat64, wuk64, wuv64 = G.to_f64(case.cache[0], G.BF16), G.to_f64(case.w_uk, G.BF16), G.to_f64(case.w_uv, G.BF16)
    got = to_host64(out_u)[0]
    for i in (0, 63, 64, 200, 256):
        ref, _ = O.mla_unabsorbed(G.to_f64(case.q_nope[0, i], G.BF16), G.to_f64(case.q_pe[0, i], G.BF16), lat64,
                                  512, wuk64, wuv64, case.kq_scale, i + 1)
        assert rel_err(got[i], ref) <= TOL[G.BF16]


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_config5_unabsorbed_sampled():
    case = G.config5_prefill_bf16(0)
    say("config 5 (expanded form) generated; running")
    out, lse = M.prefill_unabsorbed(to_dev(case.q_nope, G.BF16), to_dev(case.q_pe, G.BF16),
                                    to_dev(case.cache, G.BF16), to_dev(case.w_uk, G.BF16),
                                    to_dev(case.w_uv, G.BF16), case.kq_scale)
    torch.cuda.synchronize()
    got, glse = to_host64(out), lse.cpu().numpy()
    wuk, wuv = G.to_f64(case.w_uk, G.BF16), G.to_f64(case.w_uv, G.BF16)
    for b in range(2):
        lat = G.to_f64(case.cache[b], G.BF16)
        for i in [0, 1, 127, 128, 2049, 4095]:
            # every head of the short rows, every 4th head (and the last) of the long ones
            hs = np.arange(128) if i <= 128 else np.r_[np.arange(0, 128, 4), 127]
            ref, rl = O.mla_unabsorbed(G.to_f64(case.q_nope[b, i, hs], G.BF16), G.to_f64(case.q_pe[b, i, hs], G.BF16),
                                       lat[:i + 1], 512, wuk[hs], wuv[hs], case.kq_scale, i + 1)
            e, le = rel_err(got[b, i, hs], ref), lse_err(glse[b, i, hs], rl)
            say(f"  b={b} i={i}: {len(hs)} heads: out {e:.2e} lse {le:.2e}")
            assert e <= 2e-2 and le <= 2e-2


# ----------------------------------------------------------------------------
# full absorption
# ----------------------------------------------------------------------------
def test_full_absorption_notebook():
    """The notebook's workload (fp32, RoPE-less, 3 heads) through the fully
    absorbed path: absorbed weights, query from the query latent, latent
    decode over the cache with the new token appended, head-summed output."""
    d = G.config1_notebook(0)
    H, dh = d.H, d.d_h
    scale = 1.0 / math.sqrt(dh)
    blk = lambda W: np.stack([W[:, s * dh:(s + 1) * dh].T for s in range(H)])   # [H, d_h, d_c]
    st = lambda a: to_dev(G.storage(a, G.F32), G.F32)
    a_qk, a_vo = M.absorb_weights(st(blk(d.W_uQ)), st(blk(d.W_uK)), st(blk(d.W_uV)), st(d.W_O.T))
    ref_qk, ref_vo = O.full_absorbed_weights(blk(d.W_uQ), blk(d.W_uK), blk(d.W_uV), d.W_O.T)
    assert rel_err(to_host64(a_qk), ref_qk) <= 1e-4 and rel_err(to_host64(a_vo), ref_vo) <= 1e-4
    cache = np.vstack([d.C_KV, d.X @ d.W_dKV])
    q = M.absorb_q_full(st(d.X @ d.W_dQ), None, a_qk)
    lat, _ = M.latent_decode(q, st(cache[None]), torch.tensor([cache.shape[0]], dtype=torch.int32).cuda(),
                             d.d_c, scale)
    final = to_host64(M.out_absorbed(lat, a_vo))[0]
    _, final_ref = O.notebook_softmax_unabsorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O, d.C_KV, H,
                                                 scale)
    e = rel_err(final, final_ref)
    say(f"full absorption, notebook: final rel err {e:.2e}")
    assert e <= 1e-4


def test_full_absorption_bf16():
    rng = np.random.default_rng(31)
    H, dn, dcq, dc, dr, dv, dm = 16, 128, 1536, 512, 64, 128, 2048
    lens = [300, 1, 77, 128]
    B = len(lens)
    uq_d, uq = stored(rnd(rng, (H, dn, dcq), 1 / math.sqrt(dcq)), G.BF16)
    uk_d, uk = stored(rnd(rng, (H, dn, dc), 1 / math.sqrt(dc)), G.BF16)
    uv_d, uv = stored(rnd(rng, (H, dv, dc), 1 / math.sqrt(dc)), G.BF16)
    wo_d, wo = stored(rnd(rng, (dm, H * dv), 1 / math.sqrt(H * dv)), G.BF16)
    cq_d, cq = stored(rnd(rng, (B, dcq)), G.BF16)
    qp_d, qp = stored(rnd(rng, (B, H, dr)), G.BF16)
    case = G.decode_case(B, H, dc, dr, lens, G.BF16, seed=32, poison=False)
    scale = 1.0 / math.sqrt(dn + dr)
    a_qk, a_vo = M.absorb_weights(uq_d, uk_d, uv_d, wo_d)
    q = M.absorb_q_full(cq_d, qp_d, a_qk)
    lat, _ = M.latent_decode(q, to_dev(case.cache, G.BF16), torch.tensor(lens, dtype=torch.int32).cuda(), dc, scale)
    out = to_host64(M.out_absorbed(lat, a_vo))
    for b in range(B):
        latb = G.to_f64(G.seq_rows(case, b), G.BF16)
        ref = O.training_form_decode(cq[b], qp[b], latb, dc, uq, uk, uv, wo, scale, lens[b])
        e = rel_err(out[b], ref)
        say(f"  seq {b} len {lens[b]}: final rel err {e:.2e}")
        assert e <= TOL[G.BF16]


@pytest.mark.parametrize("H,d_cq,d_model,N,dc", [
    (64, 768, 1000, 37, 512),  # output: 4 row tiles (the last ragged) x 64 K splits of 2 blocks (one block pair)
    (64, 1280, 256, 64, 512),  # 64 tokens (the stream's largest), one output row tile
    (8, 1536, 5120, 5, 512),   # output: 20 row tiles x 12 splits of 1-2 blocks (the tail-only block path)
    (1, 256, 4, 1, 256),       # one token, 4 output rows of one 256-wide K block (one split, one block)
    (2, 256, 8, 64, 512),      # 64 tokens against 8 output rows, 4 K blocks in 4 splits
])
def test_full_absorption_weight_stream(H, d_cq, d_model, N, dc):
    """Decode-sized fully absorbed layer (bf16): the head-summed output of at
    most 64 tokens runs on the weight-streaming kernel. The latent output of
    every token against the oracle's absorbed decode (checks the query), then
    the layer output."""
    rng = np.random.default_rng(40 + H + N)
    dr = 64
    aqk_d, aqk = stored(rnd(rng, (H, dc, d_cq), 1 / math.sqrt(d_cq)), G.BF16)
    avo_d, avo = stored(rnd(rng, (d_model, H * dc), 1 / math.sqrt(H * dc)), G.BF16)
    cq_d, cq = stored(rnd(rng, (N, d_cq)), G.BF16)
    qp_d, qp = stored(rnd(rng, (N, H, dr)), G.BF16)
    lens = [int(x) for x in rng.integers(1, 40, N)]
    case = G.decode_case(N, H, dc, dr, lens, G.BF16, seed=43, poison=False)
    scale = 1.0 / math.sqrt(128 + dr)
    q = M.absorb_q_full(cq_d, qp_d, aqk_d)
    lat, _ = M.latent_decode(q, to_dev(case.cache, G.BF16), torch.tensor(lens, dtype=torch.int32).cuda(), dc,
                             scale)
    out = to_host64(M.out_absorbed(lat, avo_d))
    lat_h = to_host64(lat)
    e_lat = e_out = 0.0
    for b in range(N):
        latb = G.to_f64(G.seq_rows(case, b), G.BF16)
        ref, ref_lat = O.full_absorbed_decode(cq[b], qp[b], latb, dc, aqk, avo, scale, lens[b])
        e_lat = max(e_lat, rel_err(lat_h[b], ref_lat))
        e_out = max(e_out, rel_err(out[b], ref))
    say(f"H={H} d_cq={d_cq} d_model={d_model} N={N}: latent {e_lat:.2e} output {e_out:.2e}")
    assert e_lat <= TOL[G.BF16] and e_out <= TOL[G.BF16]


# ----------------------------------------------------------------------------
# gated MLA
# ----------------------------------------------------------------------------
def test_gated_worked_example_on_gpu(golden_dir):
    """The page's numeric example through the library: output 1.0, cache 2.0."""
    import json
    import os
    g = json.load(open(os.path.join(golden_dir, "gated_example.json")))["numeric_example"]
    t = lambda k: torch.tensor(g[k], dtype=torch.float32).cuda()
    res = M.gated_mla(t("hidden_states"), t("query_projection"), t("latent_down_projection"),
                      t("key_up_projection"), t("value_up_projection"), t("output_gate_projection"),
                      t("output_projection"), g["num_heads"], g["causal"])
    torch.cuda.synchronize()
    assert res["output"].cpu().tolist() == g["expected_output"]
    assert res["latent_cache"].cpu().tolist() == g["expected_latent_cache"]


@pytest.mark.parametrize("dtype,B,S,D,L,H,causal", [
    (G.BF16, 2, 200, 256, 64, 2, True),     # D_h = 128: per-head attention over expanded K, V, gate fused
    (G.BF16, 2, 200, 256, 64, 2, False),
    (G.BF16, 1, 150, 256, 96, 4, True),     # D_h = 64: the absorbed latent route
    (G.BF16, 1, 4096, 2048, 512, 16, True), # projections on 256 x 256 tiles ([Q | G] and [K | V] in one product each)
    (G.F32, 1, 3, 2, 1, 2, False),          # the page's second shape example
    (G.F32, 1, 2, 2, 1, 1, True),           # the page's first shape example
    (G.F32, 2, 33, 24, 8, 3, True),
])
def test_gated_mla(dtype, B, S, D, L, H, causal):
    say(f"gated MLA: {dtype} B={B} S={S} D={D} L={L} H={H} causal={causal}")
    rng = np.random.default_rng(B * 1000 + S + D + H)
    x_d, x = stored(rnd(rng, (B, S, D)), dtype)
    ws = {}
    for name, shape, fan in (("q", (D, D), D), ("c", (L, D), D), ("k", (D, L), L), ("v", (D, L), L),
                             ("g", (D, D), D), ("o", (D, D), D)):
        ws[name] = stored(rnd(rng, shape, 1 / math.sqrt(fan)), dtype)
    res = M.gated_mla(x_d, *(ws[n][0] for n in "qckvgo"), H, causal)
    torch.cuda.synchronize()
    ref = O.gated_mla(x, *(ws[n][1] for n in "qckvgo"), H, causal)
    e1 = rel_err(to_host64(res["output"]), ref["output"])
    e2 = rel_err(to_host64(res["latent_cache"]), ref["latent_cache"])
    say(f"  output {e1:.2e} latent cache {e2:.2e}")
    assert e1 <= TOL[dtype] and e2 <= TOL[dtype]
    assert res["output"].shape == (B, S, D) and res["latent_cache"].shape == (B, S, L)
