"""Seeded synthetic workloads for weight-absorbed latent attention.

Every array is produced on the host with numpy and stored either as float32
or as bf16 bit patterns (uint16, rounded to nearest even from float32). Both
the fp64 oracle and the HIP path consume exactly these stored values.

Input recipe (the pages give shapes, not data; these stand in for
DeepSeek-V2-shaped workloads):
  * latent c_t: iid N(0,1) rows, RMS-normalised (eps 1e-6, no gain), as the
    cached latent is described as RMS-normed on the ferrox-core page (module
    documentation of mla_absorbed.rs);
  * k_pe_t and q_pe: iid N(0,1), rotated by interleaved-pair RoPE with base
    10000 at their positions (key t at t, decode query at len-1, prefill
    query i at i + S_kv - S_q); the MLA tutorial's formula.md Part 3 only
    says the rope parts are rotated by R_i, so the convention is ours;
  * absorbed query q_abs: iid N(0,1)/sqrt(d_c);
  * q_nope (prefill): iid N(0,1); W_UK, W_UV: iid N(0, 1/d_c).
Random streams: one numpy SeedSequence per call, spawned into one child per
sequence (drawn in the order c, k_pe, q_abs|q_nope, q_pe), then one child
for weights and one for the page permutation. A single sequence can thus be
regenerated on its own.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np

F32 = "f32"
BF16 = "bf16"
BF16_NAN_BITS = np.uint16(0x7FC0)

__all__ = [
    "F32", "BF16", "bf16_bits", "bf16_bits_to_f32", "storage", "to_f64",
    "rms_normalise", "rope_interleaved", "decode_case", "prefill_case",
    "gemm_case", "config1_notebook", "config2_decode_f32",
    "config3_decode_bf16", "config4_paged_bf16", "config5_prefill_bf16",
    "p2_tiny_case", "xorshift32_stream", "seq_rows", "CONFIG_NAMES", "config4_lengths", "paged_layout",
]


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
         >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN_BITS
    return r


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def storage(x, dtype: str) -> np.ndarray:
    """Convert values to the storage representation of `dtype`."""
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(a, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (fp32 or bf16 bits)."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# input preparation upstream of the path
# --------------------------------------------------------------------------
def rms_normalise(z: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)


def rope_interleaved(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate pairs (x[2i], x[2i+1]) by angle pos * base**(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d == 0:
        return x.copy()
    assert d % 2 == 0, "rope width must be even"
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    pos = np.asarray(pos, dtype=np.float64)
    ang = pos[..., None] * inv  # [..., d/2]
    # broadcast ang over any middle axes of x
    while ang.ndim < x.ndim:
        ang = np.expand_dims(ang, axis=-2)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _normal(rng, shape, scale=1.0):
    return rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64) * scale


def _latent_rows(rng, n, d_c, d_r, start_pos=0):
    """Draw n cache rows [c | k_pe] (float64 before storage rounding)."""
    c = rms_normalise(_normal(rng, (n, d_c)))
    k_pe = rope_interleaved(_normal(rng, (n, d_r)), np.arange(start_pos, start_pos + n))
    return np.concatenate([c, k_pe], axis=1)


# --------------------------------------------------------------------------
# decode workloads (configs 2, 3, 4 and small parity cases)
# --------------------------------------------------------------------------
def _decode_sequence(child, length, H, d_c, d_r):
    rng = np.random.default_rng(child)
    rows = _latent_rows(rng, length, d_c, d_r)
    q_abs = _normal(rng, (H, d_c), 1.0 / math.sqrt(d_c))
    q_pe = rope_interleaved(_normal(rng, (H, d_r)), np.full(H, max(length - 1, 0)))
    return rows, np.concatenate([q_abs, q_pe], axis=1)


def decode_case(B, H, d_c, d_r, lens, dtype, seed=0, *, page_size=None,
                d_v=None, cache_rows=None, shuffle_pages=True, poison=True):
    """Absorbed-decode workload.

    Returns a namespace with q [B,H,W] and either a dense cache [B,S_cap,W]
    (page_size None) or a page pool [P,page_size,W] plus block_table
    [B,max_pages] (int32, -1 padded). Rows past each sequence's length and
    unused page slots hold NaN so that any read of them shows up.
    If d_v is given, W_UV [H,d_v,d_c] ~ N(0,1/d_c) is added.
    """
    lens = np.asarray(lens, dtype=np.int64).reshape(B)
    W = d_c + d_r
    ss = np.random.SeedSequence(seed)
    children = ss.spawn(B + 2)
    q = np.empty((B, H, W), dtype=np.uint16 if dtype == BF16 else np.float32)
    ns = SimpleNamespace(kind="decode", dtype=dtype, B=B, H=H, d_c=d_c, d_r=d_r,
                         W=W, lens=lens.astype(np.int32),
                         kq_scale=None, page_size=page_size, seed=seed)
    fill = np.nan if poison else 0.0
    if page_size is None:
        s_cap = int(cache_rows if cache_rows is not None else max(int(lens.max(initial=0)), 1))
        cache = np.empty((B, s_cap, W), dtype=q.dtype)
        for b in range(B):
            rows, qb = _decode_sequence(children[b], int(lens[b]), H, d_c, d_r)
            q[b] = storage(qb, dtype)
            full = np.full((s_cap, W), fill)
            full[: lens[b]] = rows
            cache[b] = storage(full, dtype)
        ns.cache = cache
        ns.cache_stride = s_cap
    else:
        npages = [(int(l) + page_size - 1) // page_size for l in lens]
        P = int(sum(npages))
        max_pages = max(max(npages, default=0), 1)
        prng = np.random.default_rng(children[B + 1])
        perm = prng.permutation(P) if shuffle_pages else np.arange(P)
        pool = np.empty((max(P, 1), page_size, W), dtype=q.dtype)
        if P == 0:
            pool[:] = storage(np.full((1, page_size, W), fill), dtype)
        table = np.full((B, max_pages), -1, dtype=np.int32)
        k = 0
        for b in range(B):
            rows, qb = _decode_sequence(children[b], int(lens[b]), H, d_c, d_r)
            q[b] = storage(qb, dtype)
            for j in range(npages[b]):
                blk = np.full((page_size, W), fill)
                part = rows[j * page_size:(j + 1) * page_size]
                blk[: part.shape[0]] = part
                pool[perm[k]] = storage(blk, dtype)
                table[b, j] = perm[k]
                k += 1
        ns.pages = pool
        ns.block_table = table
        ns.max_pages = max_pages
    ns.q = q
    if d_v is not None:
        wrng = np.random.default_rng(children[B])
        ns.d_v = d_v
        ns.w_uv = storage(_normal(wrng, (H, d_v, d_c), 1.0 / math.sqrt(d_c)), dtype)
    return ns


def paged_layout(lens, page_size, seed=0, shuffle_pages=True):
    """The page layout decode_case draws for these lengths and seed, without
    the values: (block_table [B, max_pages] int32, -1 padded; pool size P).
    Pages are dealt in (sequence, logical page) order from a seeded
    permutation of the pool."""
    lens = np.asarray(lens, dtype=np.int64)
    B = lens.shape[0]
    npages = [(int(l) + page_size - 1) // page_size for l in lens]
    P = int(sum(npages))
    max_pages = max(max(npages, default=0), 1)
    children = np.random.SeedSequence(seed).spawn(B + 2)
    prng = np.random.default_rng(children[B + 1])
    perm = prng.permutation(P) if shuffle_pages else np.arange(P)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        table[b, :npages[b]] = perm[k:k + npages[b]]
        k += npages[b]
    return table, P


def seq_rows(case, b) -> np.ndarray:
    """Stored cache rows [len_b, W] of sequence b (dense or paged)."""
    n = int(case.lens[b])
    if getattr(case, "page_size", None) is None:
        return case.cache[b, :n]
    ps = case.page_size
    npg = (n + ps - 1) // ps
    if npg == 0:
        return case.pages[:0, 0]
    rows = case.pages[case.block_table[b, :npg]].reshape(npg * ps, case.W)
    return rows[:n]


# --------------------------------------------------------------------------
# causal prefill workload (config 5 and small cases)
# --------------------------------------------------------------------------
def prefill_case(B, S_q, S_kv, H, d_nope, d_c, d_r, d_v, dtype, seed=0):
    """Causal prefill over the latent cache with absorb and up-projection weights.

    q_nope [B,S_q,H,d_nope], q_pe [B,S_q,H,d_r] (roped at i + S_kv - S_q),
    cache [B,S_kv,W], W_UK [H,d_nope,d_c], W_UV [H,d_v,d_c].
    """
    W = d_c + d_r
    ss = np.random.SeedSequence(seed)
    children = ss.spawn(B + 2)
    st = np.uint16 if dtype == BF16 else np.float32
    cache = np.empty((B, S_kv, W), dtype=st)
    q_nope = np.empty((B, S_q, H, d_nope), dtype=st)
    q_pe = np.empty((B, S_q, H, d_r), dtype=st)
    qpos = np.arange(S_q) + (S_kv - S_q)
    for b in range(B):
        rng = np.random.default_rng(children[b])
        cache[b] = storage(_latent_rows(rng, S_kv, d_c, d_r), dtype)
        q_nope[b] = storage(_normal(rng, (S_q, H, d_nope)), dtype)
        q_pe[b] = storage(rope_interleaved(_normal(rng, (S_q, H, d_r)), np.maximum(qpos, 0)[:, None].repeat(H, 1)), dtype)
    wrng = np.random.default_rng(children[B])
    w_uk = storage(_normal(wrng, (H, d_nope, d_c), 1.0 / math.sqrt(d_c)), dtype)
    w_uv = storage(_normal(wrng, (H, d_v, d_c), 1.0 / math.sqrt(d_c)), dtype)
    return SimpleNamespace(kind="prefill", dtype=dtype, B=B, S_q=S_q, S_kv=S_kv, H=H,
                           d_nope=d_nope, d_c=d_c, d_r=d_r, d_v=d_v, W=W,
                           kq_scale=1.0 / math.sqrt(d_nope + d_r), cache=cache,
                           q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, seed=seed)


def gemm_case(N, H, d_in, d_out, dtype, seed=0, transpose_w=True):
    """Per-head product inputs: x [N,H,d_in]; w [H,d_out,d_in] (transpose_w) or [H,d_in,d_out]."""
    rng = np.random.default_rng(seed)
    x = storage(_normal(rng, (N, H, d_in)), dtype)
    shape = (H, d_out, d_in) if transpose_w else (H, d_in, d_out)
    fan = d_in if transpose_w else d_out
    w = storage(_normal(rng, shape, 1.0 / math.sqrt(fan)), dtype)
    return SimpleNamespace(dtype=dtype, N=N, H=H, x=x, w=w)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny notebook MLA, fp32, d_model=100 d_c=20 H=3 d_h=20, cache 5+1",
    2: "absorbed decode fp32 B=4 H=16 d_c=512 d_r=64 S=1024",
    3: "DeepSeek-V2-shaped decode bf16 B=64 H=128 d_c=512 d_r=64 S=4096 + W_UV d_v=128",
    4: "ragged paged decode bf16 B=128 H=128 d_c=512 d_r=64 len~U[1,32768] page=64",
    5: "causal prefill bf16 B=2 S=4096 H=128 d_nope=128 d_c=512 d_r=64 d_v=128",
}


def config1_notebook(seed=0):
    """Draws of the tiny RoPE-less notebook (Colab gist MLA_RoPE-less.ipynb):
    legacy numpy global-style stream seeded with `seed`, standard normals in the
    notebook's order X, W_dQ, W_dKV, W_uQ, W_uK, W_uV, W_O, C_KV."""
    rs = np.random.RandomState(seed)
    d_1, d_2, d_3, h, existing = 100, 20, 60, 3, 5
    X = rs.randn(1, d_1)
    W_dQ = rs.randn(d_1, d_2)
    W_dKV = rs.randn(d_1, d_2)
    W_uQ = rs.randn(d_2, d_3)
    W_uK = rs.randn(d_2, d_3)
    W_uV = rs.randn(d_2, d_3)
    W_O = rs.randn(d_3, d_1)
    C_KV = rs.randn(existing, d_2)
    return SimpleNamespace(d_model=d_1, d_c=d_2, d_up=d_3, H=h, d_h=d_3 // h,
                           existing=existing, X=X, W_dQ=W_dQ, W_dKV=W_dKV,
                           W_uQ=W_uQ, W_uK=W_uK, W_uV=W_uV, W_O=W_O, C_KV=C_KV)


def config2_decode_f32(seed=0):
    c = decode_case(4, 16, 512, 64, [1024] * 4, F32, seed)
    c.kq_scale = 1.0 / math.sqrt(192.0)
    return c


def config3_decode_bf16(seed=0):
    c = decode_case(64, 128, 512, 64, [4096] * 64, BF16, seed, d_v=128, poison=False)
    c.kq_scale = 1.0 / math.sqrt(192.0)
    return c


def config4_lengths(seed=0, B=128, lo=1, hi=32768):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=B).astype(np.int32)


def config4_paged_bf16(seed=0):
    lens = config4_lengths(seed)
    c = decode_case(128, 128, 512, 64, lens, BF16, seed, page_size=64)
    c.kq_scale = 1.0 / math.sqrt(192.0)
    return c


def config5_prefill_bf16(seed=0):
    return prefill_case(2, 4096, 4096, 128, 128, 512, 64, 128, BF16, seed)


# --------------------------------------------------------------------------
# the ferrox-core unit-test shape (docs.rs page, mla_absorbed.rs test)
# --------------------------------------------------------------------------
def xorshift32_stream(seed: int):
    """Marsaglia's 32-bit xorshift generator ("Xorshift RNGs", Journal of
    Statistical Software 8(14), 2003) with the shift triple (13, 17, 5): the
    state x becomes x ^ (x << 13), then x ^ (x >> 17), then x ^ (x << 5)
    (mod 2^32), and each new state is mapped to float32 as x / (2^32 - 1) - 1/2.
    The ferrox-core absorbed-vs-naive test draws its inputs from this
    generator; its page supplies the seed, the triple, the [-1/2, 1/2) mapping
    and the draw order."""
    s = np.uint32(seed)
    umax = np.float32(4294967295.0)
    half = np.float32(0.5)
    while True:
        s = np.uint32(s ^ np.uint32((int(s) << 13) & 0xFFFFFFFF))
        s = np.uint32(s ^ (s >> np.uint32(17)))
        s = np.uint32(s ^ np.uint32((int(s) << 5) & 0xFFFFFFFF))
        yield np.float32(np.float32(s) / umax - half)


def p2_tiny_case():
    """Inputs at the ferrox-core test's shape (H=3, nope=4, rope=2, v=5,
    kv_lora=6, seq=7), drawn from the xorshift32 stream above in the order the
    page gives: every head's kv_b block ([nope+v, kv_lora], row-major), then
    the latent rows, then the naive query."""
    H, nope, rope, v_dim, kv_lora, seq = 3, 4, 2, 5, 6, 7
    g = xorshift32_stream(0x9E37)
    kv_b = np.array([[next(g) for _ in range((nope + v_dim) * kv_lora)] for _ in range(H)],
                    dtype=np.float32).reshape(H, nope + v_dim, kv_lora)
    latent = np.array([next(g) for _ in range(seq * (kv_lora + rope))],
                      dtype=np.float32).reshape(seq, kv_lora + rope)
    q_naive = np.array([next(g) for _ in range(H * (nope + rope))],
                       dtype=np.float32).reshape(H, nope + rope)
    return SimpleNamespace(H=H, d_nope=nope, d_r=rope, d_v=v_dim, d_c=kv_lora, seq=seq,
                           kv_b=kv_b, w_uk=np.ascontiguousarray(kv_b[:, :nope, :]),
                           w_uv=np.ascontiguousarray(kv_b[:, nope:, :]), latent=latent,
                           q_nope=np.ascontiguousarray(q_naive[:, :nope]),
                           q_pe=np.ascontiguousarray(q_naive[:, nope:]))
