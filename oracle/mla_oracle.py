"""fp64 CPU oracle for weight-absorbed Multi-head Latent Attention.

Test infrastructure: only tests/, the smoke check and the benchmark's
CPU-baseline leg use this module. It is deliberately plain and slow.

Sources (the pages are cited by title and part, never by line):
  [ferrox]   docs.rs, ferrox-core 0.23.0, src/mla_absorbed.rs: module
             documentation (score / out_lat / v formulas, kq_scale rule),
             the function `causal_mla_absorbed_attention` (layouts, two-pass
             softmax with an empty-sum guard) and its unit test
             `absorbed_equals_naive_for_the_same_kv_b` (kv_b row layout,
             per-head expansion, tolerances).
  [notebook] Colab gist "MLA_RoPE-less.ipynb": head split, full matrix
             absorption (W_aQK, W_aVO), cache append, printed shapes.
  [lab]      lynx-cortex "Lab 01 - MLA math exercise", Bloque A (cache size
             per token) and Bloque B (the identity q^T W_UK c = (W_UK^T q)^T c).
  [gated]    tensortonic "Kimi K3 step 2: Gated MLA": problem statement,
             worked example, causal-mask hint.
  [tutorial] uithub preacher-1/MLA_tutorial, formula.md Part 3: training form
             (per-head k, v from c) and inference form (absorbed q, shared
             key [c, k_pe], value c, causal sum over i <= t).

Readings adopted where the pages are silent:
  * logits are scaled by kq_scale = 1/sqrt(d_nope + d_r) ([ferrox] module
    doc); the tutorial's formula omits the scale and the notebook has no
    softmax at all;
  * causal alignment is bottom-right: query i of S_q sees cache positions
    t <= i + S_kv - S_q (the diagonal included, [gated] hint 2);
  * lse is the natural log of the softmax denominator, max included; an
    empty visible range gives a zero output and lse = -inf ([ferrox] guard).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attend_one_head", "expand_per_head", "mla_unabsorbed", "latent_attention",
    "latent_attention_expanded_v", "absorb_query", "up_project",
    "causal_visible", "latent_prefill_causal", "lse_merge",
    "mha_cache_values_per_token", "mla_cache_values_per_token", "cache_ratio",
    "notebook_head_blocks", "notebook_linear_absorbed", "notebook_linear_unabsorbed",
    "notebook_softmax_unabsorbed", "gated_mla",
    "rms_norm", "rope", "latent_cache_rows", "append_rows", "mha_attention",
    "full_absorbed_weights", "full_absorbed_decode", "training_form_decode",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# the attention definition
# --------------------------------------------------------------------------
def attend_one_head(q, K, V, scale, n_visible):
    """Scaled dot-product softmax attention of one query over one head's cache.

    q [d_k], K [T, d_k], V [T, d_v]; only positions 0..n_visible-1 take part.
    Logits s_t = (q . K_t) * scale; softmax by subtracting the max,
    exponentiating and dividing by the sum, as `causal_mla_absorbed_attention`
    does ([ferrox]); output = sum_t p_t V_t. Nothing visible => zeros, -inf.
    Returns (out [d_v], lse) with lse = max + log(sum exp(s - max)).
    Pinned by: brute-force scalar loops, the two-token closed form, the
    single-position example of [gated], shift and permutation invariances.
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    n = int(n_visible)
    if n <= 0:
        return np.zeros(V.shape[1]), -math.inf
    s = (K[:n] @ q) * scale
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    p = e / z
    return p @ V[:n], float(m + math.log(z))


def expand_per_head(latent, d_c, w_uk=None, w_uv=None, H=None):
    """Per-head key and value caches from the latent rows (the "naive" form).

    latent [T, d_c + d_r] rows [c_t | k_pe_t]. With weights (kv_b rows of
    [ferrox]'s test: W_UK[h] [d_nope, d_c], W_UV[h] [d_v, d_c]):
        k[t,h] = [W_UK[h] c_t , k_pe_t],   v[t,h] = W_UV[h] c_t
    as the test expands every position through kv_b and the tutorial's
    training form builds k, v per head from c. Without W_UK (the query is
    already in latent coordinates) the key of every head is the shared row
    [c_t | k_pe_t]; without W_UV the value of every head is c_t ([ferrox]
    module doc: one shared key per position, value a prefix of it).
    Returns K [T, H, d_k], V [T, H, d_v] in the [seq, n_heads, dim] layout.
    """
    latent = _f64(latent)
    c, k_pe = latent[:, :d_c], latent[:, d_c:]
    T = latent.shape[0]
    if w_uk is not None:
        w_uk = _f64(w_uk)
        H = w_uk.shape[0]
        k_nope = np.einsum("hij,tj->thi", w_uk, c)
        K = np.concatenate([k_nope, np.broadcast_to(k_pe[:, None, :], (T, H, k_pe.shape[1]))], axis=2)
    else:
        K = np.repeat(latent[:, None, :], H, axis=1)
    if w_uv is not None:
        w_uv = _f64(w_uv)
        V = np.einsum("hij,tj->thi", w_uv, c)
    else:
        V = np.repeat(c[:, None, :], H, axis=1)
    return K, V


def mla_unabsorbed(q_nope, q_pe, latent, d_c, w_uk, w_uv, scale, n_visible):
    """Unabsorbed MLA for one query token: expand K, V per head, then attend.

    q_nope [H, d_nope], q_pe [H, d_r]; per-head query [q_nope | q_pe] against
    k[t,h] = [W_UK[h] c_t | k_pe_t] and values W_UV[h] c_t ([ferrox] test,
    naive branch; [tutorial] training form). Returns (v [H, d_v], lse [H]).
    Pinned by: equality with the absorbed chain on the [ferrox] test inputs
    and on the notebook workload, and the wrong-scale check of that test.
    """
    q = np.concatenate([_f64(q_nope), _f64(q_pe)], axis=1)
    K, V = expand_per_head(latent, d_c, w_uk, w_uv)
    H = q.shape[0]
    out = np.zeros((H, V.shape[2]))
    lse = np.full(H, -math.inf)
    for h in range(H):
        out[h], lse[h] = attend_one_head(q[h], K[:, h, :], V[:, h, :], scale, n_visible)
    return out, lse


def latent_attention(q, latent, d_c, scale, n_visible, heads=None):
    """Attention of absorbed queries over the latent cache (the definition).

    q [H, d_c + d_r] rows [q_abs | q_pe]; latent [T, d_c + d_r]. Each head's
    key is the shared row [c_t | k_pe_t] and its value is c_t, so
        score[h,t] = (q_abs[h].c_t + q_pe[h].k_pe_t) * scale
        out_lat[h] = sum_t softmax(score[h])_t c_t
    ([ferrox] module doc; [tutorial] inference form). `heads` restricts the
    computation to a subset of heads (sampled checks at large sizes).
    Returns (out_lat [len(heads), d_c], lse [len(heads)]).
    Pinned by: the absorbed == unabsorbed equality, one-position output = c_0,
    q = 0 => mean of c, shift/permutation invariance, brute-force loops.
    """
    q, latent = _f64(q), _f64(latent)
    heads = range(q.shape[0]) if heads is None else heads
    heads = list(heads)
    out = np.zeros((len(heads), d_c))
    lse = np.full(len(heads), -math.inf)
    K = latent               # the key row of every head
    V = latent[:, :d_c]      # the value of every head
    for i, h in enumerate(heads):
        out[i], lse[i] = attend_one_head(q[h], K, V, scale, n_visible)
    return out, lse


def latent_attention_expanded_v(q, latent, d_c, w_uv, scale, n_visible, heads=None):
    """As latent_attention, but with the value expanded per head: v_t = W_UV[h] c_t.

    This is the output after the up-projection computed the unabsorbed way
    (values expanded before the weighted sum; [ferrox] test, naive branch).
    Returns (v [len(heads), d_v], lse).
    """
    q, latent, w_uv = _f64(q), _f64(latent), _f64(w_uv)
    heads = list(range(q.shape[0]) if heads is None else heads)
    out = np.zeros((len(heads), w_uv.shape[1]))
    lse = np.full(len(heads), -math.inf)
    c = latent[:, :d_c]
    for i, h in enumerate(heads):
        Vh = c @ w_uv[h].T
        out[i], lse[i] = attend_one_head(q[h], latent, Vh, scale, n_visible)
    return out, lse


# --------------------------------------------------------------------------
# the per-head products around the attention
# --------------------------------------------------------------------------
def absorb_query(q_nope, q_pe, w_uk):
    """q_abs[..., h, j] = sum_i W_UK[h, i, j] q_nope[..., h, i]; then [q_abs | q_pe].

    W_UK[h] is the k_b block of kv_b, [d_nope, d_c] ([ferrox] test, absorbed
    branch: the query pushed through k_b); it is W_UK^T q of the [lab]
    identity and q W_qc W_kc^T of the [tutorial] inference form.
    Pinned by: the [lab] identity q^T W_UK c = (W_UK^T q)^T c on random
    inputs and the absorbed == unabsorbed equality.
    """
    q_nope, w_uk = _f64(q_nope), _f64(w_uk)
    q_abs = np.einsum("hij,...hi->...hj", w_uk, q_nope)
    if q_pe is None:
        return q_abs
    return np.concatenate([q_abs, _f64(q_pe)], axis=-1)


def up_project(out_lat, w_uv):
    """v[..., h, i] = sum_j W_UV[h, i, j] out_lat[..., h, j] (W_UV[h] = v_b, [d_v, d_c]).

    [ferrox] module doc: v[h] = wv_b[h] . out_lat[h]; [tutorial] inference
    form: o_t^(s) W_v^(s). Pinned by: the absorbed == unabsorbed equality and
    associativity with the per-head expanded values.
    """
    return np.einsum("hij,...hj->...hi", _f64(w_uv), _f64(out_lat))


# --------------------------------------------------------------------------
# causal prefill
# --------------------------------------------------------------------------
def causal_visible(i, S_q, S_kv):
    """Number of cache positions query i may see: t <= i + S_kv - S_q, clamped to [0, S_kv]."""
    return int(min(max(i + 1 + S_kv - S_q, 0), S_kv))


def latent_prefill_causal(q, latent, d_c, scale, rows=None, heads=None):
    """Causal latent attention for a chunk of S_q queries over S_kv cache rows.

    q [S_q, H, W], latent [S_kv, W]. Query i attends to the cache positions
    the causal mask leaves visible ([gated]: later positions are masked
    before the softmax; [tutorial]: sums over i <= t). `rows` restricts the
    queries computed. Returns (out_lat [len(rows), H', d_c], lse [len(rows), H']).
    """
    q = _f64(q)
    S_q = q.shape[0]
    S_kv = np.asarray(latent).shape[0]
    rows = list(range(S_q) if rows is None else rows)
    hs = list(range(q.shape[1]) if heads is None else heads)
    out = np.zeros((len(rows), len(hs), d_c))
    lse = np.full((len(rows), len(hs)), -math.inf)
    for r, i in enumerate(rows):
        out[r], lse[r] = latent_attention(q[i], latent, d_c, scale, causal_visible(i, S_q, S_kv), hs)
    return out, lse


# --------------------------------------------------------------------------
# merging results over disjoint position ranges
# --------------------------------------------------------------------------
def lse_merge(outs, lses):
    """Merge softmax results computed over disjoint position ranges.

    outs [P, ..., d] (each normalised over its own range), lses [P, ...].
    lse = log sum_s exp(lse_s); out = sum_s exp(lse_s - lse) out_s. Ranges
    with lse_s = -inf contribute nothing; all empty => zeros and -inf.
    This is the exact identity behind splitting the positions of one query
    (no page states it; the split-sequence decode needs it). Pinned by:
    merging the oracle's attention over sub-ranges equals the oracle's
    attention over the whole range.
    """
    outs, lses = _f64(outs), _f64(lses)
    m = np.max(lses, axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_m), 0.0)
    z = w.sum(axis=0)
    lse = np.where(z > 0, safe_m + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    wn = np.where(z > 0, w / np.where(z > 0, z, 1.0), 0.0)
    out = np.einsum("p...,p...d->...d", wn, np.where(np.isfinite(lses)[..., None], outs, 0.0))
    return out, lse


# --------------------------------------------------------------------------
# cache accounting ([lab] Bloque A)
# --------------------------------------------------------------------------
def mha_cache_values_per_token(L, H, d_head):
    """Standard attention caches K and V per layer and head: 2 L H d_head values per token."""
    return 2 * L * H * d_head


def mla_cache_values_per_token(L, d_c, d_r):
    """MLA caches c_t and the decoupled rope key: L (d_c + d_r) values per token."""
    return L * (d_c + d_r)


def cache_ratio(H, d_head, d_c, d_r):
    """M_MHA / M_MLA = 2 H d_head / (d_c + d_r) (the layer count cancels)."""
    return 2 * H * d_head / (d_c + d_r)


# --------------------------------------------------------------------------
# the RoPE-less notebook ([notebook])
# --------------------------------------------------------------------------
def notebook_head_blocks(W_up, W_out, h):
    """Per-head blocks of the notebook's weights.

    The up-projections W_up [d_c, h d_h] hold head s in columns
    s d_h .. (s+1) d_h - 1 (the head index is the slower of the two factors
    the column index splits into); the output projection W_out [h d_h, d_model]
    holds head s in rows s d_h .. (s+1) d_h - 1. Returns (list of [d_c, d_h]
    blocks, list of [d_h, d_model] blocks).
    Pinned by: entries tagged with their own column / row index land in the
    block of their head (tests), and the per-head softmax workload.
    """
    W_up, W_out = _f64(W_up), _f64(W_out)
    d_h = W_up.shape[1] // h
    ups = [W_up[:, s * d_h:(s + 1) * d_h] for s in range(h)]
    outs = [W_out[s * d_h:(s + 1) * d_h, :] for s in range(h)]
    return ups, outs


def notebook_linear_absorbed(X, W_dQ, W_dKV, W_uQ, W_uK, W_uV, W_O, C_KV, h):
    """The notebook's fully absorbed, softmax-free computation, from its math.

    For head s: A_QK(s) = U_Q(s) U_K(s)^T ([d_c, d_c]) and
    A_VO(s) = U_V(s) O(s) ([d_c, d_model]); the cache gains the new latent
    row x W_dKV; the latent query of head s is (x W_dQ) A_QK(s); its
    unnormalised "attention" row is that query times every cache row; the
    head output is that row times (cache A_VO(s)); the result sums the heads.
    Returns the arrays whose shapes the notebook prints, keyed by its printed
    labels.
    """
    X, W_dQ, W_dKV = _f64(X), _f64(W_dQ), _f64(W_dKV)
    uQ, O_blocks = notebook_head_blocks(W_uQ, W_O, h)
    uK, _ = notebook_head_blocks(W_uK, W_O, h)
    uV, _ = notebook_head_blocks(W_uV, W_O, h)
    cache = np.vstack([_f64(C_KV), X @ W_dKV])                  # [T, d_c]
    c_q = X @ W_dQ                                              # [1, d_c]
    a_qk = np.stack([uQ[s] @ uK[s].T for s in range(h)])        # [h, d_c, d_c]
    a_vo = np.stack([uV[s] @ O_blocks[s] for s in range(h)])    # [h, d_c, d_model]
    latent_query = np.stack([c_q @ a_qk[s] for s in range(h)])  # [h, 1, d_c]
    total = np.zeros((1, O_blocks[0].shape[1]))
    for s in range(h):
        weights = latent_query[s] @ cache.T                     # [1, T], no softmax
        total += weights @ (cache @ a_vo[s])
    return {"Input Shape": X, "Latent Query": latent_query, "Latent KV Cache": cache,
            "Absorbed QK Kernel": a_qk, "Absorbed VO Kernel": a_vo, "Final Output Shape": total}


def notebook_linear_unabsorbed(X, W_dQ, W_dKV, W_uQ, W_uK, W_uV, W_O, C_KV, h):
    """The same softmax-free computation without absorption: per head s,
    q = (x W_dQ) U_Q(s), k_t = c_t U_K(s), v_t = c_t U_V(s);
    out_s = sum_t (q . k_t) v_t O(s); summed over heads."""
    X = _f64(X)
    uQ, O_blocks = notebook_head_blocks(W_uQ, W_O, h)
    uK, _ = notebook_head_blocks(W_uK, W_O, h)
    uV, _ = notebook_head_blocks(W_uV, W_O, h)
    cache = np.vstack([_f64(C_KV), X @ _f64(W_dKV)])
    c_q = (X @ _f64(W_dQ))[0]
    total = np.zeros(O_blocks[0].shape[1])
    for s in range(h):
        q = c_q @ uQ[s]
        for t in range(cache.shape[0]):
            k_t, v_t = cache[t] @ uK[s], cache[t] @ uV[s]
            total += float(q @ k_t) * (v_t @ O_blocks[s])
    return total[None, :]


def notebook_softmax_unabsorbed(X, W_dQ, W_dKV, W_uQ, W_uK, W_uV, W_O, C_KV, h, scale):
    """The notebook's workload with softmax attention, computed unabsorbed.

    Per head s: q = x W_dQ U_Q(s), k_t = c_t U_K(s), v_t = c_t U_V(s) over the
    cache with the new token appended (it attends to itself); the softmax
    uses `scale`. Returns (v [h, d_h], final [d_model] = sum_s v_s O(s)).
    """
    X = _f64(X)
    uQ, O_blocks = notebook_head_blocks(W_uQ, W_O, h)
    uK, _ = notebook_head_blocks(W_uK, W_O, h)
    uV, _ = notebook_head_blocks(W_uV, W_O, h)
    cache = np.vstack([_f64(C_KV), X @ _f64(W_dKV)])
    c_q = (X @ _f64(W_dQ))[0]
    v = np.zeros((h, uV[0].shape[1]))
    final = np.zeros(O_blocks[0].shape[1])
    for s in range(h):
        v[s], _ = attend_one_head(c_q @ uQ[s], cache @ uK[s], cache @ uV[s], scale, cache.shape[0])
        final += v[s] @ O_blocks[s]
    return v, final


# --------------------------------------------------------------------------
# gated MLA ([gated]) -- a different variant; used here to pin the
# single-position behaviour with the page's worked example
# --------------------------------------------------------------------------
def gated_mla(x, W_q, W_c, W_k, W_v, W_g, W_o, num_heads, causal):
    """Gated multi-head latent attention as the tensortonic page states it.

    Q = X W_q^T, C = X W_c^T, K = C W_k^T, V = C W_v^T; per head
    A = softmax(Q K^T / sqrt(D_h) + M) with M masking later positions when
    causal; heads concatenated to O~; Y = [sigmoid(X W_g^T) * O~] W_o^T.
    Returns dict(output [B,S,D], latent_cache [B,S,L]); inputs not modified.
    """
    x = _f64(x)
    B, S, D = x.shape
    Hn = int(num_heads)
    Dh = D // Hn
    Q = x @ _f64(W_q).T
    C = x @ _f64(W_c).T
    K = C @ _f64(W_k).T
    V = C @ _f64(W_v).T
    Ot = np.zeros((B, S, D))
    for b in range(B):
        for hh in range(Hn):
            sl = slice(hh * Dh, (hh + 1) * Dh)
            for i in range(S):
                n = i + 1 if causal else S
                o, _ = attend_one_head(Q[b, i, sl], K[b, :, sl], V[b, :, sl], 1.0 / math.sqrt(Dh), n)
                Ot[b, i, sl] = o
    gate = 1.0 / (1.0 + np.exp(-(x @ _f64(W_g).T)))
    Y = (gate * Ot) @ _f64(W_o).T
    return {"output": Y, "latent_cache": C}


# --------------------------------------------------------------------------
# the step before the path: the new token's latent row ([tutorial] training
# form c_i = x_i W_c and k_i's rope half x_i W_kr R_i, taken from x and not
# from c; [ferrox] module doc: the cached latent is RMS-normed and the rope
# key roped; [notebook] update-cache step: the new row is appended before the
# query attends, so the token sees itself)
# --------------------------------------------------------------------------
def rms_norm(z, eps, gain=None):
    """Root-mean-square normalisation over the last axis: z / sqrt(mean(z^2) + eps),
    times `gain` when given. Pinned by: unit RMS of the result, invariance
    under scaling z, brute-force sums."""
    z = _f64(z)
    r = z / np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)
    return r if gain is None else r * _f64(gain)


def rope(x, positions, base):
    """Rotary position rotation of the last axis in interleaved pairs.

    Pair i = (x[2i], x[2i+1]) turns by the angle p * base^(-2i/d) at position
    p (the tutorial's R_i: a position-dependent rotation of the rope part).
    positions broadcast against x's leading axes. Pinned by: identity at
    position 0, norm of every pair kept, R(m) R(n) = R(m + n), dot products of
    two rotated vectors depending only on the position difference, and
    hand-computed quarter turns."""
    x = _f64(x)
    d = x.shape[-1]
    if d == 0:
        return x.copy()
    assert d % 2 == 0, "rope width must be even"
    i = np.arange(d // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * theta
    while ang.ndim < x.ndim:
        ang = np.expand_dims(ang, -2)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def latent_cache_rows(x, w_c, w_kr, positions, eps, base, gain=None):
    """Cache rows of new tokens: [RMSNorm(W_c x) | RoPE(W_kr x, pos)].

    x [N, d_model]; w_c [d_c, d_model] (c = W_c x, the tutorial's x W_c with
    its matrix stored output-major); w_kr [d_r, d_model]; positions [N].
    Returns rows [N, d_c + d_r]. Pinned by: brute-force sums of the two
    projections, the rms_norm and rope pins, and the rope half depending on x
    only through W_kr (not on c)."""
    x = _f64(x)
    c = rms_norm(x @ _f64(w_c).T, eps, gain)
    k_pe = rope(x @ _f64(w_kr).T, positions, base)
    return np.concatenate([c, k_pe], axis=1)


def append_rows(cache, rows, seq_ids, positions, block_table=None):
    """A copy of `cache` with row n written at sequence seq_ids[n], position
    positions[n]: dense cache [B, S, W] at [seq, pos]; paged pool
    [P, page, W] at page block_table[seq, pos // page], slot pos % page.
    Every other element is unchanged. Pinned by: rows tagged with their own
    (sequence, position) read back from where the block table says."""
    out = np.array(cache, copy=True)
    for n, (b, p) in enumerate(zip(seq_ids, positions)):
        if block_table is None:
            out[b, p] = rows[n]
        else:
            ps = out.shape[1]
            out[block_table[b, p // ps], p % ps] = rows[n]
    return out


# --------------------------------------------------------------------------
# standard per-head attention over expanded keys and values (the unabsorbed
# prefill form: [tutorial] training form, k and v built per head from c;
# [ferrox] test's naive branch)
# --------------------------------------------------------------------------
def mha_attention(q, k, v, scale, causal, rows=None):
    """q [S_q, H, d_k], k [S_kv, H, d_k], v [S_kv, H, d_v]. Query i sees keys
    t <= i + S_kv - S_q when causal (bottom-right alignment), else all.
    Returns (out [len(rows), H, d_v], lse [len(rows), H]). Pinned by:
    brute-force loops, and equality with the latent form when k, v are the
    MLA expansion of a latent cache."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S_q, H = q.shape[0], q.shape[1]
    S_kv = k.shape[0]
    rows = list(range(S_q) if rows is None else rows)
    out = np.zeros((len(rows), H, v.shape[2]))
    lse = np.full((len(rows), H), -math.inf)
    for r, i in enumerate(rows):
        n = causal_visible(i, S_q, S_kv) if causal else S_kv
        for h in range(H):
            out[r, h], lse[r, h] = attend_one_head(q[i, h], k[:, h], v[:, h], scale, n)
    return out, lse


# --------------------------------------------------------------------------
# full absorption ([notebook] matrix absorption and head sum; [tutorial]
# inference form c' W_qc W_kc^T)
# --------------------------------------------------------------------------
def full_absorbed_weights(w_uq, w_uk, w_uv, w_o):
    """Absorbed weights of the query and output sides.

    Per head: q_nope[h] = W_UQ[h] c' (W_UQ [H, d_nope, d_cq]), k_nope = W_UK[h] c
    (W_UK [H, d_nope, d_c]), v = W_UV[h] c (W_UV [H, d_v, d_c]), and the layer
    output sums W_O[:, h block] v[h] over heads (W_O [d_model, H d_v], head h
    in columns h d_v .. (h+1) d_v - 1). Absorbing the query side gives
        a_qk[h] = W_UK[h]^T W_UQ[h]            [d_c, d_cq]: q_abs[h] = a_qk[h] c'
    (the notebook's W_aQK = W_uQ W_uK^T, transposed), and the output side
        a_vo[:, h d_c .. (h+1) d_c] = W_O[:, h block] W_UV[h]    [d_model, H d_c]
    (the notebook's W_aVO = W_uV W_O per head, transposed), so that
    final = a_vo . concat_h(out_lat[h]) performs the head sum. Pinned by:
    equality with the training form and the notebook's printed shapes."""
    w_uq, w_uk, w_uv, w_o = _f64(w_uq), _f64(w_uk), _f64(w_uv), _f64(w_o)
    H, d_v = w_uv.shape[0], w_uv.shape[1]
    a_qk = np.stack([w_uk[h].T @ w_uq[h] for h in range(H)])
    a_vo = np.concatenate([w_o[:, h * d_v:(h + 1) * d_v] @ w_uv[h] for h in range(H)], axis=1)
    return a_qk, a_vo


def full_absorbed_decode(c_q, q_pe, latent, d_c, a_qk, a_vo, scale, n_visible):
    """One token through the fully absorbed layer: q_abs[h] = a_qk[h] c',
    latent attention with [q_abs | q_pe] over the cache, then
    final = a_vo . concat_h(out_lat[h]). Returns (final [d_model], out_lat [H, d_c])."""
    c_q, a_qk = _f64(c_q), _f64(a_qk)
    H = a_qk.shape[0]
    q_abs = np.stack([a_qk[h] @ c_q for h in range(H)])
    q = q_abs if q_pe is None else np.concatenate([q_abs, _f64(q_pe)], axis=1)
    out_lat, _ = latent_attention(q, latent, d_c, scale, n_visible)
    return _f64(a_vo) @ out_lat.reshape(-1), out_lat


def training_form_decode(c_q, q_pe, latent, d_c, w_uq, w_uk, w_uv, w_o, scale, n_visible):
    """The same token in the training form: per head q = [W_UQ[h] c' | q_pe[h]],
    keys [W_UK[h] c_t | k_pe_t], values W_UV[h] c_t, softmax attention, then
    final = sum_h W_O[:, h block] v[h]."""
    q_nope = np.einsum("hij,j->hi", _f64(w_uq), _f64(c_q))
    H = q_nope.shape[0]
    qp = np.zeros((H, 0)) if q_pe is None else _f64(q_pe)
    v, _ = mla_unabsorbed(q_nope, qp, latent, d_c, w_uk, w_uv, scale, n_visible)
    d_v = v.shape[1]
    w_o = _f64(w_o)
    return sum(w_o[:, h * d_v:(h + 1) * d_v] @ v[h] for h in range(H))
