"""Pins of the oracle functions for the steps around the core path: the new
token's cache row (RMS norm, rotary rotation, placement in the paged cache),
standard attention over per-head expanded keys and values (the unabsorbed
prefill), and the fully absorbed query/output weights. Each pin ties a
function to a closed form, brute-force sums or an identity, so that a dropped
term, a wrong sign, index or transpose fails one of them."""
import math

import numpy as np

import oracle as O
from test_oracle_pins import bf_attend


def fsum_matvec(W, x):
    return np.array([math.fsum(W[i, j] * x[j] for j in range(W.shape[1])) for i in range(W.shape[0])])


# ----------------------------------------------------------------------------
# RMS norm
# ----------------------------------------------------------------------------
def test_rms_norm_closed_forms():
    rng = np.random.default_rng(20)
    z = rng.standard_normal((5, 12))
    r = O.rms_norm(z, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, axis=1)), 1.0, rtol=1e-14)   # unit RMS
    np.testing.assert_allclose(O.rms_norm(7.5 * z, 0.0), r, rtol=1e-13)              # scale invariant
    # a row of equal values c normalises to sign(c) everywhere; with eps the
    # factor is |c| / sqrt(c^2 + eps)
    np.testing.assert_allclose(O.rms_norm(np.full((1, 4), -3.0), 0.0), -1.0, rtol=1e-15)
    np.testing.assert_allclose(O.rms_norm(np.full((1, 4), 2.0), 5.0), 2.0 / 3.0, rtol=1e-15)
    g = rng.standard_normal(12)
    np.testing.assert_allclose(O.rms_norm(z, 1e-6, g), O.rms_norm(z, 1e-6) * g, rtol=1e-14)
    # brute force: exact sums
    for row in z:
        ms = math.fsum(v * v for v in row) / len(row)
        want = [v / math.sqrt(ms + 1e-6) for v in row]
        np.testing.assert_allclose(O.rms_norm(row[None], 1e-6)[0], want, rtol=1e-14)


# ----------------------------------------------------------------------------
# rotary rotation
# ----------------------------------------------------------------------------
def test_rope_quarter_turns_and_identity():
    x = np.array([0.3, -1.7])
    np.testing.assert_array_equal(O.rope(x, 0, 10000.0), x)                 # position 0: identity
    # d = 2: one pair, frequency 1: a quarter turn at p = pi/2 maps (a, b) to (-b, a)
    np.testing.assert_allclose(O.rope(x, math.pi / 2, 10000.0), [1.7, 0.3], atol=1e-15)
    np.testing.assert_allclose(O.rope(x, math.pi, 10000.0), [-0.3, 1.7], atol=1e-15)
    # d = 4, base 10^4: pair 1 turns at base^(-2/4) = 1/100 per position, so
    # p = 50 pi is a quarter turn of pair 1 and 25 whole turns of pair 0
    y = np.array([1.0, 2.0, 3.0, 4.0])
    np.testing.assert_allclose(O.rope(y, 50 * math.pi, 10000.0), [1.0, 2.0, -4.0, 3.0], atol=1e-12)
    # pairs are (0,1), (2,3): a non-interleaved (half-split) layout would move x[1] into pair 1
    z = np.array([0.0, 1.0, 0.0, 0.0])
    np.testing.assert_allclose(O.rope(z, math.pi / 2, 10000.0)[2:], [0.0, 0.0], atol=1e-15)


def test_rope_group_and_relative_properties():
    rng = np.random.default_rng(21)
    d, base = 16, 10000.0
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(3, 11), (0, 7), (1000, 1)]:
        # rotations compose: R(n) R(m) = R(m + n)
        np.testing.assert_allclose(O.rope(O.rope(q, m, base), n, base), O.rope(q, m + n, base), atol=1e-12)
        # pair norms are kept
        a = O.rope(q, m, base)
        np.testing.assert_allclose(a[0::2] ** 2 + a[1::2] ** 2, q[0::2] ** 2 + q[1::2] ** 2, rtol=1e-12)
        # the score of two rotated vectors depends on the position difference only
        s1 = O.rope(q, m, base) @ O.rope(k, n, base)
        s2 = O.rope(q, m + 37, base) @ O.rope(k, n + 37, base)
        assert abs(s1 - s2) < 1e-11
    # per-row positions broadcast over a head axis
    x = rng.standard_normal((3, 2, d))
    pos = np.array([0, 5, 9])
    got = O.rope(x, pos[:, None], base)
    for i in range(3):
        for h in range(2):
            np.testing.assert_array_equal(got[i, h], O.rope(x[i, h], pos[i], base))


# ----------------------------------------------------------------------------
# the new token's cache row and its placement
# ----------------------------------------------------------------------------
def test_latent_cache_rows_parts():
    rng = np.random.default_rng(22)
    N, d_model, d_c, d_r = 3, 9, 6, 4
    x = rng.standard_normal((N, d_model))
    w_c, w_kr = rng.standard_normal((d_c, d_model)), rng.standard_normal((d_r, d_model))
    pos = np.array([0, 4, 13])
    rows = O.latent_cache_rows(x, w_c, w_kr, pos, 1e-6, 10000.0)
    assert rows.shape == (N, d_c + d_r)
    for n in range(N):
        c = fsum_matvec(w_c, x[n])                   # W_c x by exact sums
        kr = fsum_matvec(w_kr, x[n])
        np.testing.assert_allclose(rows[n, :d_c], O.rms_norm(c[None], 1e-6)[0], rtol=1e-13)
        np.testing.assert_allclose(rows[n, d_c:], O.rope(kr, pos[n], 10000.0), rtol=1e-12, atol=1e-14)
    # the rope half comes from x, not from c: changing W_c leaves it alone
    rows2 = O.latent_cache_rows(x, 2 * w_c + 1, w_kr, pos, 1e-6, 10000.0)
    np.testing.assert_array_equal(rows2[:, d_c:], rows[:, d_c:])
    # a gain scales the latent half only (a gain of 2 doubles it exactly)
    rows_g = O.latent_cache_rows(x, w_c, w_kr, pos, 1e-6, 10000.0, gain=np.full(d_c, 2.0))
    np.testing.assert_array_equal(rows_g[:, :d_c], 2.0 * rows[:, :d_c])
    np.testing.assert_array_equal(rows_g[:, d_c:], rows[:, d_c:])
    # position 0's rope half is the plain projection
    np.testing.assert_allclose(rows[0, d_c:], fsum_matvec(w_kr, x[0]), rtol=1e-13)


def test_append_rows_placement():
    B, ps, W, P = 2, 4, 3, 5
    table = np.array([[3, 0, -1], [4, 1, 2]])
    pool = np.full((P, ps, W), -1.0)
    seq = [0, 1, 1, 0]
    pos = [5, 0, 9, 2]
    rows = np.array([[100 * b + p] * W for b, p in zip(seq, pos)], dtype=np.float64)  # tagged
    out = O.append_rows(pool, rows, seq, pos, table)
    assert out[0, 1, 0] == 5          # seq 0, pos 5: logical page 1 -> pool page 0, slot 1
    assert out[4, 0, 0] == 100        # seq 1, pos 0: page 4 slot 0
    assert out[2, 1, 0] == 109        # seq 1, pos 9: logical page 2 -> pool page 2, slot 1
    assert out[3, 2, 0] == 2          # seq 0, pos 2: page 3, slot 2
    assert np.count_nonzero(out != pool) == 4 * W   # nothing else written
    assert np.all(pool == -1.0)                     # input not modified
    dense = O.append_rows(np.zeros((B, 10, W)), rows, seq, pos)
    assert dense[1, 9, 0] == 109 and dense[0, 2, 0] == 2 and np.count_nonzero(dense) == 4 * W


# ----------------------------------------------------------------------------
# standard attention over per-head expanded keys and values
# ----------------------------------------------------------------------------
def test_mha_attention_brute_force():
    rng = np.random.default_rng(23)
    S_q, S_kv, H, dk, dv = 3, 5, 2, 4, 3
    q, k, v = rng.standard_normal((S_q, H, dk)), rng.standard_normal((S_kv, H, dk)), rng.standard_normal((S_kv, H, dv))
    for causal in (True, False):
        out, lse = O.mha_attention(q, k, v, 0.6, causal)
        for i in range(S_q):
            n = i + 1 + S_kv - S_q if causal else S_kv
            for h in range(H):
                bo, bl = bf_attend(q[i, h].tolist(), k[:, h].tolist(), v[:, h].tolist(), 0.6, n)
                np.testing.assert_allclose(out[i, h], bo, rtol=1e-12, atol=1e-14)
                assert abs(lse[i, h] - bl) < 1e-12


def test_mha_over_expansion_equals_latent_form():
    """With k = [W_UK c | k_pe], v = W_UV c and q = [q_nope | q_pe], standard
    attention equals the latent form with the absorbed query, up-projected."""
    rng = np.random.default_rng(24)
    S, H, dn, dc, dr, dv = 6, 3, 4, 7, 2, 5
    lat = rng.standard_normal((S, dc + dr))
    wuk, wuv = rng.standard_normal((H, dn, dc)), rng.standard_normal((H, dv, dc))
    qn, qp = rng.standard_normal((S, H, dn)), rng.standard_normal((S, H, dr))
    K, V = O.expand_per_head(lat, dc, wuk, wuv)
    out, lse = O.mha_attention(np.concatenate([qn, qp], axis=2), K, V, 0.4, True)
    qa = O.absorb_query(qn, qp, wuk)
    lo, ll = O.latent_prefill_causal(qa, lat, dc, 0.4)
    np.testing.assert_allclose(out, O.up_project(lo, wuv), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, ll, rtol=1e-12)


# ----------------------------------------------------------------------------
# full absorption
# ----------------------------------------------------------------------------
def test_full_absorption_equals_training_form():
    rng = np.random.default_rng(25)
    H, dn, dcq, dc, dr, dv, dm, T = 3, 4, 6, 5, 2, 3, 7, 9
    wuq, wuk = rng.standard_normal((H, dn, dcq)), rng.standard_normal((H, dn, dc))
    wuv, wo = rng.standard_normal((H, dv, dc)), rng.standard_normal((dm, H * dv))
    lat = rng.standard_normal((T, dc + dr))
    cq, qp = rng.standard_normal(dcq), rng.standard_normal((H, dr))
    a_qk, a_vo = O.full_absorbed_weights(wuq, wuk, wuv, wo)
    assert a_qk.shape == (H, dc, dcq) and a_vo.shape == (dm, H * dc)
    for n in (1, 5, T):
        got, _ = O.full_absorbed_decode(cq, qp, lat, dc, a_qk, a_vo, 0.3, n)
        want = O.training_form_decode(cq, qp, lat, dc, wuq, wuk, wuv, wo, 0.3, n)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)
    # the query side alone: a_qk[h] c' dotted with c equals (W_UQ c') . (W_UK c)
    c = rng.standard_normal(dc)
    for h in range(H):
        lhs = math.fsum((a_qk[h] @ cq) * c)
        rhs = math.fsum(fsum_matvec(wuq[h], cq) * fsum_matvec(wuk[h], c))
        assert abs(lhs - rhs) < 1e-11 * max(1.0, abs(rhs))
    # no rope part (the notebook's RoPE-less case)
    got, _ = O.full_absorbed_decode(cq, None, lat[:, :dc], dc, a_qk, a_vo, 0.3, T)
    want = O.training_form_decode(cq, None, lat[:, :dc], dc, wuq, wuk, wuv, wo, 0.3, T)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_full_absorption_matches_notebook_weights():
    """The notebook's W_aQK [h, d_c', d_c] and W_aVO [h, d_c, d_model] (shapes
    it prints: (3, 20, 20), (3, 20, 100)) are these absorbed weights in
    another orientation: its head blocks map to W_UQ[h] = W_uQ[:, blk]^T and
    W_O[:, blk] = W_O_nb[blk, :]^T."""
    import workloads as G
    d = G.config1_notebook(0)
    H, dh = d.H, d.d_h
    blk = lambda W: np.stack([W[:, s * dh:(s + 1) * dh].T for s in range(H)])   # [H, d_h, d_c]
    a_qk, a_vo = O.full_absorbed_weights(blk(d.W_uQ), blk(d.W_uK), blk(d.W_uV), d.W_O.T)
    nb = O.notebook_linear_absorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O, d.C_KV, H)
    W_aQK, W_aVO = nb["Absorbed QK Kernel"], nb["Absorbed VO Kernel"]
    assert W_aQK.shape == (3, 20, 20) and W_aVO.shape == (3, 20, 100)
    for h in range(H):
        np.testing.assert_allclose(a_qk[h].T, W_aQK[h], rtol=1e-12)
        np.testing.assert_allclose(a_vo[:, h * d.d_c:(h + 1) * d.d_c].T, W_aVO[h], rtol=1e-12)
