"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: a value or
shape printed on a page, an assertion of the ferrox-core unit test, a closed
form, an invariance, or brute-force scalar loops. A plausible slip in the
oracle (dropped rope term, wrong scale, transposed weight, off-by-one causal
offset, wrong lse) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import workloads as G

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# brute force: pure-Python scalar loops with exactly rounded sums
# ----------------------------------------------------------------------------
def bf_attend(q, K, V, scale, n):
    if n <= 0:
        return [0.0] * len(V[0]), -math.inf
    s = [math.fsum(q[d] * K[t][d] for d in range(len(q))) * scale for t in range(n)]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = math.fsum(e)
    out = [math.fsum(e[t] / z * V[t][d] for t in range(n)) for d in range(len(V[0]))]
    return out, m + math.log(z)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_brute_force_latent_attention():
    rng = np.random.default_rng(1)
    H, d_c, d_r, T = 3, 5, 2, 6
    q = _rand(rng, H, d_c + d_r)
    lat = _rand(rng, T, d_c + d_r)
    for n in (0, 1, 4, 6):
        out, lse = O.latent_attention(q, lat, d_c, 0.37, n)
        for h in range(H):
            K = lat.tolist()
            V = lat[:, :d_c].tolist()
            bo, bl = bf_attend(q[h].tolist(), K, V, 0.37, n)
            np.testing.assert_allclose(out[h], bo, rtol=1e-12, atol=1e-14)
            if n == 0:
                assert lse[h] == -math.inf
            else:
                assert abs(lse[h] - bl) < 1e-12


def test_brute_force_causal_prefill_bottom_right():
    rng = np.random.default_rng(2)
    S_q, S_kv, H, d_c, d_r = 3, 5, 2, 4, 2
    q = _rand(rng, S_q, H, d_c + d_r)
    lat = _rand(rng, S_kv, d_c + d_r)
    out, lse = O.latent_prefill_causal(q, lat, d_c, 0.5)
    for i in range(S_q):
        n = i + 1 + (S_kv - S_q)  # query i sees t <= i + S_kv - S_q
        for h in range(H):
            bo, bl = bf_attend(q[i, h].tolist(), lat.tolist(), lat[:, :d_c].tolist(), 0.5, n)
            np.testing.assert_allclose(out[i, h], bo, rtol=1e-12, atol=1e-14)
            assert abs(lse[i, h] - bl) < 1e-12
    # more queries than cache rows: the first S_q - S_kv queries see nothing
    q2 = _rand(rng, 4, 1, d_c + d_r)
    out2, lse2 = O.latent_prefill_causal(q2, lat[:2], d_c, 0.5)
    assert np.all(out2[:2] == 0) and np.all(np.isneginf(lse2[:2]))
    bo, _ = bf_attend(q2[3, 0].tolist(), lat[:2].tolist(), lat[:2, :d_c].tolist(), 0.5, 2)
    np.testing.assert_allclose(out2[3, 0], bo, rtol=1e-12)


def test_brute_force_absorb_and_up_project():
    rng = np.random.default_rng(3)
    N, H, dn, dc, dr, dv = 2, 3, 4, 5, 2, 3
    qn, qp = _rand(rng, N, H, dn), _rand(rng, N, H, dr)
    wuk, wuv = _rand(rng, H, dn, dc), _rand(rng, H, dv, dc)
    q = O.absorb_query(qn, qp, wuk)
    lat = _rand(rng, N, H, dc)
    v = O.up_project(lat, wuv)
    for n in range(N):
        for h in range(H):
            for j in range(dc):
                assert abs(q[n, h, j] - math.fsum(wuk[h, i, j] * qn[n, h, i] for i in range(dn))) < 1e-12
            np.testing.assert_array_equal(q[n, h, dc:], qp[n, h])
            for i in range(dv):
                assert abs(v[n, h, i] - math.fsum(wuv[h, i, j] * lat[n, h, j] for j in range(dc))) < 1e-12


# ----------------------------------------------------------------------------
# the lab's identity and the ferrox-core unit test
# ----------------------------------------------------------------------------
def test_lab_identity_orientation():
    """q^T W_UK c = (W_UK^T q)^T c: absorb_query must produce W_UK^T q_nope."""
    rng = np.random.default_rng(4)
    H, dn, dc = 4, 8, 16
    qn, w, c = _rand(rng, H, dn), _rand(rng, H, dn, dc), _rand(rng, dc)
    qa = O.absorb_query(qn, None, w)
    for h in range(H):
        k_nope = [math.fsum(w[h, i, j] * c[j] for j in range(dc)) for i in range(dn)]  # W_UK c
        lhs = math.fsum(qn[h, i] * k_nope[i] for i in range(dn))
        rhs = float(qa[h] @ c)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def _ferrox_chain(case, scale):
    qa = O.absorb_query(case.q_nope, case.q_pe, case.w_uk)
    out_lat, lse = O.latent_attention(qa, case.latent, case.d_c, scale, case.seq)
    return O.up_project(out_lat, case.w_uv), out_lat


def test_ferrox_absorbed_equals_unabsorbed(golden_dir):
    g = _load(golden_dir, "ferrox_test.json")
    case = G.p2_tiny_case()
    assert (case.H, case.d_nope, case.d_r, case.d_v, case.d_c, case.seq) == (
        g["n_heads"], g["nope"], g["rope"], g["v_dim"], g["kv_lora"], g["seq"])
    scale = 1.0 / math.sqrt(case.d_nope + case.d_r)
    naive, _ = O.mla_unabsorbed(case.q_nope, case.q_pe, case.latent, case.d_c,
                                case.w_uk, case.w_uv, scale, case.seq)
    absorbed, _ = _ferrox_chain(case, scale)
    # the page's tolerance (f32), and far tighter in f64
    assert np.max(np.abs(naive - absorbed)) < g["absorbed_vs_naive_abs_tol"]
    assert np.max(np.abs(naive - absorbed)) < 1e-13
    # inputs really are the page's stream: values in [-0.5, 0.5), not constant
    assert case.kv_b.min() >= -0.5 and case.kv_b.max() < 0.5 and np.std(case.latent) > 0.1


def test_ferrox_wrong_scale_is_detectable(golden_dir):
    g = _load(golden_dir, "ferrox_test.json")
    case = G.p2_tiny_case()
    right = 1.0 / math.sqrt(case.d_nope + case.d_r)
    wrong = 1.0 / math.sqrt(case.d_c + case.d_r)
    _, lat_r = _ferrox_chain(case, right)
    _, lat_w = _ferrox_chain(case, wrong)
    assert np.max(np.abs(lat_r - lat_w)) > g["wrong_scale_min_abs_change"]


def test_xorshift_stream_definition():
    # first outputs of xorshift32 from 0x9E37, computed by hand with the shifts 13, 17, 5
    s = 0x9E37
    vals = []
    for _ in range(3):
        s ^= (s << 13) & 0xFFFFFFFF
        s ^= s >> 17
        s ^= (s << 5) & 0xFFFFFFFF
        vals.append(np.float32(np.float32(s) / np.float32(4294967295.0) - np.float32(0.5)))
    g = G.xorshift32_stream(0x9E37)
    assert [next(g) for _ in range(3)] == vals


# ----------------------------------------------------------------------------
# the notebook (config 1)
# ----------------------------------------------------------------------------
def test_notebook_printed_shapes(golden_dir):
    g = _load(golden_dir, "notebook_shapes.json")
    d = G.config1_notebook(0)
    res = O.notebook_linear_absorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O, d.C_KV, d.H)
    for k, shp in g["shapes"].items():
        assert list(res[k].shape) == shp, k


def test_notebook_linear_absorption_is_associativity():
    d = G.config1_notebook(0)
    a = O.notebook_linear_absorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O, d.C_KV,
                                   d.H)["Final Output Shape"]
    u = O.notebook_linear_unabsorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O, d.C_KV, d.H)
    assert np.max(np.abs(a - u)) <= 1e-10 * np.max(np.abs(u))


def test_notebook_head_blocks_are_head_major():
    """The notebook splits the up-projection columns head-major (reshape to
    (d_c, h, d_h), heads to the front): head s owns columns s*d_h .. s*d_h+d_h-1,
    and the output projection's rows likewise. Entries tagged with their own
    column (row) index must land in their head's block, in order; a d_h-major
    split (column j -> head j % h) puts them elsewhere."""
    d_c, h, d_h, d_model = 4, 3, 5, 7
    cols = np.tile(np.arange(h * d_h, dtype=np.float64), (d_c, 1))          # W[i, j] = j
    rows = np.tile(np.arange(h * d_h, dtype=np.float64)[:, None], (1, d_model))  # W_O[i, j] = i
    ups, outs = O.notebook_head_blocks(cols, rows, h)
    assert len(ups) == h and len(outs) == h
    for s in range(h):
        want = np.arange(s * d_h, (s + 1) * d_h, dtype=np.float64)
        assert ups[s].shape == (d_c, d_h) and outs[s].shape == (d_h, d_model)
        assert np.all(ups[s] == want[None, :]) and np.all(outs[s] == want[:, None])
    # the notebook's own reshape/transpose of a tagged matrix gives the same blocks
    nb = cols.reshape(d_c, h, d_h).transpose(1, 0, 2)
    for s in range(h):
        np.testing.assert_array_equal(ups[s], nb[s])


def test_notebook_head_split_decides_the_softmax_workload():
    """With a d_h-major split the softmax workload changes: the result is
    sensitive to the split (so the pin above is the one that fixes it)."""
    d = G.config1_notebook(0)
    scale = 1.0 / math.sqrt(d.d_h)
    v, final = O.notebook_softmax_unabsorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV, d.W_O,
                                             d.C_KV, d.H, scale)
    perm = np.arange(d.H * d.d_h).reshape(d.d_h, d.H).T.reshape(-1)    # column j -> head j % h
    v2, final2 = O.notebook_softmax_unabsorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ[:, perm], d.W_uK[:, perm],
                                               d.W_uV[:, perm], d.W_O[perm], d.C_KV, d.H, scale)
    assert np.max(np.abs(final - final2)) > 1e-3 * np.max(np.abs(final))


def _config1_path_inputs(d):
    """Config 1 expressed in the path's layouts (host-side preparation; the
    head blocks are sliced here directly, not through the oracle)."""
    H, dh = d.H, d.d_h
    blk = lambda W: np.stack([W[:, s * dh:(s + 1) * dh] for s in range(H)])   # head-major column blocks
    cache = np.vstack([d.C_KV, d.X @ d.W_dKV])            # 6 rows, d_r = 0
    q_nope = np.einsum("i,hij->hj", (d.X @ d.W_dQ)[0], blk(d.W_uQ))      # [H, d_h]
    w_uk = blk(d.W_uK).transpose(0, 2, 1)                  # [H, d_h, d_c]
    w_uv = blk(d.W_uV).transpose(0, 2, 1)                  # [H, d_h, d_c]
    Ow = np.stack([d.W_O[s * dh:(s + 1) * dh] for s in range(H)])          # [H, d_h, d_model]
    return cache, q_nope, w_uk, w_uv, Ow


def test_config1_absorbed_equals_unabsorbed_f64():
    d = G.config1_notebook(0)
    scale = 1.0 / math.sqrt(d.d_h)
    v_ref, final_ref = O.notebook_softmax_unabsorbed(d.X, d.W_dQ, d.W_dKV, d.W_uQ, d.W_uK, d.W_uV,
                                                     d.W_O, d.C_KV, d.H, scale)
    cache, q_nope, w_uk, w_uv, Ow = _config1_path_inputs(d)
    qa = O.absorb_query(q_nope, np.zeros((d.H, 0)), w_uk)
    lat, _ = O.latent_attention(qa, cache, d.d_c, scale, cache.shape[0])
    v = O.up_project(lat, w_uv)
    final = np.einsum("hi,hio->o", v, Ow)
    assert np.max(np.abs(v - v_ref)) <= 1e-10 * np.max(np.abs(v_ref))
    assert np.max(np.abs(final - final_ref)) <= 1e-10 * np.max(np.abs(final_ref))


# ----------------------------------------------------------------------------
# the gated-MLA page's worked example (single position => softmax weight 1)
# ----------------------------------------------------------------------------
def test_gated_worked_example(golden_dir):
    g = _load(golden_dir, "gated_example.json")["numeric_example"]
    res = O.gated_mla(np.array(g["hidden_states"]), np.array(g["query_projection"]),
                      np.array(g["latent_down_projection"]), np.array(g["key_up_projection"]),
                      np.array(g["value_up_projection"]), np.array(g["output_gate_projection"]),
                      np.array(g["output_projection"]), g["num_heads"], g["causal"])
    assert res["output"].tolist() == g["expected_output"]
    assert res["latent_cache"].tolist() == g["expected_latent_cache"]


def test_gated_shape_examples(golden_dir):
    rng = np.random.default_rng(5)
    for ex in _load(golden_dir, "gated_example.json")["shape_examples"]:
        B, S, D = ex["hidden_shape"]
        L = ex["latent_width"]
        x = rng.standard_normal((B, S, D))
        x0 = x.copy()
        res = O.gated_mla(x, rng.standard_normal((D, D)), rng.standard_normal((L, D)),
                          rng.standard_normal((D, L)), rng.standard_normal((D, L)),
                          rng.standard_normal((D, D)), rng.standard_normal((D, D)),
                          ex["num_heads"], ex["causal"])
        assert list(res["output"].shape) == ex["output_shape"]
        assert list(res["latent_cache"].shape) == ex["latent_cache_shape"]
        np.testing.assert_array_equal(x, x0)  # inputs not mutated


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _gated_two_positions(causal):
    """Two positions, D = 4, one head (D_h = 4, scale 1/2), latent width 1.
    W_q = I, so Q_i = x_i; W_c picks channel 0, so C_j = x_j[0]; W_k = ones
    (K_j = C_j (1,1,1,1)); W_v picks the latent into channel 0 (V_j = (C_j, 0,
    0, 0)); gate weights 0 (sigmoid 1/2); W_o = I.
    x_0 = (1,0,0,0), x_1 = (2,1,0,1): C = (1, 2); logit(i, j) = sum(x_i) C_j / 2.
    Row 1 sees both positions: logits (2, 4); context = 1 + sigmoid(4 - 2).
    Row 0: causal sees only position 0 (context 1); non-causal logits (1/2, 1),
    context 1 + sigmoid(1/2). Output = context / 2 in channel 0."""
    x = np.array([[[1.0, 0, 0, 0], [2.0, 1, 0, 1]]])
    W_q, W_o = np.eye(4), np.eye(4)
    W_c = np.array([[1.0, 0, 0, 0]])
    W_k = np.ones((4, 1))
    W_v = np.array([[1.0], [0], [0], [0]])
    W_g = np.zeros((4, 4))
    res = O.gated_mla(x, W_q, W_c, W_k, W_v, W_g, W_o, 1, causal)
    want = np.zeros((1, 2, 4))
    want[0, 0, 0] = 0.5 * (1.0 if causal else 1.0 + _sig(0.5))
    want[0, 1, 0] = 0.5 * (1.0 + _sig(2.0))
    return res, want


def test_gated_two_positions_causal():
    res, want = _gated_two_positions(True)
    np.testing.assert_allclose(res["output"], want, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(res["latent_cache"], [[[1.0], [2.0]]])


def test_gated_two_positions_non_causal():
    res, want = _gated_two_positions(False)
    np.testing.assert_allclose(res["output"], want, rtol=1e-14, atol=1e-15)


def test_gated_heads_are_channel_blocks():
    """Two heads of width 2 (scale 1/sqrt 2) own channels {0,1} and {2,3}.
    W_q = I, C_j = x_j[0], K_j = C_j (1, 0, 0, 3), V_j = C_j (1, 1, 1, 1),
    gate 1/2, W_o = I; x_0 = (1,0,0,0), x_1 = (2,0,0,1): C = (1, 2).
    Causal row 1: head 0 logits 2 C / sqrt 2 -> context 1 + sigmoid(sqrt 2) in
    channels 0, 1; head 1 logits 3 C / sqrt 2 -> 1 + sigmoid(3 / sqrt 2) in
    channels 2, 3 (an interleaved head split mixes them)."""
    x = np.array([[[1.0, 0, 0, 0], [2.0, 0, 0, 1]]])
    W_c = np.array([[1.0, 0, 0, 0]])
    W_k = np.array([[1.0], [0], [0], [3.0]])
    W_v = np.ones((4, 1))
    res = O.gated_mla(x, np.eye(4), W_c, W_k, W_v, np.zeros((4, 4)), np.eye(4), 2, True)
    a, b = 0.5 * (1 + _sig(math.sqrt(2.0))), 0.5 * (1 + _sig(3 / math.sqrt(2.0)))
    np.testing.assert_allclose(res["output"][0, 1], [a, a, b, b], rtol=1e-14)
    np.testing.assert_allclose(res["output"][0, 0], [0.5] * 4, rtol=1e-14)


def test_single_position_returns_latent_row():
    rng = np.random.default_rng(6)
    q = _rand(rng, 4, 9)
    lat = _rand(rng, 3, 9)
    out, lse = O.latent_attention(q, lat, 7, 0.3, 1)
    for h in range(4):
        assert np.array_equal(out[h], lat[0, :7])
        assert abs(lse[h] - float(q[h] @ lat[0]) * 0.3) < 1e-14
    # causal prefill row 0 (S_q == S_kv) sees only position 0
    outp, _ = O.latent_prefill_causal(rng.standard_normal((3, 2, 9)), lat, 7, 0.3, rows=[0])
    assert np.array_equal(outp[0, 0], lat[0, :7]) and np.array_equal(outp[0, 1], lat[0, :7])


# ----------------------------------------------------------------------------
# closed forms and invariances
# ----------------------------------------------------------------------------
def test_two_position_closed_form():
    rng = np.random.default_rng(7)
    q, lat = _rand(rng, 1, 6), _rand(rng, 2, 6)
    scale = 0.8
    s0, s1 = float(q[0] @ lat[0]) * scale, float(q[0] @ lat[1]) * scale
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out, lse = O.latent_attention(q, lat, 4, scale, 2)
    np.testing.assert_allclose(out[0], p0 * lat[0, :4] + (1 - p0) * lat[1, :4], rtol=1e-13)
    assert abs(lse[0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-13


def test_zero_query_gives_mean():
    rng = np.random.default_rng(8)
    lat = _rand(rng, 11, 10)
    out, lse = O.latent_attention(np.zeros((2, 10)), lat, 8, 0.1, 9)
    np.testing.assert_allclose(out[0], lat[:9, :8].mean(axis=0), rtol=1e-13, atol=1e-15)
    assert abs(lse[0] - math.log(9)) < 1e-14


def test_identical_heads_and_shift_invariance():
    rng = np.random.default_rng(9)
    d_c, d_r, T = 6, 2, 10
    lat = _rand(rng, T, d_c + d_r)
    lat[:, d_c] = 1.0            # one rope coordinate constant over positions
    q = np.repeat(_rand(rng, 1, d_c + d_r), 3, axis=0)
    q[2, d_c] += 5.0             # shifts every logit of head 2 by 5 * scale
    out, lse = O.latent_attention(q, lat, d_c, 0.7, T)
    np.testing.assert_array_equal(out[0], out[1])
    np.testing.assert_allclose(out[2], out[0], rtol=1e-12, atol=1e-14)
    assert abs((lse[2] - lse[0]) - 5.0 * 0.7) < 1e-12


def test_permutation_invariance():
    rng = np.random.default_rng(10)
    lat = _rand(rng, 13, 9)
    q = _rand(rng, 2, 9)
    perm = rng.permutation(13)
    a, la = O.latent_attention(q, lat, 7, 0.4, 13)
    b, lb = O.latent_attention(q, lat[perm], 7, 0.4, 13)
    np.testing.assert_allclose(a, b, rtol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_value_side_associativity():
    rng = np.random.default_rng(11)
    H, d_c, d_r, d_v, T = 3, 8, 2, 5, 12
    q, lat, w = _rand(rng, H, d_c + d_r), _rand(rng, T, d_c + d_r), _rand(rng, H, d_v, d_c)
    lat_out, _ = O.latent_attention(q, lat, d_c, 0.3, T)
    v_expanded, _ = O.latent_attention_expanded_v(q, lat, d_c, w, 0.3, T)
    np.testing.assert_allclose(O.up_project(lat_out, w), v_expanded, rtol=1e-11, atol=1e-13)


def test_lse_merge_equals_whole_range():
    rng = np.random.default_rng(12)
    H, d_c, T = 4, 5, 17
    q, lat = _rand(rng, H, d_c + 3), _rand(rng, T, d_c + 3)
    whole, lw = O.latent_attention(q, lat, d_c, 0.6, T)
    cuts = [0, 0, 5, 5, 11, 17]  # includes empty ranges
    outs, lses = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = O.latent_attention(q, lat[a:b], d_c, 0.6, b - a)
        outs.append(o)
        lses.append(l)
    m, lm = O.lse_merge(np.array(outs), np.array(lses))
    np.testing.assert_allclose(m, whole, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, lw, rtol=1e-13)
    # all-empty merge
    z, lz = O.lse_merge(np.zeros((2, H, d_c)), np.full((2, H), -np.inf))
    assert np.all(z == 0) and np.all(np.isneginf(lz))


def test_expand_per_head_layout():
    """k[t,h] = [W_UK[h] c_t | k_pe_t], v[t,h] = W_UV[h] c_t, layout [seq, heads, dim]."""
    rng = np.random.default_rng(13)
    T, H, dn, dc, dr, dv = 3, 2, 4, 5, 2, 3
    lat, wuk, wuv = _rand(rng, T, dc + dr), _rand(rng, H, dn, dc), _rand(rng, H, dv, dc)
    K, V = O.expand_per_head(lat, dc, wuk, wuv)
    assert K.shape == (T, H, dn + dr) and V.shape == (T, H, dv)
    for t in range(T):
        for h in range(H):
            for i in range(dn):
                assert abs(K[t, h, i] - math.fsum(wuk[h, i, j] * lat[t, j] for j in range(dc))) < 1e-12
            np.testing.assert_array_equal(K[t, h, dn:], lat[t, dc:])
            for i in range(dv):
                assert abs(V[t, h, i] - math.fsum(wuv[h, i, j] * lat[t, j] for j in range(dc))) < 1e-12


# ----------------------------------------------------------------------------
# cache accounting
# ----------------------------------------------------------------------------
def test_cache_size_table(golden_dir):
    for r in _load(golden_dir, "cache_table.json")["rows"]:
        assert O.mha_cache_values_per_token(r["L"], r["H"], r["d_head"]) == r["mha"]
        assert O.mla_cache_values_per_token(r["L"], r["d_c"], r["d_r"]) == r["mla"]
        assert abs(O.cache_ratio(r["H"], r["d_head"], r["d_c"], r["d_r"]) - r["ratio"]) < 1e-12
        assert r["mha"] / r["mla"] == pytest.approx(r["ratio"], rel=1e-15)
