"""Pins for the CPU oracle: closed forms, worked examples, invariants and a
pure-Python brute force.  None of these retypes the oracle's own formula; each
is chosen so that a plausible mistake (dropped eps, wrong rotation sign or
pairing, transposed operand, wrong head mapping, wrong scale, norm/RoPE order,
re-rotating cached keys, a broken merge) fails at least one test.
"""

import itertools
import math

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(12345)


def rnd(*shape, scale=1.0):
    return scale * RNG.standard_normal(shape)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_vector_closed_form():
    # x = c * ones: mean(x^2) = c^2, so y_i = gamma_i * c / sqrt(c^2 + eps).
    # c^2 equal to eps makes a dropped or misplaced eps visible.
    d, c, eps = 128, 1e-3, 1e-6
    gamma = np.linspace(0.5, 1.5, d)
    y = O.rms_norm(np.full(d, c), gamma, eps)
    assert np.allclose(y, gamma * (1.0 / math.sqrt(2.0)), rtol=1e-14, atol=0)


def test_rmsnorm_worked_example_small_d():
    # x = (3, 4), eps = 0: mean square 12.5, rms 3.5355..; gamma = (1, 2)
    y = O.rms_norm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    r = 1.0 / math.sqrt(12.5)
    assert np.allclose(y, [3.0 * r, 8.0 * r], rtol=1e-15)
    # the mean is over d, not a sum: sum would give 1/5, not 1/sqrt(12.5)
    assert not np.isclose(y[0], 3.0 / 5.0)


def test_rmsnorm_scale_invariance_and_onehot_gamma():
    x = rnd(4, 128)
    assert np.allclose(O.rms_norm(7.5 * x, np.ones(128), 0.0), O.rms_norm(x, np.ones(128), 0.0), rtol=1e-13)
    g = np.zeros(128)
    g[17] = 1.0
    y = O.rms_norm(x, g, 0.0)
    assert np.all(y[:, np.arange(128) != 17] == 0.0)
    rms = np.sqrt(np.mean(x * x, axis=-1))
    assert np.allclose(y[:, 17], x[:, 17] / rms, rtol=1e-14)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero():
    x = rnd(3, 128)
    assert np.array_equal(O.rope(x, np.zeros(3), 1e6), x)


def test_rope_frequency_table_worked_values():
    # theta^(-2i/d): i = 0 -> 1; d = 128, theta = 1e6, i = 32 -> 1e6^-0.5 = 1e-3;
    # i = 64 would be out of range (only d/2 pairs).
    f = O.rope_frequencies(128, 1e6)
    assert f.shape == (64,)
    assert f[0] == 1.0
    assert math.isclose(f[32], 1e-3, rel_tol=1e-14)
    assert math.isclose(f[16], 1e6 ** -0.25, rel_tol=1e-14)   # 0.0316227..


def test_rope_unit_vector_rotates_into_partner_half():
    # e_32 at position 1000 with theta = 1e6 turns by exactly 1 rad into the
    # partner dimension 32 + 64 = 96 with a positive sine (half-split pairing,
    # counter-clockwise sign).  An interleaved pairing would move it to dim 33.
    x = np.zeros(128)
    x[32] = 1.0
    y = O.rope(x, 1000.0, 1e6)
    exp = np.zeros(128)
    exp[32], exp[96] = math.cos(1.0), math.sin(1.0)
    assert np.allclose(y, exp, atol=1e-15)
    x2 = np.zeros(128)
    x2[96] = 1.0
    y2 = O.rope(x2, 1000.0, 1e6)
    exp2 = np.zeros(128)
    exp2[32], exp2[96] = -math.sin(1.0), math.cos(1.0)
    assert np.allclose(y2, exp2, atol=1e-15)


def test_rope_d4_worked_example():
    # d = 4, theta = 100: f = (1, 0.1); at p = 10 the angles are (10, 1) rad.
    # pairs (x0, x2) = (1, 3) and (x1, x3) = (2, 4).
    y = O.rope(np.array([1.0, 2.0, 3.0, 4.0]), 10.0, 100.0)
    c0, s0, c1, s1 = math.cos(10), math.sin(10), math.cos(1), math.sin(1)
    exp = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    assert np.allclose(y, exp, atol=1e-14)


def test_rope_norm_preserving_composition_and_relative_position():
    x, k = rnd(128), rnd(128)
    y = O.rope(x, 131071.0, 5e5)
    assert math.isclose(np.linalg.norm(y), np.linalg.norm(x), rel_tol=1e-13)
    assert np.allclose(O.rope(O.rope(x, 300.0, 1e6), 77.0, 1e6), O.rope(x, 377.0, 1e6), atol=1e-12)
    # q.k after rotation depends only on the position difference
    d1 = O.rope(x, 1000.0, 1e6) @ O.rope(k, 990.0, 1e6)
    d2 = O.rope(x, 51234.0, 1e6) @ O.rope(k, 51224.0, 1e6)
    assert math.isclose(d1, d2, rel_tol=1e-9, abs_tol=1e-9)


def test_prologue_order_norm_then_rope_worked_example():
    # d = 2, theta > 0 -> f0 = 1; p = 1 rad.  x = (3, 4), gamma = (1, 2), eps = 0.
    # norm then rope: y = (3r, 8r) rotated by 1 rad.  rope-then-norm differs.
    r = 1.0 / math.sqrt(12.5)
    c, s = math.cos(1.0), math.sin(1.0)
    exp = [3 * r * c - 8 * r * s, 8 * r * c + 3 * r * s]
    y = O.prologue(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 1.0, 10.0, 0.0)
    assert np.allclose(y, exp, atol=1e-15)
    wrong = [(3 * c - 4 * s) * r * 1.0, (4 * c + 3 * s) * r * 2.0]
    assert not np.allclose(y, wrong, atol=1e-3)


def test_prologue_reciprocal_folding_is_linear():
    # "folding the QK-norm reciprocal" works because RoPE is linear in a
    # per-row scalar: rope(r x) = r rope(x)
    x = rnd(128)
    for r in (0.25, 3.0, -1.5):
        assert np.allclose(O.rope(r * x, 4095.0, 1e6), r * O.rope(x, 4095.0, 1e6), atol=1e-13)


def test_prologue_switches():
    x, g = rnd(2, 128), rnd(128)
    assert np.array_equal(O.prologue(x, None, 5.0, 0.0, 1e-6), x)
    assert np.allclose(O.prologue(x, None, 5.0, 1e6, 1e-6), O.rope(x, 5.0, 1e6))
    assert np.allclose(O.prologue(x, g, 5.0, -1.0, 1e-6), O.rms_norm(x, g, 1e-6))


# ---------------------------------------------------------------- attention core

def test_single_key_returns_value_exactly():
    q, K, V = rnd(5, 128), rnd(1, 128), rnd(1, 128)
    o, lse, p = O.attend(q, K, V, 1 / math.sqrt(128))
    assert np.array_equal(o, np.repeat(V, 5, axis=0))
    assert np.array_equal(p, np.ones((5, 1)))


def test_two_key_closed_form_pins_scale_sign_and_operands():
    # k0 = 0, k1 = a e_0, q = b e_0: scores (0, scale*a*b);
    # out = (1 - w) V0 + w V1 with w = 1 / (1 + exp(-scale*a*b)).
    a, b, scale = 2.0, 3.0, 0.125
    K = np.zeros((2, 8))
    K[1, 0] = a
    q = np.zeros((1, 8))
    q[0, 0] = b
    V = rnd(2, 8)
    w = 1.0 / (1.0 + math.exp(-scale * a * b))
    o, lse, _ = O.attend(q, K, V, scale)
    assert np.allclose(o[0], (1 - w) * V[0] + w * V[1], atol=1e-15)
    assert math.isclose(lse[0], math.log(1.0 + math.exp(scale * a * b)), rel_tol=1e-14)


def test_constant_keys_give_mean_of_values():
    K = np.tile(rnd(1, 128), (37, 1))
    V = rnd(37, 128)
    o, _, p = O.attend(rnd(4, 128), K, V, 0.0883)
    assert np.allclose(o, np.tile(V.mean(axis=0), (4, 1)), atol=1e-13)


def test_softmax_rows_sum_to_one_and_nonnegative():
    _, _, p = O.attend(rnd(6, 128), rnd(50, 128), rnd(50, 128), 1 / math.sqrt(128))
    assert np.all(p >= 0)
    assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-14)


def test_linearity_in_values_and_key_permutation_invariance():
    q, K, V1, V2 = rnd(3, 128), rnd(20, 128), rnd(20, 128), rnd(20, 128)
    sc = 1 / math.sqrt(128)
    o1, _, _ = O.attend(q, K, V1, sc)
    o2, _, _ = O.attend(q, K, V2, sc)
    o12, _, _ = O.attend(q, K, 2.0 * V1 - 0.5 * V2, sc)
    assert np.allclose(o12, 2.0 * o1 - 0.5 * o2, atol=1e-13)
    perm = RNG.permutation(20)
    op, _, _ = O.attend(q, K[perm], V1[perm], sc)
    assert np.allclose(op, o1, atol=1e-13)


def test_masked_keys_do_not_contribute():
    q, K, V = rnd(1, 16), rnd(6, 16), rnd(6, 16)
    vis = np.array([[True] * 3 + [False] * 3])
    V_big = V.copy()
    V_big[3:] = 1e30
    K_big = K.copy()
    K_big[3:] = 1e3
    o, _, _ = O.attend(q, K_big, V_big, 0.25, vis)
    o_ref, _, _ = O.attend(q, K[:3], V[:3], 0.25)
    assert np.allclose(o, o_ref, atol=1e-14)


# ---------------------------------------------------------------- decode

def _decode_case(B, Hq, Hkv, S, d, lens, norm=True, theta=1e6, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    gq = 1 + 0.1 * rng.standard_normal(d) if norm else None
    gk = 1 + 0.1 * rng.standard_normal(d) if norm else None
    lens = np.asarray(lens, dtype=np.int64)
    pos = np.maximum(lens - 1, 0) + 3
    return q, k, v, lens, pos, gq, gk, theta


@pytest.mark.parametrize("G,d", [(1, 2), (2, 4), (5, 128), (8, 128), (5, 6)])
def test_decode_matches_brute_force(G, d):
    Hkv = 2
    q, k, v, lens, pos, gq, gk, th = _decode_case(2, G * Hkv, Hkv, 9, d, [9, 4], seed=G * 7 + d)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    bf = O.brute_decode(q.tolist(), k.tolist(), v.tolist(), lens, pos,
                        None if gq is None else gq.tolist(), None if gk is None else gk.tolist(), th)
    assert np.max(np.abs(ref - np.array(bf))) <= 1e-12


def test_decode_gqa_equals_mha_with_repeated_kv():
    G, Hkv = 5, 2
    q, k, v, lens, pos, gq, gk, th = _decode_case(1, G * Hkv, Hkv, 12, 128, [12], seed=3)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    k_rep, v_rep = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)     # head h -> kv h // G
    mha = O.decode_ref(q, k_rep, v_rep, lens, pos, gq, gk, th)
    assert np.allclose(ref, mha, atol=1e-14)
    # tiling (h % Hkv) would be a different model: make sure it differs
    bad = O.decode_ref(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), lens, pos, gq, gk, th)
    assert not np.allclose(ref, bad, atol=1e-3)


def test_decode_group_isolation():
    G, Hkv = 5, 3
    q, k, v, lens, pos, gq, gk, th = _decode_case(1, G * Hkv, Hkv, 10, 128, [10], seed=4)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    v2 = v.copy()
    v2[0, 1] += 1.0
    alt = O.decode_ref(q, k, v2, lens, pos, gq, gk, th)
    changed = np.any(ref != alt, axis=-1)[0]
    assert list(np.nonzero(changed)[0]) == list(range(G, 2 * G))


def test_decode_only_new_key_row_is_transformed():
    # Cached rows [0, L-2] are already post-prologue and must be used as-is;
    # only row L-1 goes through norm + RoPE.  Build the expectation from the
    # pieces: attention (pinned above) over a key set whose last row alone is
    # transformed, with the query transformed.
    q, k, v, lens, pos, gq, gk, th = _decode_case(1, 5, 1, 8, 128, [8], seed=5)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    K = k[0, 0].copy()
    K[7] = O.rope(O.rms_norm(K[7], gk, 1e-6), float(pos[0]), th)
    Q = O.rope(O.rms_norm(q[0], gq, 1e-6), float(pos[0]), th)
    o, _, _ = O.attend(Q, K, v[0, 0], 1 / math.sqrt(128))
    assert np.allclose(ref[0], o, atol=1e-14)
    # re-rotating every cached row would be a different result
    Kall = O.rope(O.rms_norm(k[0, 0], gk, 1e-6), float(pos[0]), th)
    o_bad, _, _ = O.attend(Q, Kall, v[0, 0], 1 / math.sqrt(128))
    assert not np.allclose(ref[0], o_bad, atol=1e-3)


def test_decode_empty_and_clamped_lengths():
    q, k, v, lens, pos, gq, gk, th = _decode_case(3, 4, 2, 6, 8, [0, 6, 9], seed=6)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    assert np.all(ref[0] == 0.0)
    clamped = O.decode_ref(q, k, v, np.array([0, 6, 6]), pos, gq, gk, th)
    assert np.array_equal(ref[2], clamped[2])


def test_decode_single_token_returns_value_row():
    q, k, v, lens, pos, gq, gk, th = _decode_case(1, 8, 1, 4, 128, [1], seed=7)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    assert np.array_equal(ref[0], np.repeat(v[0, 0, :1], 8, axis=0))


@pytest.mark.parametrize("T", [1, 2, 3, 7, 64, 512, 600])
def test_split_merge_equals_unsplit(T):
    q, k, v, lens, pos, gq, gk, th = _decode_case(2, 10, 2, 600, 128, [600, 131], seed=8)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, th)
    sp = O.decode_split_ref(q, k, v, lens, pos, gq, gk, th, split_tokens=T)
    assert np.max(np.abs(sp - ref)) <= 1e-12


def test_merge_associative_and_commutative():
    sc = 0.0883
    q, K, V = rnd(5, 128), rnd(30, 128), rnd(30, 128)
    parts = [O.partial_state(q, K[i:i + 10], V[i:i + 10], sc) for i in (0, 10, 20)]
    full = O.finalize(O.partial_state(q, K, V, sc))
    for perm in itertools.permutations(range(3)):
        st = O.merge(O.merge(parts[perm[0]], parts[perm[1]]), parts[perm[2]])
        assert np.allclose(O.finalize(st), full, atol=1e-13)
        st2 = O.merge(parts[perm[0]], O.merge(parts[perm[1]], parts[perm[2]]))
        assert np.allclose(O.finalize(st2), full, atol=1e-13)
    q1, K1, V1, lens, pos, gq, gk, th = _decode_case(1, 5, 1, 40, 128, [40], seed=9)
    rev = O.decode_split_ref(q1, K1, V1, lens, pos, gq, gk, th, split_tokens=7, order=[5, 3, 1, 0, 2, 4])
    assert np.max(np.abs(rev - O.decode_ref(q1, K1, V1, lens, pos, gq, gk, th))) <= 1e-12


def test_partial_state_lse_matches_attend():
    q, K, V = rnd(3, 128), rnd(17, 128), rnd(17, 128)
    m, l, Ou = O.partial_state(q, K, V, 0.1)
    o, lse, _ = O.attend(q, K, V, 0.1)
    assert np.allclose(m + np.log(l), lse, atol=1e-13)
    assert np.allclose(Ou / l[:, None], o, atol=1e-13)


# ---------------------------------------------------------------- prefill

def _prefill_case(B, Hq, Hkv, S, d, lens, norm=True, theta=1e6, seed=0, p0=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    gq = 1 + 0.1 * rng.standard_normal(d) if norm else None
    gk = 1 + 0.1 * rng.standard_normal(d) if norm else None
    return q, k, v, np.asarray(lens), np.full(B, p0), gq, gk, theta


@pytest.mark.parametrize("G,d,causal", [(1, 2, True), (2, 4, True), (5, 8, True), (8, 128, True), (5, 4, False)])
def test_prefill_matches_brute_force(G, d, causal):
    Hkv = 1 if G == 8 else 2
    q, k, v, lens, pos, gq, gk, th = _prefill_case(2, G * Hkv, Hkv, 7, d, [7, 4], seed=G + d, p0=11)
    ref = O.prefill_ref(q, k, v, lens, pos, gq, gk, th, causal=causal)
    bf = O.brute_prefill(q.tolist(), k.tolist(), v.tolist(), lens, pos,
                         None if gq is None else gq.tolist(), None if gk is None else gk.tolist(), th, causal=causal)
    assert np.max(np.abs(ref - np.array(bf))) <= 1e-12


def test_prefill_first_row_is_first_value_and_rows_match_decode():
    q, k, v, lens, pos, gq, gk, th = _prefill_case(1, 4, 2, 16, 128, [16], norm=False, theta=0.0, seed=10)
    ref = O.prefill_ref(q, k, v, lens, pos, gq, gk, th)
    assert np.array_equal(ref[0, :, 0], np.repeat(v[0, :, 0], 2, axis=0))
    for i in (1, 5, 15):
        dec = O.decode_ref(q[:, :, i], k, v, np.array([i + 1]), np.array([i]), None, None, 0.0)
        assert np.allclose(ref[0, :, i], dec[0], atol=1e-13)


def test_prefill_last_row_equals_decode_over_transformed_cache():
    # With the prologue on, decode at L = S over a cache whose rows < S-1 hold
    # the transformed keys equals prefill's last query row.
    S = 12
    q, k, v, lens, pos, gq, gk, th = _prefill_case(1, 5, 1, S, 128, [S], seed=11, p0=100)
    ref = O.prefill_ref(q, k, v, lens, pos, gq, gk, th)
    positions = 100 + np.arange(S)
    kt = O.prologue(k[0, 0], gk, positions, th, 1e-6)
    cache = k.copy()
    cache[0, 0, :S - 1] = kt[:S - 1]
    dec = O.decode_ref(q[:, :, S - 1], cache, v, np.array([S]), np.array([100 + S - 1]), gq, gk, th)
    assert np.allclose(ref[0, :, S - 1], dec[0], atol=1e-13)


def test_prefill_relative_position_invariance():
    q, k, v, lens, pos, gq, gk, th = _prefill_case(1, 2, 1, 10, 128, [10], seed=12)
    a = O.prefill_ref(q, k, v, lens, np.array([0]), gq, gk, th)
    b = O.prefill_ref(q, k, v, lens, np.array([5000]), gq, gk, th)
    assert np.allclose(a, b, atol=1e-9)


def test_prefill_ragged_rows_and_row_subsets():
    q, k, v, lens, pos, gq, gk, th = _prefill_case(2, 4, 2, 9, 16, [9, 3], seed=13)
    ref = O.prefill_ref(q, k, v, lens, pos, gq, gk, th)
    assert np.all(ref[1, :, 3:] == 0.0)
    sub = O.prefill_ref(q, k, v, lens, pos, gq, gk, th, heads=[1, 2], rows=np.array([0, 4, 8]))
    for hq in (1, 2):
        for r in (0, 4, 8):
            assert np.array_equal(sub[0, hq, r], ref[0, hq, r])
    assert np.all(sub[0, 0] == 0.0)


def test_causal_tile_classes_count_lower_triangle():
    # ADR-0060 §5.4 / §11: with aligned square tiles the non-skipped pairs are
    # the lower triangle including the diagonal: T(T+1)/2 of T^2.
    for n, bm in ((4096, 128), (1000, 64), (64, 64)):
        T = -(-n // bm)
        c = O.causal_tile_pairs(n, bm, bm)
        assert c["past"] + c["partial"] == T * (T + 1) // 2
        assert c["partial"] == T
        assert c["future"] == T * (T - 1) // 2
    assert O.causal_tile_class(128, 256, 0, 128) == "past"
    assert O.causal_tile_class(128, 256, 256, 384) == "future"
    assert O.causal_tile_class(128, 256, 192, 256) == "partial"
