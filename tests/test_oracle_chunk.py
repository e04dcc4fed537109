"""Pins for the chunked-prefill oracle (prefill_chunk_ref): a query block of
T_q new tokens after P cached ones, aligned at the bottom right of the causal
score matrix.  Each pin ties it to something other than its own formula: the
scalar brute force, the decode oracle (T_q = 1), the full prefill oracle
(P = 0, and two chunks that compose into one prefill), closed forms of the
visibility rule, and the clamping reading.
"""

import numpy as np
import pytest

import oracle as O


def case(B, Hq, Hkv, S_max, T_max, d, past, chunk, norm=True, theta=1e6, seed=0, p0=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T_max, d))
    k = rng.standard_normal((B, Hkv, S_max, d))
    v = rng.standard_normal((B, Hkv, S_max, d))
    gq = 1 + 0.1 * rng.standard_normal(d) if norm else None
    gk = 1 + 0.1 * rng.standard_normal(d) if norm else None
    return q, k, v, np.asarray(past), np.asarray(chunk), np.full(B, p0), gq, gk, theta


def lists(x):
    return None if x is None else np.asarray(x).tolist()


@pytest.mark.parametrize("G,d,causal", [(1, 2, True), (2, 4, True), (5, 8, True), (5, 4, False)])
def test_chunk_matches_brute_force(G, d, causal):
    Hkv = 2
    q, k, v, P, T, pos, gq, gk, th = case(3, G * Hkv, Hkv, 11, 5, d, [4, 0, 9], [5, 3, 2], seed=G + d)
    ref = O.prefill_chunk_ref(q, k, v, P, T, pos, gq, gk, th, causal=causal)
    bf = O.brute_prefill_chunk(lists(q), lists(k), lists(v), P, T, pos, lists(gq), lists(gk), th, causal=causal)
    assert np.max(np.abs(ref - np.array(bf))) <= 1e-12


def test_single_token_chunk_equals_decode():
    # T_q = 1 after P cached tokens is one decode step at L = P + 1 whose new
    # token sits at position positions[b] + P
    q, k, v, P, T, pos, gq, gk, th = case(2, 10, 2, 40, 1, 128, [17, 39], [1, 1], seed=5, p0=100)
    ref = O.prefill_chunk_ref(q, k, v, P, T, pos, gq, gk, th)
    dec = O.decode_ref(q[:, :, 0], k, v, P + 1, pos + P, gq, gk, th)
    assert np.allclose(ref[:, :, 0], dec, atol=1e-12)


def test_empty_past_equals_full_prefill():
    q, k, v, P, T, pos, gq, gk, th = case(2, 4, 2, 12, 12, 16, [0, 0], [12, 7], seed=6)
    ref = O.prefill_chunk_ref(q, k, v, P, T, pos, gq, gk, th)
    full = O.prefill_ref(q, k, v, T, pos, gq, gk, th)
    assert np.allclose(ref, full, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_two_chunks_compose_into_one_prefill(causal):
    # prefill of n tokens == chunk [0, T1) then chunk [T1, n) over a cache
    # whose first T1 rows hold the keys after the prologue (non-causal: the
    # second chunk's queries see every key, the first chunk's only the first
    # T1, so only the causal case composes row for row; non-causal checks the
    # second chunk's rows)
    n, T1, d = 13, 5, 32
    q, k, v, _, _, pos, gq, gk, th = case(1, 4, 2, n, n, d, [0], [n], seed=7, p0=40)
    full = O.prefill_ref(q, k, v, np.array([n]), pos, gq, gk, th, causal=causal)
    a = O.prefill_chunk_ref(q[:, :, :T1], k, v, np.array([0]), np.array([T1]), pos, gq, gk, th, causal=causal)
    cache = k.copy()
    for h in range(2):
        cache[0, h, :T1] = O.prologue(k[0, h, :T1], gk, 40 + np.arange(T1), th, 1e-6)
    b = O.prefill_chunk_ref(q[:, :, T1:], cache, v, np.array([T1]), np.array([n - T1]), pos, gq, gk, th,
                            causal=causal)
    assert np.allclose(b[:, :, :n - T1], full[:, :, T1:], atol=1e-12)
    if causal:
        assert np.allclose(a[:, :, :T1], full[:, :, :T1], atol=1e-12)


def test_visibility_bottom_right_closed_form():
    # with no prologue and one-hot values, the weight a query puts on key j
    # is read off the output; query t must put zero weight on keys j > P + t
    P, T, S = 6, 4, 12
    d = S
    q, k, v, _, _, pos, _, _, _ = case(1, 1, 1, S, T, d, [P], [T], norm=False, theta=0.0, seed=8)
    v = np.eye(S)[None, None]                      # value row j = e_j
    ref = O.prefill_chunk_ref(q, k, v, np.array([P]), np.array([T]), pos, None, None, 0.0)
    for t in range(T):
        w = ref[0, 0, t]
        assert np.all(w[P + t + 1:] == 0.0) and np.all(w[:P + t + 1] > 0.0)
        assert abs(w.sum() - 1.0) < 1e-12


def test_cached_rows_are_not_transformed():
    # changing the prologue of the chunk must not touch rows j < P: with the
    # prologue off the cached rows and raw rows give the plain attention
    q, k, v, P, T, pos, gq, gk, th = case(1, 2, 1, 9, 3, 8, [6], [3], seed=9)
    ref = O.prefill_chunk_ref(q, k, v, P, T, pos, None, None, 0.0)
    vis = np.arange(9)[None, :] <= (6 + np.arange(3))[:, None]
    out, _, _ = O.attend(q[0, 0, :3], k[0, 0, :9], v[0, 0, :9], 1 / np.sqrt(8), vis)
    assert np.allclose(ref[0, 0, :3], out, atol=1e-13)


def test_clamping_reading():
    # P clamps to [0, S_max]; T to [0, min(T_max, S_max - P)]; rows t >= T stay 0
    q, k, v, _, _, pos, gq, gk, th = case(3, 2, 1, 10, 4, 8, [0, 0, 0], [0, 0, 0], seed=10)
    ref = O.prefill_chunk_ref(q, k, v, np.array([8, 12, -3]), np.array([9, 2, 2]), pos, gq, gk, th)
    assert np.all(ref[0, :, 2:] == 0.0) and np.any(ref[0, :, :2] != 0.0)   # T = min(9, 4, 10 - 8) = 2
    assert np.all(ref[1] == 0.0)                                             # P = 10: no room
    want = O.prefill_chunk_ref(q[2:], k[2:], v[2:], np.array([0]), np.array([2]), pos[2:], gq, gk, th)
    assert np.array_equal(ref[2:], want)                                     # P = -3 -> 0
