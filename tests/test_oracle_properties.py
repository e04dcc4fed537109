"""Property-based pins of the oracle (CPU): on randomly drawn tiny shapes, the
vectorised fp64 reference equals the pure-Python scalar-loop brute force, and
the split-KV path (chunked partials folded by the log-sum-exp merge of
"ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)", section 4) equals
the unsplit result for any chunk length and merge order.

The drawn parameters cover what the fixed-case tests pin at chosen points:
group sizes, head dims, ragged and empty lengths, RMSNorm on or off, RoPE on
or off at varied positions, causal and full masks, cached prefixes of a
chunked prefill."""

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle as O

SETTINGS = dict(max_examples=25, deadline=None, derandomize=True)

shape = st.fixed_dictionaries({
    "B": st.integers(1, 2),
    "G": st.sampled_from([1, 2, 3, 5, 8]),
    "Hkv": st.integers(1, 2),
    "d": st.sampled_from([2, 4, 6, 8]),
    "S": st.integers(1, 9),
    "norm": st.booleans(),
    "theta": st.sampled_from([0.0, 1e4, 1e6]),
    "seed": st.integers(0, 2**31 - 1),
})


def _draw(p):
    rng = np.random.Generator(np.random.PCG64(p["seed"]))
    B, Hkv, d, S = p["B"], p["Hkv"], p["d"], p["S"]
    Hq = p["G"] * Hkv
    gq = 1 + 0.1 * rng.standard_normal(d) if p["norm"] else None
    gk = 1 + 0.1 * rng.standard_normal(d) if p["norm"] else None
    return rng, B, Hq, Hkv, d, S, gq, gk


def _lists(x):
    return None if x is None else x.tolist()


@settings(**SETTINGS)
@given(shape)
def test_decode_equals_brute_force(p):
    rng, B, Hq, Hkv, d, S, gq, gk = _draw(p)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    lens = rng.integers(0, S + 1, size=B)
    pos = rng.integers(0, 5000, size=B)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, p["theta"])
    bf = np.array(O.brute_decode(q.tolist(), k.tolist(), v.tolist(), lens, pos, _lists(gq), _lists(gk), p["theta"]))
    assert np.max(np.abs(ref - bf)) <= 1e-12


@settings(**SETTINGS)
@given(shape, st.integers(1, 9), st.booleans())
def test_split_merge_equals_unsplit(p, T, reverse):
    rng, B, Hq, Hkv, d, S, gq, gk = _draw(p)
    q = rng.standard_normal((B, Hq, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    lens = rng.integers(0, S + 1, size=B)
    pos = rng.integers(0, 5000, size=B)
    ref = O.decode_ref(q, k, v, lens, pos, gq, gk, p["theta"])
    n = -(-S // T)
    order = list(range(n))[::-1] if reverse else None
    sp = O.decode_split_ref(q, k, v, lens, pos, gq, gk, p["theta"], split_tokens=T, order=order)
    assert np.max(np.abs(ref - sp)) <= 1e-12


@settings(**SETTINGS)
@given(shape, st.booleans())
def test_prefill_equals_brute_force(p, causal):
    rng, B, Hq, Hkv, d, S, gq, gk = _draw(p)
    q = rng.standard_normal((B, Hq, S, d))
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    lens = rng.integers(0, S + 1, size=B)
    pos = rng.integers(0, 5000, size=B)
    ref = O.prefill_ref(q, k, v, lens, pos, gq, gk, p["theta"], causal=causal)
    bf = np.array(O.brute_prefill(q.tolist(), k.tolist(), v.tolist(), lens, pos, _lists(gq), _lists(gk),
                                  p["theta"], causal=causal))
    for b in range(B):   # rows past a sequence's length are not outputs
        L = int(lens[b])
        assert np.max(np.abs(ref[b, :, :L] - bf[b, :, :L]), initial=0.0) <= 1e-12


@settings(**SETTINGS)
@given(shape, st.integers(1, 6), st.booleans())
def test_prefill_chunk_equals_brute_force(p, T_max, causal):
    rng, B, Hq, Hkv, d, S, gq, gk = _draw(p)
    S_max = S + T_max
    q = rng.standard_normal((B, Hq, T_max, d))
    k = rng.standard_normal((B, Hkv, S_max, d))
    v = rng.standard_normal((B, Hkv, S_max, d))
    past = rng.integers(0, S + 1, size=B)
    chunk = rng.integers(0, T_max + 1, size=B)
    pos = rng.integers(0, 5000, size=B)
    ref = O.prefill_chunk_ref(q, k, v, past, chunk, pos, gq, gk, p["theta"], causal=causal)
    bf = np.array(O.brute_prefill_chunk(q.tolist(), k.tolist(), v.tolist(), past, chunk, pos, _lists(gq),
                                        _lists(gk), p["theta"], causal=causal))
    for b in range(B):
        T = int(chunk[b])
        assert np.max(np.abs(ref[b, :, :T] - bf[b, :, :T]), initial=0.0) <= 1e-12
