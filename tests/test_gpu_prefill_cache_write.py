"""GPU checks of the prefill key-cache write-back (descriptor flag
write_k_cache) and of an engine's sequence of calls run by the library alone.

With write_k_cache the key phase of gqa_attn_prefill / _chunk / _chunk_paged
stores every new token's post-prologue key k'_s (rounded to bf16) over its raw
row; the output and every other cache byte are unchanged.  Expected rows come
from the fp64 oracle's prologue, never from the GPU: a stored row may differ
from the oracle's by the bf16 rounding of the f32 result (half an ulp, 2^-8
relative) plus the f32 arithmetic error.
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL = 1e-2
EPS = 1e-6
THETA = 1e6


def bf(x):
    return synth.bf16_round(np.asarray(x, dtype=np.float32))


def row_bound(ref):
    return 2.0 ** -8 * np.abs(ref) + 1e-5


def rows_close(got, ref, what):
    err = np.abs(got - ref)
    assert np.all(err <= row_bound(ref)), f"{what}: max stored-row error {err.max()}"


def test_prefill_write_k_cache_stores_the_prologue_rows():
    torch = require_gpu()
    rng = np.random.default_rng(51)
    B, Hq, Hkv, S = 2, 10, 2, 300
    lens, pos0 = np.array([300, 129], dtype=np.int32), np.array([0, 77], dtype=np.int32)
    q, k, v = (bf(rng.standard_normal((B, h, S, 128))) for h in (Hq, Hkv, Hkv))
    gq, gk = bf(1 + 0.1 * rng.standard_normal(128)), bf(1 + 0.1 * rng.standard_normal(128))
    t = torch.bfloat16
    k0, k1, vd, qd = dev(k, t), dev(k, t), dev(v, t), dev(q, t)
    # rows past a sequence's length are not written: both outputs start equal
    a = G.prefill(qd, k0, vd, ints(lens), ints(pos0), dev(gq, t), dev(gk, t), THETA, eps=EPS,
                  out=torch.zeros(B, Hq, S, 128, device="cuda"))
    b = G.prefill(qd, k1, vd, ints(lens), ints(pos0), dev(gq, t), dev(gk, t), THETA, eps=EPS, write_k_cache=True,
                  out=torch.zeros(B, Hq, S, 128, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(a, b), "write_k_cache changed the output"
    assert torch.equal(k0, dev(k, t)), "flag off wrote the cache"
    assert torch.equal(vd, dev(v, t)), "v written"
    kc = k1.float().cpu().numpy()
    for bi in range(B):
        n = int(lens[bi])
        want = O.prologue(k[bi][:, :n], gk, pos0[bi] + np.arange(n), THETA, EPS)
        rows_close(kc[bi][:, :n], want, f"b={bi}")
        assert np.array_equal(kc[bi][:, n:], k[bi][:, n:]), f"b={bi}: rows past the sequence changed"


def test_prefill_write_k_cache_without_prologue_writes_nothing():
    torch = require_gpu()
    rng = np.random.default_rng(52)
    q, k, v = (bf(rng.standard_normal((1, h, 160, 128))) for h in (10, 2, 2))
    t = torch.bfloat16
    kd = dev(k, t)
    G.prefill(dev(q, t), kd, dev(v, t), ints([160]), ints([0]), None, None, 0.0, write_k_cache=True)
    torch.cuda.synchronize()
    assert torch.equal(kd, dev(k, t))


@pytest.mark.parametrize("bs", [0, 64])
def test_chunk_write_k_cache_stores_only_the_chunk_rows(bs):
    torch = require_gpu()
    rng = np.random.default_rng(53 + bs)
    B, Hq, Hkv, S, Tmax = 2, 10, 2, 512, 128
    past, chunk, pos0 = np.array([300, 0], np.int32), np.array([128, 77], np.int32), np.array([3, 9], np.int32)
    gq, gk = bf(1 + 0.1 * rng.standard_normal(128)), bf(1 + 0.1 * rng.standard_normal(128))
    q = bf(rng.standard_normal((B, Hq, Tmax, 128)))
    k, v = bf(rng.standard_normal((B, Hkv, S, 128))), bf(rng.standard_normal((B, Hkv, S, 128)))
    for b in range(B):   # cached rows hold post-prologue keys
        P = int(past[b])
        k[b][:, :P] = bf(O.prologue(k[b][:, :P], gk, pos0[b] + np.arange(P), THETA, EPS))
    t = torch.bfloat16
    log(f"case chunk write_k_cache bs={bs}")
    zeros = lambda: torch.zeros(B, Hq, Tmax, 128, device="cuda")   # rows past a chunk are not written
    if bs == 0:
        k0, k1, vd = dev(k, t), dev(k, t), dev(v, t)
        call = lambda kk, w: G.prefill_chunk(dev(q, t), kk, vd, ints(past), ints(chunk), ints(pos0), dev(gq, t),
                                             dev(gk, t), THETA, eps=EPS, write_k_cache=w, out=zeros())
        logical = lambda kk: kk.float().cpu().numpy()
    else:
        nb = S // bs
        perm = rng.permutation(B * nb)
        table = perm.reshape(B, nb).astype(np.int32)
        kp = np.zeros((B * nb, Hkv, bs, 128), np.float32)
        vp = np.zeros_like(kp)
        for b in range(B):
            for i in range(nb):
                kp[table[b, i]] = k[b][:, i * bs:(i + 1) * bs]
                vp[table[b, i]] = v[b][:, i * bs:(i + 1) * bs]
        k0, k1, vd = dev(kp, t), dev(kp, t), dev(vp, t)
        call = lambda kk, w: G.prefill_chunk_paged(dev(q, t), kk, vd, ints(table), ints(past), ints(chunk),
                                                   ints(pos0), dev(gq, t), dev(gk, t), THETA, eps=EPS,
                                                   write_k_cache=w, out=zeros())
        logical = lambda kk: O.paged_gather(kk.float().cpu().numpy(), table, np.full(B, S), bs, S)
    a = call(k0, False)
    b2 = call(k1, True)
    torch.cuda.synchronize()
    assert torch.equal(a, b2), "write_k_cache changed the output"
    kc = logical(k1)
    for b in range(B):
        P, T = int(past[b]), int(chunk[b])
        want = O.prologue(k[b][:, P:P + T], gk, pos0[b] + P + np.arange(T), THETA, EPS)
        rows_close(kc[b][:, P:P + T], want, f"b={b}")
        assert np.array_equal(kc[b][:, :P], k[b][:, :P]), f"b={b}: cached rows changed"
        assert np.array_equal(kc[b][:, P + T:], k[b][:, P + T:]), f"b={b}: rows past the chunk changed"


def test_engine_sequence_prefill_chunks_then_decode():
    """prefill of 1000 tokens -> chunk of 500 -> chunk of 96 -> three decode
    steps, on one bf16 cache that only the library writes (write_k_cache,
    then write_new_k).  Every output against the oracle, whose own cache
    history holds its transformed rows rounded to bf16."""
    torch = require_gpu()
    rng = np.random.default_rng(57)
    Hq, Hkv, S = 10, 2, 1600
    plan = [("prefill", 1000), ("chunk", 500), ("chunk", 96), ("decode", 1), ("decode", 1), ("decode", 1)]
    N = sum(n for _, n in plan)
    pos0 = 21
    qraw = bf(rng.standard_normal((Hq, N, 128)))
    kraw = bf(rng.standard_normal((Hkv, N, 128)))
    vraw = bf(rng.standard_normal((Hkv, N, 128)))
    gq, gk = bf(1 + 0.1 * rng.standard_normal(128)), bf(1 + 0.1 * rng.standard_normal(128))
    t = torch.bfloat16
    kd = torch.full((1, Hkv, S, 128), float("nan"), dtype=t, device="cuda")
    vd = torch.full((1, Hkv, S, 128), float("nan"), dtype=t, device="cuda")
    ocache = np.full((1, Hkv, S, 128), np.nan, np.float32)   # the oracle's own cache
    ovals = np.full((1, Hkv, S, 128), np.nan, np.float32)
    done = 0
    for kind, n in plan:
        lo, hi = done, done + n
        # the caller appends the new tokens' raw keys and values to the caches
        kd[0, :, lo:hi] = dev(kraw[:, lo:hi], t)
        vd[0, :, lo:hi] = dev(vraw[:, lo:hi], t)
        ocache[0, :, lo:hi] = kraw[:, lo:hi]
        ovals[0, :, lo:hi] = vraw[:, lo:hi]
        log(f"case engine sequence: {kind} of tokens [{lo}, {hi})")
        if kind == "prefill":
            q = np.full((1, Hq, S, 128), np.nan, np.float32)
            q[0, :, :n] = qraw[:, lo:hi]
            out = G.prefill(dev(q, t), kd, vd, ints([n]), ints([pos0]), dev(gq, t), dev(gk, t), THETA, eps=EPS,
                            write_k_cache=True)
            torch.cuda.synchronize()
            want = O.prefill_ref(q, ocache, ovals, [n], [pos0], gq, gk, THETA, EPS)
            got = out.cpu().numpy()[:, :, :n]
            want = want[:, :, :n]
        elif kind == "chunk":
            q = qraw[None, :, lo:hi]
            out = G.prefill_chunk(dev(q, t), kd, vd, ints([lo]), ints([n]), ints([pos0]), dev(gq, t), dev(gk, t),
                                  THETA, eps=EPS, write_k_cache=True)
            torch.cuda.synchronize()
            want = O.prefill_chunk_ref(q, ocache, ovals, [lo], [n], [pos0], gq, gk, THETA, EPS)
            got = out.cpu().numpy()
        else:
            q = qraw[None, :, lo]
            out = G.decode(dev(q, t), kd, vd, ints([hi]), ints([pos0 + lo]), dev(gq, t), dev(gk, t), THETA,
                           eps=EPS, write_new_k=True)
            torch.cuda.synchronize()
            want = O.decode_ref(q, ocache, ovals, [hi], [pos0 + lo], gq, gk, THETA, EPS)
            got = out.cpu().numpy()
        compare(got, want, ATOL, f"engine {kind} [{lo}, {hi})")
        # the stored rows against the oracle's prologue; the oracle's history
        # takes its own transformed rows, not the GPU's
        rows = O.prologue(kraw[:, lo:hi], gk, pos0 + np.arange(lo, hi), THETA, EPS)
        rows_close(kd[0, :, lo:hi].float().cpu().numpy(), rows, f"engine {kind} stored rows")
        ocache[0, :, lo:hi] = bf(rows)
        assert torch.equal(vd[0, :, :hi], dev(ovals[0, :, :hi], t)), "v_cache written"
        done = hi
