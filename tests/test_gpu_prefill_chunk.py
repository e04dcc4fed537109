"""GPU parity of gqa_attn_prefill_chunk (through the C ABI) against the fp64
chunked-prefill oracle.  bf16 inputs, fp16 MFMA operands, f32 accumulation
and output: max |err| <= 1e-2.  Cached rows j < P hold the oracle's own post-prologue
keys rounded to bf16; the chunk's rows are raw; rows past P + T of the caches
and rows past T of q are NaN, so a read of them shows up in the output.
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def make(B, Hq, Hkv, S, Tmax, past, chunk, norm=True, theta=1e6, p0=3, seed=61):
    rng = np.random.default_rng(seed)
    bf = lambda x: synth.bf16_round(x.astype(np.float32))
    q = bf(rng.standard_normal((B, Hq, Tmax, 128)))
    k = bf(rng.standard_normal((B, Hkv, S, 128)))
    v = bf(rng.standard_normal((B, Hkv, S, 128)))
    gq = bf(1 + 0.1 * rng.standard_normal(128)) if norm else None
    gk = bf(1 + 0.1 * rng.standard_normal(128)) if norm else None
    past, chunk = np.asarray(past, dtype=np.int32), np.asarray(chunk, dtype=np.int32)
    pos = np.full(B, p0, dtype=np.int32)
    for b in range(B):
        P = min(max(int(past[b]), 0), S)
        T = min(max(int(chunk[b]), 0), Tmax, S - P)
        for h in range(Hkv):
            k[b, h, :P] = bf(O.prologue(k[b, h, :P], gk, p0 + np.arange(P), theta, 1e-6))
        k[b, :, P + T:] = np.nan
        v[b, :, P + T:] = np.nan
        q[b, :, T:] = np.nan
    return dict(q=q, k=k, v=v, past=past, chunk=chunk, pos=pos, gq=gq, gk=gk, theta=theta)


def run(c, causal=True, out=None):
    torch = require_gpu()
    bfd = torch.bfloat16
    o = G.prefill_chunk(dev(c["q"], bfd), dev(c["k"], bfd), dev(c["v"], bfd), ints(c["past"]), ints(c["chunk"]),
                        ints(c["pos"]), dev(c["gq"], bfd), dev(c["gk"], bfd), c["theta"], out=out, causal=causal)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def ref(c, causal=True, **kw):
    return O.prefill_chunk_ref(c["q"], c["k"], c["v"], c["past"], c["chunk"], c["pos"], c["gq"], c["gk"],
                               c["theta"], causal=causal, **kw)


def valid(out, c):
    o = out.copy()
    for b in range(o.shape[0]):
        T = min(max(int(c["chunk"][b]), 0), o.shape[2], c["k"].shape[2] - min(max(int(c["past"][b]), 0), c["k"].shape[2]))
        o[b, :, T:] = 0.0
    return o


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_chunks_after_cached_prefixes(causal):
    c = make(B=3, Hq=10, Hkv=2, S=300, Tmax=130, past=[100, 0, 250], chunk=[130, 64, 37])
    log(f"case chunked prefill ragged causal={causal}")
    out = run(c, causal)
    compare(valid(out, c), ref(c, causal), ATOL, f"chunked prefill causal={causal}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (16, 2), (40, 8)])
def test_group_sizes(Hq, Hkv):
    c = make(B=1, Hq=Hq, Hkv=Hkv, S=200, Tmax=96, past=[77], chunk=[96], seed=62)
    compare(valid(run(c), c), ref(c), ATOL, f"chunk Hq={Hq} Hkv={Hkv}")


def test_edges_empty_full_and_clamped():
    torch = require_gpu()
    # T = 0; P + T = max_seq exactly; P = max_seq (T clamps to 0); T > T_max - clamped
    c = make(B=4, Hq=10, Hkv=2, S=160, Tmax=64, past=[10, 96, 160, 120], chunk=[0, 64, 5, 70], seed=63)
    out_t = torch.full((4, 10, 64, 128), 777.0, device="cuda")
    out = run(c, out=out_t)
    assert np.all(out[0] == 777.0) and np.all(out[2] == 777.0)   # nothing written
    assert np.all(out[3, :, 40:] == 777.0)                       # T = min(70, 64, 160 - 120) = 40
    compare(valid(out, c), ref(c), ATOL, "chunk edges")


def test_single_token_chunk_matches_decode():
    torch = require_gpu()
    c = make(B=2, Hq=10, Hkv=2, S=256, Tmax=1, past=[255, 40], chunk=[1, 1], seed=64, p0=9)
    out = run(c)
    bfd = torch.bfloat16
    k = np.nan_to_num(c["k"])
    dec = G.decode(dev(c["q"][:, :, 0], bfd), dev(k, bfd), dev(np.nan_to_num(c["v"]), bfd), ints(c["past"] + 1),
                   ints(c["pos"] + c["past"]), dev(c["gq"], bfd), dev(c["gk"], bfd), c["theta"])
    torch.cuda.synchronize()
    compare(out[:, :, 0], dec.cpu().numpy(), 5e-3, "T=1 chunk vs decode")
    compare(out, ref(c), ATOL, "T=1 chunk")


def test_empty_past_equals_plain_prefill_bitwise():
    torch = require_gpu()
    c = make(B=2, Hq=10, Hkv=2, S=200, Tmax=200, past=[0, 0], chunk=[200, 131], seed=65)
    a = run(c)
    bfd = torch.bfloat16
    p = G.prefill(dev(c["q"], bfd), dev(c["k"], bfd), dev(c["v"], bfd), ints(c["chunk"]), ints(c["pos"]),
                  dev(c["gq"], bfd), dev(c["gk"], bfd), c["theta"])
    torch.cuda.synchronize()
    assert np.array_equal(valid(a, c), valid(p.cpu().numpy(), c))


def test_qwen3_chunk_3072_plus_1024_full():
    # the last 1024 tokens of a 4096-token Qwen3-14B prompt as one chunk after
    # 3072 cached ones (40 / 8 heads): every element, out pre-filled with NaN
    torch = require_gpu()
    c = make(B=1, Hq=40, Hkv=8, S=4096, Tmax=1024, past=[3072], chunk=[1024], seed=66)
    log("case chunked prefill qwen3 3072+1024 (out pre-filled with NaN)")
    out_t = torch.full((1, 40, 1024, 128), float("nan"), dtype=torch.float32, device="cuda")
    out = run(c, out=out_t)
    compare(out, ref(c), ATOL, "qwen3 chunk 3072+1024, all heads and rows")


@pytest.mark.parametrize("past,chunk", [(4000, 96), (3968, 128)])
def test_qwen3_short_chunk_after_long_prefix_full(past, chunk):
    # a short chunk after a long cached prefix: few query blocks, so each
    # block's key range is split over several workgroups whose partials the
    # last one merges; every element, out pre-filled with NaN
    torch = require_gpu()
    c = make(B=1, Hq=40, Hkv=8, S=past + chunk, Tmax=chunk, past=[past], chunk=[chunk], seed=67)
    log(f"case chunked prefill qwen3 {past}+{chunk} (out pre-filled with NaN)")
    out_t = torch.full((1, 40, chunk, 128), float("nan"), dtype=torch.float32, device="cuda")
    out = run(c, out=out_t)
    compare(out, ref(c), ATOL, f"qwen3 chunk {past}+{chunk}, all heads and rows")


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_paged_chunk_equals_contiguous_bitwise(bs):
    torch = require_gpu()
    S = 512
    c = make(B=2, Hq=10, Hkv=2, S=S, Tmax=128, past=[300, 0], chunk=[128, 77], seed=67)
    log(f"case paged chunked prefill bs={bs}")
    # the same logical cache as shuffled pages; blocks past the sequence are unmapped (-1)
    rng = np.random.default_rng(bs)
    nb = S // bs
    perm = rng.permutation(2 * nb + 2)
    table = perm[:2 * nb].reshape(2, nb).astype(np.int32)
    kp = np.full((2 * nb + 2, 2, bs, 128), np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    for b in range(2):
        used = -(-int(c["past"][b] + c["chunk"][b]) // bs)
        for i in range(nb):
            kp[table[b, i]] = c["k"][b][:, i * bs:(i + 1) * bs]
            vp[table[b, i]] = c["v"][b][:, i * bs:(i + 1) * bs]
        table[b, used:] = -1
    bfd = torch.bfloat16
    paged = G.prefill_chunk_paged(dev(c["q"], bfd), dev(kp, bfd), dev(vp, bfd), ints(table), ints(c["past"]),
                                  ints(c["chunk"]), ints(c["pos"]), dev(c["gq"], bfd), dev(c["gk"], bfd), c["theta"])
    torch.cuda.synchronize()
    cont = run(c)
    assert np.array_equal(valid(paged.cpu().numpy(), c), valid(cont, c))
    K = O.paged_gather(kp, table, c["past"] + c["chunk"], bs, S)
    V = O.paged_gather(vp, table, c["past"] + c["chunk"], bs, S)
    want = O.prefill_chunk_ref(c["q"], K, V, c["past"], c["chunk"], c["pos"], c["gq"], c["gk"], c["theta"])
    compare(valid(paged.cpu().numpy(), c), want, ATOL, f"paged chunk bs={bs}")
