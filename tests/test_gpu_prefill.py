"""GPU parity of gqa_attn_prefill (through the C ABI) against the fp64 oracle.

bf16 inputs, fp16 MFMA operands (q', k', P rounded to fp16, v converted
exactly), f32 accumulation, f32 output: max |err| <= 1e-2.
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL_BF16 = 1e-2


def gpu_inputs(inp):
    torch = require_gpu()
    bf = torch.bfloat16
    return dict(q=dev(inp["q"], bf), k=dev(inp["k"], bf), v=dev(inp["v"], bf), qw=dev(inp["q_norm_w"], bf),
                kw=dev(inp["k_norm_w"], bf), sl=ints(inp["seq_lens"]), pos=ints(inp["positions"]))


PATHS = ["two_phase", "single_kernel"]


def run(inp, out_dtype=None, g=None, out=None, path="two_phase"):
    """path: two_phase (workspace given: key prologue once, then attention) or
    single_kernel (no workspace: key prologue per key tile)."""
    torch = require_gpu()
    g = g or gpu_inputs(inp)
    o = G.prefill(g["q"], g["k"], g["v"], g["sl"], g["pos"], g["qw"], g["kw"], inp["rope_theta"], out=out,
                  causal=inp["causal"], eps=inp["eps"], out_dtype=out_dtype or torch.float32,
                  workspace="auto" if path == "two_phase" else None)
    torch.cuda.synchronize()
    return o


def ref(inp, **kw):
    return O.prefill_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["positions"], inp["q_norm_w"],
                         inp["k_norm_w"], inp["rope_theta"], inp["eps"], causal=inp["causal"], **kw)


def small(B=2, Hq=10, Hkv=2, S=300, lens=None, causal=True, norm=True, theta=1e6, p0=0, seed=21):
    w = synth.PrefillWorkload(f"small_prefill_b{B}_h{Hq}_{Hkv}_s{S}", B, Hq, Hkv, S, "bf16", norm, theta,
                              causal=causal, position0=p0, seed=seed)
    inp = synth.make_prefill(w, poison=False)
    if lens is not None:
        inp["seq_lens"] = np.asarray(lens, dtype=np.int32)
    for b in range(B):
        n = max(0, min(int(inp["seq_lens"][b]), S))
        for key in ("q", "k", "v"):
            inp[key][b, :, n:] = np.nan
    return inp


def valid_rows(out, inp):
    """Zero rows at or past each sequence length (they are not written)."""
    o = out.copy()
    for b, n in enumerate(inp["seq_lens"]):
        o[b, :, max(0, int(n)):] = 0.0
    return o


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("causal", [True, False])
def test_small_ragged_multi_tile(causal, path):
    inp = small(B=2, Hq=10, Hkv=2, S=300, lens=[300, 129], causal=causal, p0=0)
    inp["positions"] = np.array([0, 1000], dtype=np.int32)
    log(f"case small prefill causal={causal} path={path}")
    out = run(inp, path=path).cpu().numpy()
    compare(valid_rows(out, inp), ref(inp), ATOL_BF16, f"prefill causal={causal} {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (8, 1), (12, 4), (14, 2)])
def test_group_sizes(Hq, Hkv, path):
    inp = small(B=1, Hq=Hq, Hkv=Hkv, S=200, lens=[200])
    out = run(inp, path=path).cpu().numpy()
    compare(valid_rows(out, inp), ref(inp), ATOL_BF16, f"Hq={Hq} Hkv={Hkv} {path}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("norm,theta", [(False, 0.0), (True, 0.0), (False, 5e5)])
def test_prologue_switches(norm, theta, path):
    inp = small(B=1, Hq=10, Hkv=2, S=160, lens=[160], norm=norm, theta=theta)
    out = run(inp, path=path).cpu().numpy()
    compare(valid_rows(out, inp), ref(inp), ATOL_BF16, f"norm={norm} theta={theta} {path}")


@pytest.mark.parametrize("path", PATHS)
def test_short_and_empty_sequences(path):
    inp = small(B=4, Hq=10, Hkv=2, S=130, lens=[1, 0, 64, 130])
    torch = require_gpu()
    out_t = torch.full((4, 10, 130, 128), 777.0, device="cuda")
    run(inp, out=out_t, path=path)
    out = out_t.cpu().numpy()
    assert np.all(out[1] == 777.0)                 # n = 0: nothing written
    assert np.all(out[0, :, 1:] == 777.0)          # rows past n untouched
    compare(valid_rows(out, inp), ref(inp), ATOL_BF16, "short/empty")


def test_first_row_equals_first_value_row():
    inp = small(B=1, Hq=10, Hkv=2, S=128, lens=[128])
    out = run(inp).cpu().numpy()
    v0 = np.repeat(inp["v"][0, :, 0], 5, axis=0)
    assert np.max(np.abs(out[0, :, 0] - v0)) <= 1e-6


def test_bf16_output():
    torch = require_gpu()
    inp = small(B=1, Hq=10, Hkv=2, S=256, lens=[256])
    r = ref(inp)
    out = run(inp, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(out - r) <= ATOL_BF16 + np.abs(r) * 2.0 ** -8)


@pytest.mark.parametrize("path", PATHS)
def test_deterministic_bitwise(path):
    inp = small(B=1, Hq=10, Hkv=2, S=384, lens=[384])
    g = gpu_inputs(inp)
    a = run(inp, g=g, path=path).cpu().numpy()
    b = run(inp, g=g, path=path).cpu().numpy()
    assert np.array_equal(a, b)


def test_paths_agree():
    # k' is rounded to fp16 the same way on both paths, but P is rounded to
    # fp16 against each path's own running maximum and the paths sum in
    # different orders, so the two differ by rounding noise well inside the
    # oracle bound
    inp = small(B=1, Hq=10, Hkv=2, S=256, lens=[256])
    a = run(inp, path="two_phase").cpu().numpy()
    b = run(inp, path="single_kernel").cpu().numpy()
    compare(a, b, ATOL_BF16, "two-phase vs single-kernel")


@pytest.mark.parametrize("path", PATHS)
def test_qwen3_prefill_s4096_sampled(path):
    # the full Qwen3-14B causal prefill (S = 4096, 40 / 8 heads), checked on
    # sampled heads and rows that span first, diagonal, ragged-tile and last rows
    w = synth.QWEN3_PREFILL
    log(f"case {w.name} {path}")
    inp = synth.make_prefill(w)
    out = run(inp, path=path).cpu().numpy()
    heads = [0, 4, 5, 17, 39]
    rows = np.array([0, 1, 63, 64, 127, 128, 129, 1000, 2047, 2048, 3071, 4094, 4095])
    r = ref(inp, heads=heads, rows=rows)
    compare(out[0][heads][:, rows], r[0][heads][:, rows], ATOL_BF16, "qwen3 prefill sampled")
    assert np.all(np.isfinite(out))


def test_prefill_last_row_matches_decode():
    # decode at L = S over a cache holding the oracle-transformed keys of rows
    # < S-1 equals prefill's last row (both on the GPU)
    torch = require_gpu()
    S = 256
    inp = small(B=1, Hq=10, Hkv=2, S=S, lens=[S], p0=50)
    pre = run(inp).cpu().numpy()
    pos = 50 + np.arange(S)
    kt = O.prologue(inp["k"][0], inp["k_norm_w"], pos, inp["rope_theta"], inp["eps"])
    cache = inp["k"].copy()
    cache[0, :, :S - 1] = synth.bf16_round(kt[:, :S - 1].astype(np.float32))
    bf = torch.bfloat16
    o = G.decode(dev(inp["q"][:, :, S - 1], bf), dev(cache, bf), dev(inp["v"], bf), ints([S]), ints([50 + S - 1]),
                 dev(inp["q_norm_w"], bf), dev(inp["k_norm_w"], bf), inp["rope_theta"], kv_split_tokens=64,
                 eps=inp["eps"])
    torch.cuda.synchronize()
    compare(o.cpu().numpy()[0], pre[0, :, S - 1], 5e-3, "prefill last row vs decode")
