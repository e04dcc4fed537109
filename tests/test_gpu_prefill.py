"""GPU parity of gqa_attn_prefill (through the C ABI) against the fp64 oracle.

bf16 inputs, fp16 MFMA operands (q', k', P rounded to fp16, v converted
exactly), f32 accumulation, f32 output: max |err| <= 1e-2.
"""

import math

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
@pytest.mark.parametrize("theta", [1e6, 5e5])
def test_large_positions(theta, path):
    # RoPE angles of queries and keys up to ~130159 rad: the product and its
    # reduction to revolutions in double on both sides
    inp = small(B=2, Hq=10, Hkv=2, S=160, lens=[160, 100], theta=theta)
    inp["positions"] = np.array([130000, 65537], dtype=np.int32)
    log(f"case prefill large positions theta={theta} {path}")
    out = run(inp, path=path).cpu().numpy()
    compare(valid_rows(out, inp), ref(inp), ATOL_BF16, f"large positions theta={theta} {path}")


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


def test_phases_equal_prefill_and_attend_replays():
    # keys then attend is the two-phase prefill bitwise; the attention phase
    # repeated over one key phase gives the same output every time, also for
    # a plan that splits key ranges (8 query heads x 16 blocks = 128 items:
    # two spans per long block, whose arrival counters return to zero)
    torch = require_gpu()
    for B, Hq, Hkv, S in ((1, 10, 2, 384), (1, 8, 1, 2048)):
        inp = small(B=B, Hq=Hq, Hkv=Hkv, S=S, lens=[S])
        g = gpu_inputs(inp)
        log(f"case prefill phases B={B} Hq={Hq} Hkv={Hkv} S={S}")
        whole = run(inp, g=g).cpu().numpy()
        out = torch.full((B, Hq, S, 128), float("nan"), device="cuda")
        desc = G.prefill_desc(g["q"], g["k"], g["v"], out, True, inp["eps"])
        ws = G.prefill_workspace(desc, "cuda")
        args = lambda: (desc, g["q"].data_ptr(), g["k"].data_ptr(), g["v"].data_ptr(), g["sl"].data_ptr(),
                        g["pos"].data_ptr(), g["qw"].data_ptr(), g["kw"].data_ptr(), inp["rope_theta"],
                        out.data_ptr(), ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
        assert G.gqa_attn_prefill_keys(*args()) == G.GQA_OK
        for rep in range(3):
            out.fill_(float("nan"))
            assert G.gqa_attn_prefill_attend(*args()) == G.GQA_OK
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), whole), f"attend replay {rep} differs"
        compare(whole, ref(inp), ATOL_BF16, f"phases S={S}")


@pytest.mark.parametrize("path", PATHS)
def test_fp16_range_saturates_v(path):
    # v enters the P V products in fp16: elements beyond +-65504 saturate, and
    # the call returns the oracle's result for v clamped to that range.  Every
    # key row is the same, so every score of a row is the same, P = 1 for
    # every visible key and out is the running mean of v, free of the fp16
    # rounding of q', k' and P.  59904 (bf16-exact) is inside the range,
    # -70144 and 70144 are not.
    inp = small(B=1, Hq=10, Hkv=2, S=160, lens=[160], norm=False, theta=0.0)
    inp["k"][0] = inp["k"][0][:, :1]
    inp["v"][0, 0, 0, 3] = 59904.0
    inp["v"][0, 1, 0, 7] = -70144.0
    inp["v"][0, 1, 40, 9] = 70144.0
    clamped = dict(inp, v=np.clip(inp["v"], -65504.0, 65504.0))
    log(f"case fp16 range of v, {path}")
    out = run(inp, path=path).cpu().numpy()
    assert np.all(np.isfinite(out))
    # row 0 sees key 0 alone: the stored value, saturated where out of range
    assert np.allclose(out[0, 0:5, 0, 3], 59904.0, rtol=1e-6, atol=0)
    assert np.allclose(out[0, 5:10, 0, 7], -65504.0, rtol=1e-6, atol=0)
    compare(out, ref(clamped), ATOL_BF16, f"saturated v {path}")


@pytest.mark.parametrize("path", PATHS)
def test_fp16_range_saturates_k(path):
    # k' enters QK^T in fp16: an element beyond +-65504 saturates, and the call
    # returns the oracle's result for k clamped to that range.  Key 9 of KV
    # head 1 has the element 70144 in dim 11; the queries of that head have
    # q[11] = +-1, so key 9 scores about +-8000 (log2 units) against every
    # query that sees it: weight 1 or 0 to all digits.
    inp = small(B=1, Hq=10, Hkv=2, S=160, lens=[160], norm=False, theta=0.0)
    inp["k"][0, 1, 9, 11] = 70144.0
    inp["q"][0, 5:8, :, 11] = 1.0
    inp["q"][0, 8:10, :, 11] = -1.0
    clamped = dict(inp, k=np.clip(inp["k"], -65504.0, 65504.0))
    log(f"case fp16 range of k, {path}")
    out = run(inp, path=path).cpu().numpy()
    want = ref(clamped)
    # rows that see key 9 with q[11] = +1 are v[9] (both paths divide the P V
    # products by the sum of the same fp16 P)
    assert np.allclose(out[0, 5:8, 9:], np.broadcast_to(inp["v"][0, 1, 9], (3, 151, 128)), rtol=2.0 ** -10,
                       atol=1e-6)
    compare(out, want, ATOL_BF16, f"saturated k {path}")


@pytest.mark.parametrize("path", PATHS)
def test_fp16_range_saturates_q(path):
    # q' = q * scale * log2(e) (no norm) enters QK^T in fp16: q[11] = +-2^20
    # gives q'[11] = +-133712, which saturates to +-65504, so the call returns
    # the oracle's result for q[11] = +-65504 / (scale log2 e).  In KV head 1
    # only key 9 has a nonzero dim 11 (1.0): it takes all the weight of the
    # rows with q[11] = +2^20 that see it and none of those with -2^20.  An
    # unsaturated q' would be +-inf, and inf * 0 makes those rows NaN.
    inp = small(B=1, Hq=10, Hkv=2, S=160, lens=[160], norm=False, theta=0.0)
    inp["k"][0, 1, :, 11] = 0.0
    inp["k"][0, 1, 9, 11] = 1.0
    inp["q"][0, 5:8, :, 11] = 2.0 ** 20
    inp["q"][0, 8:10, :, 11] = -(2.0 ** 20)
    lim = 65504.0 / ((1.0 / math.sqrt(128.0)) * math.log2(math.e))
    clamped = dict(inp, q=np.clip(inp["q"], -lim, lim))
    log(f"case fp16 range of q, {path}")
    out = run(inp, path=path).cpu().numpy()
    assert np.all(np.isfinite(out))
    assert np.allclose(out[0, 5:8, 9:], np.broadcast_to(inp["v"][0, 1, 9], (3, 151, 128)), rtol=2.0 ** -10,
                       atol=1e-6)
    compare(out, ref(clamped), ATOL_BF16, f"saturated q {path}")


# ---- the full Qwen3-14B causal prefill (S = 4096, 40 query heads over 8 KV
# heads): every element of out against the oracle.  out starts as NaN, so a
# block the kernels leave unwritten fails.  The GPU output is computed once
# per path; the oracle once per KV group (5 query heads each) and shared by
# both paths.

_QWEN3 = {}


def qwen3_inputs():
    if "inp" not in _QWEN3:
        _QWEN3["inp"] = synth.make_prefill(synth.QWEN3_PREFILL)
    return _QWEN3["inp"]


def qwen3_oracle_group(kv):
    key = ("ref", kv)
    if key not in _QWEN3:
        heads = list(range(5 * kv, 5 * kv + 5))
        _QWEN3[key] = ref(qwen3_inputs(), heads=heads)[0, heads]
    return _QWEN3[key]


@pytest.fixture(scope="module", params=PATHS)
def qwen3_gpu(request):
    torch = require_gpu()
    inp = qwen3_inputs()
    log(f"case {synth.QWEN3_PREFILL.name} {request.param} (out pre-filled with NaN)")
    out = torch.full(inp["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    run(inp, out=out, path=request.param)
    return request.param, out.cpu().numpy()


@pytest.mark.parametrize("kv", range(8))
def test_qwen3_prefill_s4096_full(qwen3_gpu, kv):
    path, out = qwen3_gpu
    heads = list(range(5 * kv, 5 * kv + 5))
    compare(out[0, heads], qwen3_oracle_group(kv), ATOL_BF16, f"qwen3 prefill {path} KV group {kv} (heads {heads[0]}-{heads[-1]}, all rows)")


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
