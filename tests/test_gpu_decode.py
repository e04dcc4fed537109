"""GPU parity of gqa_attn_decode (through the C ABI) against the fp64 oracle.

Tolerances: max |err| <= 1e-5 for f32 inputs and <= 1e-2 for bf16 inputs
(f32 accumulation, f32 output); a bf16 output adds half a bf16 ulp of |ref|.
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL_F32 = 1e-5
ATOL_BF16 = 1e-2


def tdtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def gpu_inputs(inp, dtype):
    torch = require_gpu()
    dt = tdtype(dtype)
    return dict(q=dev(inp["q"], dt), k=dev(inp["k"], dt), v=dev(inp["v"], dt), qw=dev(inp["q_norm_w"], dt),
                kw=dev(inp["k_norm_w"], dt), sl=ints(inp["seq_lens"]), pos=ints(inp["positions"]))


def run(inp, dtype, split=0, out_dtype=None, g=None, out=None, workspace=None):
    torch = require_gpu()
    g = g or gpu_inputs(inp, dtype)
    o = G.decode(g["q"], g["k"], g["v"], g["sl"], g["pos"], g["qw"], g["kw"], inp["rope_theta"], out=out,
                 workspace=workspace, kv_split_tokens=split, eps=inp["eps"], out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    return o


def ref(inp):
    return O.decode_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["positions"], inp["q_norm_w"],
                        inp["k_norm_w"], inp["rope_theta"], inp["eps"])


def small(B=3, Hq=10, Hkv=2, S=300, dtype="bf16", lens=None, norm=True, theta=1e6, seed=11):
    w = synth.DecodeWorkload(f"small_decode_b{B}_h{Hq}_{Hkv}_s{S}", B, Hq, Hkv, S, dtype, norm, theta, 0,
                             seed=seed)
    inp = synth.make_decode(w)
    if lens is not None:
        inp["seq_lens"] = np.asarray(lens, dtype=np.int32)
        inp["positions"] = np.maximum(inp["seq_lens"], 1).astype(np.int32) - 1 + 7
        k, v = synth.make_decode(w, poison=False)["k"], synth.make_decode(w, poison=False)["v"]
        for b in range(B):
            L = max(0, min(int(lens[b]), S))
            k[b, :, L:] = np.nan
            v[b, :, L:] = np.nan
        inp["k"], inp["v"] = k, v
    return inp


# ------------------------------------------------------------------ the five workloads' decode shapes

def test_tiny_decode_f32_full():
    inp = synth.make_decode(synth.TINY_DECODE_F32)
    log(f"case {synth.TINY_DECODE_F32.name}")
    out = run(inp, "f32", split=synth.TINY_DECODE_F32.split_tokens)
    compare(out.cpu().numpy(), ref(inp), ATOL_F32, "tiny f32 decode")


def test_qwen3_decode_b1_s4096_full():
    w = synth.QWEN3_DECODE
    log(f"case {w.name}")
    inp = synth.make_decode(w)
    out = run(inp, w.dtype, split=w.split_tokens)
    compare(out.cpu().numpy(), ref(inp), ATOL_BF16, w.name)


def test_qwen3_ragged_b32_full():
    w = synth.QWEN3_RAGGED
    log(f"case {w.name}")
    inp = synth.make_decode(w)
    out = run(inp, w.dtype, split=w.split_tokens)
    compare(out.cpu().numpy(), ref(inp), ATOL_BF16, w.name)


def test_llama70b_long_decode_full():
    w = synth.LLAMA70B_LONG
    log(f"case {w.name}")
    inp = synth.make_decode(w)
    out = run(inp, w.dtype, split=w.split_tokens)
    compare(out.cpu().numpy(), ref(inp), ATOL_BF16, w.name)


# ------------------------------------------------------------------ shapes, splits, edge cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G_", [1, 2, 5, 8, 16])
def test_group_sizes(dtype, G_):
    Hkv = 2
    inp = small(B=2, Hq=G_ * Hkv, Hkv=Hkv, S=200, dtype=dtype, lens=[200, 77], seed=G_)
    log(f"case group={G_} dtype={dtype}")
    for split in (0, 64, 200):
        out = run(inp, dtype, split=split)
        compare(out.cpu().numpy(), ref(inp), ATOL_F32 if dtype == "f32" else ATOL_BF16, f"G={G_} split={split}")


@pytest.mark.parametrize("split", [32, 96, 100, 512])
def test_many_chunks_per_workgroup_ragged(split):
    # enough chunks that a partition workgroup sweeps several consecutive chunks
    # (split a multiple of 32), with lengths ending inside a workgroup's range;
    # split 100 keeps one chunk per workgroup
    inp = small(B=2, Hq=40, Hkv=8, S=4096, dtype="bf16", lens=[4096, 1000], seed=17)
    log(f"case many chunks split={split}")
    out = run(inp, "bf16", split=split)
    compare(out.cpu().numpy(), ref(inp), ATOL_BF16, f"many chunks split {split}")


@pytest.mark.parametrize("split", [1, 7, 32, 100, 128, 300, 1000])
def test_split_sweep_ragged(split):
    inp = small(B=3, Hq=10, Hkv=2, S=300, dtype="bf16", lens=[300, 133, 1])
    log(f"case split={split}")
    out = run(inp, "bf16", split=split)
    compare(out.cpu().numpy(), ref(inp), ATOL_BF16, f"split {split}")


def test_split_sweep_f32():
    inp = small(B=2, Hq=5, Hkv=1, S=513, dtype="f32", lens=[513, 65])
    r = ref(inp)
    for split in (0, 1, 31, 33, 64, 513):
        out = run(inp, "f32", split=split)
        compare(out.cpu().numpy(), r, ATOL_F32, f"f32 split {split}")


def test_empty_and_clamped_lengths():
    inp = small(B=4, Hq=10, Hkv=2, S=96, dtype="bf16", lens=[0, 96, 5, 96])
    inp["seq_lens"] = np.array([0, 96, 5, 1000], dtype=np.int32)   # 1000 is clamped to 96
    for split in (0, 32, 96):
        out = run(inp, "bf16", split=split).cpu().numpy()
        assert np.all(out[0] == 0.0)
        compare(out, ref(inp), ATOL_BF16, f"empty/clamped split {split}")


@pytest.mark.parametrize("B,Hq,Hkv,S,split,dtype", [
    (72, 8, 8, 256, 64, "bf16"),    # 576 groups: 72 per XCD, the 4-wave form
    (72, 8, 8, 256, 64, "f32"),
    (67, 5, 1, 128, 32, "bf16"),    # 67 groups, not a multiple of 8: groups served in order
    (9, 40, 8, 2048, 128, "bf16"),  # several chunks per workgroup
])
def test_live_ranges_first_grid(B, Hq, Hkv, S, split, dtype):
    """The partition grid serves the key ranges that hold keys first, found on
    the device by a prefix sum over the groups' lengths (in passes of 64
    groups): empty sequences, lengths on and off chunk boundaries, more than
    64 groups per pass."""
    rng = np.random.default_rng(B * 1000 + S)
    lens = rng.integers(0, S + 1, size=B)
    lens[::7] = 0
    lens[1::5] = split * rng.integers(1, S // split + 1, size=len(lens[1::5]))   # whole chunks
    lens[2::11] = S
    inp = small(B=B, Hq=Hq, Hkv=Hkv, S=S, dtype=dtype, lens=lens.tolist(), seed=B)
    log(f"case live-first grid B={B} Hkv={Hkv} S={S} split={split} {dtype}")
    out = run(inp, dtype, split=split).cpu().numpy()
    assert np.all(out[lens == 0] == 0.0)
    compare(out, ref(inp), ATOL_F32 if dtype == "f32" else ATOL_BF16, f"live-first B={B} split={split}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [0, 1, 31, 128, 129, 1000, 2047, 2048])
def test_single_sequence_lengths(dtype, L):
    """A batch of one maps its partition workgroups statically (KV head, chunk
    range) and returns those past the length: empty, one-key, partial-step,
    chunk-boundary and full lengths, unsplit, single-chunk and multi-chunk
    workgroups (split 32 over 2048 keys: several chunks per workgroup)."""
    inp = small(B=1, Hq=40, Hkv=8, S=2048, dtype=dtype, lens=[L], seed=L + 5)
    r = ref(inp)
    for split in (0, 32, 128, 2048):
        log(f"case single sequence L={L} split={split} {dtype}")
        out = run(inp, dtype, split=split).cpu().numpy()
        if L == 0:
            assert np.all(out == 0.0)
        compare(out, r, ATOL_F32 if dtype == "f32" else ATOL_BF16, f"B=1 L={L} split={split}")


@pytest.mark.parametrize("norm,theta", [(False, 0.0), (True, 0.0), (False, 5e5)])
def test_prologue_switches(norm, theta):
    for dtype in ("f32", "bf16"):
        inp = small(B=2, Hq=16, Hkv=2, S=160, dtype=dtype, lens=[160, 40], norm=norm, theta=theta)
        out = run(inp, dtype, split=64)
        compare(out.cpu().numpy(), ref(inp), ATOL_F32 if dtype == "f32" else ATOL_BF16, f"norm={norm} theta={theta} {dtype}")


def test_large_positions_rope_precision():
    # positions far beyond the cache length: angles up to ~131071 rad must be exact enough
    inp = small(B=2, Hq=8, Hkv=1, S=64, dtype="f32", lens=[64, 64], theta=5e5)
    inp["positions"] = np.array([131071, 100003], dtype=np.int32)
    out = run(inp, "f32", split=0)
    compare(out.cpu().numpy(), ref(inp), ATOL_F32, "large positions f32")


def test_bf16_output():
    torch = require_gpu()
    inp = small(B=2, Hq=10, Hkv=2, S=256, dtype="bf16", lens=[256, 100])
    r = ref(inp)
    out = run(inp, "bf16", split=64, out_dtype=torch.bfloat16).float().cpu().numpy()
    tol = ATOL_BF16 + np.abs(r) * 2.0 ** -8
    assert np.all(np.abs(out - r) <= tol)


def test_ones_value_column_pin():
    # one V column of ones: that output column is sum_j p_j = 1
    for dtype, tol in (("f32", 1e-6), ("bf16", 3e-3)):
        inp = small(B=2, Hq=10, Hkv=2, S=300, dtype=dtype, lens=[300, 45])
        inp["v"][:, :, :, 17] = np.where(np.isnan(inp["v"][:, :, :, 17]), np.nan, 1.0)
        out = run(inp, dtype, split=64).cpu().numpy()
        err = np.abs(out[:, :, 17] - 1.0).max()
        log(f"  ones column {dtype}: {err:.2e}")
        assert err <= tol


def test_deterministic_bitwise():
    inp = small(B=2, Hq=40, Hkv=8, S=1024, dtype="bf16", lens=[1024, 999])
    g = gpu_inputs(inp, "bf16")
    a = run(inp, "bf16", split=128, g=g).cpu().numpy()
    b = run(inp, "bf16", split=128, g=g).cpu().numpy()
    assert np.array_equal(a, b)


def test_poisoned_workspace_and_output_canaries():
    torch = require_gpu()
    inp = small(B=2, Hq=10, Hkv=2, S=300, dtype="bf16", lens=[300, 123])
    g = gpu_inputs(inp, "bf16")
    desc = G.decode_desc(g["q"], g["k"], g["v"], torch.empty(2, 10, 128, device="cuda"), kv_split_tokens=64)
    ws = G.decode_workspace(desc, "cuda")
    ws.view(torch.float32).fill_(float("nan"))
    # out lives inside a larger buffer whose other elements are canaries
    big = torch.full((2, 12, 160), 12345.0, device="cuda")
    out = big[:, 1:11, 16:144]
    run(inp, "bf16", split=64, g=g, out=out, workspace=ws)
    got = big.cpu().numpy()
    compare(got[:, 1:11, 16:144], ref(inp), ATOL_BF16, "strided out, NaN workspace")
    mask = np.ones_like(got, dtype=bool)
    mask[:, 1:11, 16:144] = False
    assert np.all(got[mask] == 12345.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_workspace_reuse_across_lengths(dtype):
    # one workspace, successive calls whose lengths change the number of
    # chunks per sequence: stale partials of earlier calls must not leak in
    torch = require_gpu()
    inp = small(B=3, Hq=10, Hkv=2, S=512, dtype=dtype)   # every cache row holds data
    g = gpu_inputs(inp, dtype)
    desc = G.decode_desc(g["q"], g["k"], g["v"], torch.empty(3, 10, 128, device="cuda"), kv_split_tokens=32)
    ws = G.decode_workspace(desc, "cuda")
    tol = ATOL_F32 if dtype == "f32" else ATOL_BF16
    for lens in ([512, 200, 3], [33, 480, 64], [1, 1, 511], [512, 0, 96]):
        case = dict(inp)
        case["seq_lens"] = np.array(lens, dtype=np.int32)
        case["positions"] = np.maximum(case["seq_lens"], 1) - 1 + 3
        g2 = dict(g, sl=ints(case["seq_lens"]), pos=ints(case["positions"]))
        out = run(case, dtype, split=32, g=g2, workspace=ws)
        compare(out.cpu().numpy(), ref(case), tol, f"reuse lens={lens}")


def test_decode_equals_partition_then_merge():
    # gqa_attn_decode against gqa_attn_decode_partition + gqa_attn_decode_merge: bitwise equal
    torch = require_gpu()
    inp = small(B=2, Hq=16, Hkv=2, S=1000, dtype="bf16", lens=[1000, 555])
    g = gpu_inputs(inp, "bf16")
    a = run(inp, "bf16", split=64, g=g).cpu().numpy()
    out = torch.empty(2, 16, 128, device="cuda")
    desc = G.decode_desc(g["q"], g["k"], g["v"], out, kv_split_tokens=64)
    ws = G.decode_workspace(desc, "cuda")
    p = lambda x: None if x is None else x.data_ptr()
    args = (desc, p(g["q"]), p(g["k"]), p(g["v"]), p(g["sl"]), p(g["pos"]), p(g["qw"]), p(g["kw"]),
            inp["rope_theta"], p(out), p(ws), ws.numel())
    assert G.gqa_attn_decode_partition(*args, None) == G.GQA_OK
    assert G.gqa_attn_decode_merge(desc, p(g["sl"]), p(out), p(ws), ws.numel(), None) == G.GQA_OK
    torch.cuda.synchronize()
    assert np.array_equal(a, out.cpu().numpy())
    compare(a, ref(inp), ATOL_BF16, "decode vs oracle")


def test_token_major_cache_layout_and_strided_q():
    # caches stored [B, S, Hkv, d] (strides b, h, s = S*Hkv*d, d, Hkv*d); q with a padded head stride
    torch = require_gpu()
    inp = small(B=2, Hq=10, Hkv=2, S=200, dtype="bf16", lens=[200, 61])
    kt = dev(np.ascontiguousarray(inp["k"].transpose(0, 2, 1, 3)), torch.bfloat16).permute(0, 2, 1, 3)
    vt = dev(np.ascontiguousarray(inp["v"].transpose(0, 2, 1, 3)), torch.bfloat16).permute(0, 2, 1, 3)
    qpad = torch.zeros(2, 10, 136, dtype=torch.bfloat16, device="cuda")
    qpad[:, :, :128] = dev(inp["q"], torch.bfloat16)
    q = qpad[:, :, :128]
    g = dict(q=q, k=kt, v=vt, qw=dev(inp["q_norm_w"], torch.bfloat16), kw=dev(inp["k_norm_w"], torch.bfloat16),
             sl=ints(inp["seq_lens"]), pos=ints(inp["positions"]))
    out = run(inp, "bf16", split=64, g=g)
    compare(out.cpu().numpy(), ref(inp), ATOL_BF16, "token-major cache")
