"""GPU checks of the split-KV partials and their log-sum-exp merge (ADR-0060
section 4) in gqa_attn_decode: each partition workgroup writes one partial per
query head of its group (the merge of the chunks it swept, folded in registers
when it sweeps several), and the merge kernel combines the partials of the
workgroups that hold keys.

Checked: parity with the fp64 oracle over plans that exercise the merge
kernel (16 groups of 32 lanes over up to 64 partials per head, G = 1 .. 16)
and the in-workgroup fold (workgroups that sweep 4 chunks), sequences with no
key or a single partial; the two-launch form (partition, then merge) equals
gqa_attn_decode bitwise; repeated calls and HIP-graph replays are bitwise
equal.  Tolerances as for decode: 1e-5 (f32 inputs), 1e-2 (bf16 inputs).
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL = {"f32": 1e-5, "bf16": 1e-2}


def make(B, Hq, Hkv, S, dtype, lens, seed=91, norm=True, theta=1e6):
    w = synth.DecodeWorkload(f"merge_b{B}_h{Hq}_{Hkv}_s{S}", B, Hq, Hkv, S, dtype, norm, theta, 0, seed=seed)
    inp = synth.make_decode(w, poison=False)
    inp["seq_lens"] = np.asarray(lens, dtype=np.int32)
    inp["positions"] = (np.maximum(inp["seq_lens"], 1) - 1 + 5).astype(np.int32)
    for b, L in enumerate(inp["seq_lens"]):   # rows past a length are never read
        L = max(0, min(int(L), S))
        inp["k"][b, :, L:] = np.nan
        inp["v"][b, :, L:] = np.nan
    return inp


def tdtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


class Case:
    """Device tensors, a zeroed workspace and the raw C-ABI arguments of one decode."""

    def __init__(self, inp, dtype, split):
        torch = require_gpu()
        dt = tdtype(dtype)
        self.inp = inp
        self.q, self.k, self.v = dev(inp["q"], dt), dev(np.nan_to_num(inp["k"]), dt), dev(np.nan_to_num(inp["v"]), dt)
        self.qw, self.kw = dev(inp["q_norm_w"], dt), dev(inp["k_norm_w"], dt)
        self.sl, self.pos = ints(inp["seq_lens"]), ints(inp["positions"])
        B, Hq = inp["q"].shape[:2]
        self.out = torch.full((B, Hq, 128), 777.0, device="cuda")
        self.desc = G.decode_desc(self.q, self.k, self.v, self.out, kv_split_tokens=split, eps=inp["eps"])
        self.ws = G.decode_workspace(self.desc, "cuda")
        st, self.T, self.n = G.gqa_attn_decode_plan(self.desc)
        assert st == G.GQA_OK

    def args(self):
        p = lambda t: None if t is None else t.data_ptr()
        return (self.desc, p(self.q), p(self.k), p(self.v), p(self.sl), p(self.pos), p(self.qw), p(self.kw),
                self.inp["rope_theta"], p(self.out), p(self.ws), 0 if self.ws is None else self.ws.numel())

    def decode(self, stream):
        assert G.gqa_attn_decode(*self.args(), stream) == G.GQA_OK

    def ref(self):
        i = self.inp
        return O.decode_ref(i["q"], i["k"], i["v"], i["seq_lens"], i["positions"], i["q_norm_w"], i["k_norm_w"],
                            i["rope_theta"], i["eps"])


# (B, Hq, Hkv, S, split, lens): G = 1, 3, 5, 8, 16; partial counts from 1 to 64
# per head (64 partials: four per 32-lane group of the merge kernel); the
# 20 / 4 heads case sweeps 4 chunks per workgroup; L = 0 and L inside the
# first chunk
SHAPES = [
    (2, 2, 2, 4096, 64, [4096, 1000]),
    (2, 6, 2, 4096, 64, [4096, 65]),
    (4, 20, 4, 4096, 64, [4096, 0, 1, 2049]),
    (2, 16, 2, 4096, 64, [4096, 513]),
    (2, 32, 2, 4096, 64, [4096, 64]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"b{s[0]}_h{s[1]}_{s[2]}_T{s[4]}")
def test_decode_merge_parity(shape, dtype):
    B, Hq, Hkv, S, split, lens = shape
    c = Case(make(B, Hq, Hkv, S, dtype, lens), dtype, split)
    log(f"case merge {dtype} B={B} Hq={Hq} Hkv={Hkv} T={c.T} n={c.n}")
    torch = require_gpu()
    c.decode(None)
    torch.cuda.synchronize()
    compare(c.out.cpu().numpy(), c.ref(), ATOL[dtype], f"merge {dtype} Hq={Hq}")


def test_workgroups_sweeping_several_chunks():
    # one (sequence, KV head) group over 32768 keys in 32-key chunks: each
    # partition workgroup folds 4 chunks in registers (1024 chunks, 256
    # workgroups), and the merge kernel combines 256 partials per head
    c = Case(make(1, 8, 1, 32768, "bf16", [32768], seed=92), "bf16", 32)
    log(f"case merge multi-chunk T={c.T} n={c.n}")
    torch = require_gpu()
    c.decode(None)
    torch.cuda.synchronize()
    compare(c.out.cpu().numpy(), c.ref(), ATOL["bf16"], "multi-chunk workgroups")
    one = c.out.cpu().numpy()
    # the two-launch form: the same kernels
    c.out.fill_(777.0)
    a = c.args()
    assert G.gqa_attn_decode_partition(*a, None) == G.GQA_OK
    assert G.gqa_attn_decode_merge(a[0], a[4], a[9], a[10], a[11], None) == G.GQA_OK
    torch.cuda.synchronize()
    assert np.array_equal(one, c.out.cpu().numpy())


def test_repeated_calls_and_graph_replays_bitwise():
    torch = require_gpu()
    c = Case(make(3, 10, 2, 2048, "bf16", [2048, 700, 33], seed=93), "bf16", 64)
    log(f"case merge repeat/graph T={c.T} n={c.n}")
    c.decode(None)
    torch.cuda.synchronize()
    first = c.out.clone()
    compare(first.cpu().numpy(), c.ref(), ATOL["bf16"], "first call")
    for _ in range(20):
        c.out.fill_(777.0)
        c.decode(None)
    torch.cuda.synchronize()
    assert torch.equal(c.out, first), "repeated call differs"
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        c.decode(s.cuda_stream)
    for r in range(4):
        c.out.fill_(777.0)      # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.out, first), f"graph replay {r} differs"


def test_paged_equals_contiguous_with_folded_chunks():
    # 256 chunks of 32 keys over 2 KV heads: 2 chunks per workgroup on both paths
    torch = require_gpu()
    inp = make(1, 16, 2, 8192, "bf16", [8000], seed=94)
    c = Case(inp, "bf16", 32)
    assert c.n == 256
    c.decode(None)
    torch.cuda.synchronize()
    bs = 64
    nb = 8192 // bs
    rng = np.random.default_rng(5)
    perm = rng.permutation(nb)
    table = perm.reshape(1, nb).astype(np.int32)
    kc, vc = np.nan_to_num(inp["k"]), np.nan_to_num(inp["v"])
    kp = np.zeros((nb, 2, bs, 128), dtype=np.float32)
    vp = np.zeros_like(kp)
    for b in range(1):
        for i in range(nb):
            kp[table[b, i]] = kc[b][:, i * bs:(i + 1) * bs]
            vp[table[b, i]] = vc[b][:, i * bs:(i + 1) * bs]
    bfd = torch.bfloat16
    out = G.decode_paged(dev(inp["q"], bfd), dev(kp, bfd), dev(vp, bfd), ints(table), ints(inp["seq_lens"]),
                         ints(inp["positions"]), dev(inp["q_norm_w"], bfd), dev(inp["k_norm_w"], bfd),
                         inp["rope_theta"], kv_split_tokens=32, eps=inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(out, c.out), "paged decode differs from contiguous"
    compare(out.cpu().numpy(), c.ref(), ATOL["bf16"], "paged, folded chunks")
