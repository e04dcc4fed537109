"""GPU parity of the two-phase prefill when the attention grid splits the key
range of long query blocks over several workgroups ("ADR-0060: AHBM GQA Fused
Attention Kernel (Llama3-70B)" section 4: partials of disjoint key ranges
combine by the log-sum-exp merge; the last workgroup of a block merges).

The split is taken when the grid has fewer than 384 workgroups (a single
sequence or few heads here), with key spans of at least 16 tiles of 32 keys;
blocks that see more keys than one span are split.  Checked against the fp64 oracle on every
output element (bf16 inputs, fp16 products, f32 accumulation: max |err| <=
1e-2), against the single-kernel path (which never splits), bitwise between
repeated calls (the merge order is fixed), and bitwise between the contiguous
and paged chunked forms.
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def make(B, Hq, Hkv, S, lens, causal=True, seed=81):
    w = synth.PrefillWorkload(f"split_prefill_b{B}_h{Hq}_{Hkv}_s{S}", B, Hq, Hkv, S, "bf16", True, 1e6,
                              causal=causal, position0=3, seed=seed)
    inp = synth.make_prefill(w, poison=False)
    inp["seq_lens"] = np.asarray(lens, dtype=np.int32)
    for b in range(B):
        n = max(0, min(int(lens[b]), S))
        for key in ("q", "k", "v"):
            inp[key][b, :, n:] = np.nan
    return inp


def run(inp, workspace="auto"):
    torch = require_gpu()
    bf = torch.bfloat16
    o = G.prefill(dev(inp["q"], bf), dev(inp["k"], bf), dev(inp["v"], bf), ints(inp["seq_lens"]),
                  ints(inp["positions"]), dev(inp["q_norm_w"], bf), dev(inp["k_norm_w"], bf), inp["rope_theta"],
                  causal=inp["causal"], eps=inp["eps"], workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def ref(inp):
    return O.prefill_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["positions"], inp["q_norm_w"],
                         inp["k_norm_w"], inp["rope_theta"], inp["eps"], causal=inp["causal"])


def valid(out, lens):
    o = out.copy()
    for b, n in enumerate(lens):
        o[b, :, n:] = 0.0
    return o


def split_planned(B, Hq, Hkv, S, causal=True, max_chunk=0):
    """The workspace holds split partials exactly when the grid splits."""
    d = G.GqaPrefillDesc(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, max_seq=S, in_dtype=G.GQA_BF16,
                         out_dtype=G.GQA_F32, causal=int(causal), q_stride_b=Hq * S * 128, q_stride_h=S * 128,
                         q_stride_s=128, k_stride_b=Hkv * S * 128, k_stride_h=S * 128, k_stride_s=128,
                         v_stride_b=Hkv * S * 128, v_stride_h=S * 128, v_stride_s=128, out_stride_b=Hq * S * 128,
                         out_stride_h=S * 128, out_stride_s=128, eps=1e-6, scale=0.0, max_chunk=max_chunk)
    st, nbytes = G.gqa_attn_prefill_workspace_size(d)
    assert st == G.GQA_OK
    return nbytes > B * Hkv * (-(-S // 32)) * 9216 * 2


def test_causal_split_blocks_full_parity():
    # 2560 keys, 100 workgroups unsplit: spans of 32 tiles; query blocks 8..19
    # see 36..80 tiles and are split in two or three
    inp = make(1, 5, 1, 2560, [2560])
    assert split_planned(1, 5, 1, 2560)
    log("case split prefill causal S=2560")
    out = run(inp)
    compare(out, ref(inp), ATOL, "split causal S=2560")
    single = run(inp, workspace=None)
    compare(out, single, ATOL, "split vs single kernel")
    assert np.array_equal(out, run(inp)), "repeated call differs"


def test_noncausal_ragged_split_and_unsplit_sequences():
    # non-causal: every block of sequence 0 sees 80 tiles (three spans);
    # sequence 1 (1500 keys, 47 tiles) two spans; sequence 2 is empty
    lens = [2560, 1500, 0]
    inp = make(3, 4, 2, 2560, lens, causal=False, seed=82)
    assert split_planned(3, 4, 2, 2560, causal=False)
    log("case split prefill non-causal ragged")
    compare(valid(run(inp), lens), ref(inp), ATOL, "split non-causal ragged")


@pytest.mark.parametrize("paged", [False, True])
def test_chunk_after_long_prefix_split(paged):
    # 560 new tokens after 2000 cached ones: every block sees 67..80 tiles (three spans)
    torch = require_gpu()
    S, P, T = 2560, 2000, 560
    assert split_planned(1, 5, 1, S, max_chunk=T)
    rng = np.random.default_rng(83)
    bf = lambda x: synth.bf16_round(x.astype(np.float32))
    q = bf(rng.standard_normal((1, 5, T, 128)))
    k = bf(rng.standard_normal((1, 1, S, 128)))
    v = bf(rng.standard_normal((1, 1, S, 128)))
    gq, gk = bf(1 + 0.1 * rng.standard_normal(128)), bf(1 + 0.1 * rng.standard_normal(128))
    k[0, 0, :P] = bf(O.prologue(k[0, 0, :P], gk, 3 + np.arange(P), 1e6, 1e-6))
    past, chunk, pos = np.array([P], np.int32), np.array([T], np.int32), np.array([3], np.int32)
    bfd = torch.bfloat16
    log(f"case split chunk paged={paged}")
    cont = G.prefill_chunk(dev(q, bfd), dev(k, bfd), dev(v, bfd), ints(past), ints(chunk), ints(pos), dev(gq, bfd),
                           dev(gk, bfd), 1e6)
    torch.cuda.synchronize()
    want = O.prefill_chunk_ref(q, k, v, past, chunk, pos, gq, gk, 1e6)
    compare(cont.cpu().numpy(), want, ATOL, "split chunk")
    if paged:
        bs = 64
        nb = S // bs
        perm = np.random.default_rng(7).permutation(nb)
        kp = np.zeros((nb, 1, bs, 128), np.float32)
        vp = np.zeros_like(kp)
        for i in range(nb):
            kp[perm[i]] = k[0][:, i * bs:(i + 1) * bs]
            vp[perm[i]] = v[0][:, i * bs:(i + 1) * bs]
        out = G.prefill_chunk_paged(dev(q, bfd), dev(kp, bfd), dev(vp, bfd), ints(perm.reshape(1, nb)), ints(past),
                                    ints(chunk), ints(pos), dev(gq, bfd), dev(gk, bfd), 1e6)
        torch.cuda.synchronize()
        assert torch.equal(out, cont), "paged split chunk differs from contiguous"
