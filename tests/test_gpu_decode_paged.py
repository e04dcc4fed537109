"""GPU parity of gqa_attn_decode_paged (through the C ABI) against the fp64
paged-decode oracle, and bitwise against the contiguous decode of the same
logical cache (paging only changes addresses; with the same chunk length the
arithmetic is identical).  Physical pages are shuffled; table entries past a
sequence's last block are -1 and page rows past its length are NaN, so any
read of them shows up.  Tolerances as for decode: 1e-5 (f32), 1e-2 (bf16).
"""

import numpy as np
import pytest

import gqa_attention_attn_amd as G
import oracle as O
import synth
from gpu_util import compare, dev, ints, log, require_gpu

pytestmark = pytest.mark.gpu

ATOL = {"f32": 1e-5, "bf16": 1e-2}


def tdtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def paged(B, Hq, Hkv, S, bs, dtype, lens, seed=71, norm=True, theta=1e6, spare=3):
    """Inputs with a shuffled page pool of B * S / bs + spare pages."""
    rng = np.random.default_rng(seed)
    rnd = lambda *sh: rng.standard_normal(sh).astype(np.float32)
    cast = (lambda x: synth.bf16_round(x)) if dtype == "bf16" else (lambda x: x)
    nb = S // bs
    npages = B * nb + spare
    kp, vp = cast(rnd(npages, Hkv, bs, 128)), cast(rnd(npages, Hkv, bs, 128))
    perm = rng.permutation(npages)[:B * nb]
    table = perm.reshape(B, nb).astype(np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    for b in range(B):
        L = int(min(max(lens[b], 0), S))
        used = -(-L // bs)
        if used:
            last = table[b, used - 1]
            kp[last, :, L - (used - 1) * bs:] = np.nan
            vp[last, :, L - (used - 1) * bs:] = np.nan
        table[b, used:] = -1
    return dict(q=cast(rnd(B, Hq, 128)), kp=kp, vp=vp, table=table, lens=lens,
                pos=(np.maximum(lens, 1) - 1 + 5).astype(np.int32), gq=cast(1 + 0.1 * rnd(128)) if norm else None,
                gk=cast(1 + 0.1 * rnd(128)) if norm else None, theta=theta, bs=bs, S=S)


def run_paged(c, dtype, split=0, kp=None, write=False):
    torch = require_gpu()
    dt = tdtype(dtype)
    o = G.decode_paged(dev(c["q"], dt), kp if kp is not None else dev(c["kp"], dt), dev(c["vp"], dt),
                       ints(c["table"]), ints(c["lens"]), ints(c["pos"]), dev(c["gq"], dt), dev(c["gk"], dt),
                       c["theta"], kv_split_tokens=split, write_new_k=write)
    torch.cuda.synchronize()
    return o.cpu().numpy()


def ref(c):
    return O.decode_paged_ref(c["q"], c["kp"], c["vp"], c["table"], c["lens"], c["pos"], c["gq"], c["gk"],
                              c["theta"], block_size=c["bs"])


def gathered(c):
    K = O.paged_gather(c["kp"], c["table"], c["lens"], c["bs"], c["S"])
    V = O.paged_gather(c["vp"], c["table"], c["lens"], c["bs"], c["S"])
    return K, V


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [32, 64, 256])
@pytest.mark.parametrize("split", [0, 100, 512])
def test_paged_decode_parity_and_bitwise(dtype, bs, split):
    torch = require_gpu()
    c = paged(B=4, Hq=10, Hkv=2, S=1024, bs=bs, dtype=dtype, lens=[1024, 1, 0, 300])
    log(f"case paged decode {dtype} bs={bs} split={split}")
    out = run_paged(c, dtype, split)
    compare(out, ref(c), ATOL[dtype], f"paged {dtype} bs={bs} split={split}")
    # the contiguous decode of the gathered cache with the same (rounded) chunk length
    K, V = gathered(c)
    dt = tdtype(dtype)
    T = 0 if split == 0 else -(-split // 32) * 32
    cont = G.decode(dev(c["q"], dt), dev(np.nan_to_num(K), dt), dev(np.nan_to_num(V), dt), ints(c["lens"]),
                    ints(c["pos"]), dev(c["gq"], dt), dev(c["gk"], dt), c["theta"], kv_split_tokens=T)
    torch.cuda.synchronize()
    assert np.array_equal(out, cont.cpu().numpy()), "paged and contiguous decode differ"


def test_paged_many_chunks_per_workgroup():
    # 2 groups: chunks are swept several per workgroup across page boundaries
    c = paged(B=1, Hq=10, Hkv=2, S=8192, bs=64, dtype="bf16", lens=[8000], seed=72)
    for split in (64, 96, 512):
        compare(run_paged(c, "bf16", split), ref(c), ATOL["bf16"], f"paged multi-chunk split={split}")


@pytest.mark.parametrize("L", [0, 1, 65, 3000, 4096])
def test_paged_single_sequence_lengths(L):
    # a batch of one: workgroups past the length return before any page is
    # looked up (table entries past the last block are -1)
    c = paged(B=1, Hq=40, Hkv=8, S=4096, bs=64, dtype="bf16", lens=[L], seed=75 + L)
    for split in (0, 128, 512):
        log(f"case paged single sequence L={L} split={split}")
        out = run_paged(c, "bf16", split)
        if L == 0:
            assert np.all(out == 0.0)
        compare(out, ref(c), ATOL["bf16"], f"paged B=1 L={L} split={split}")


def test_paged_write_new_k_lands_in_its_page():
    torch = require_gpu()
    c = paged(B=3, Hq=10, Hkv=2, S=512, bs=64, dtype="bf16", lens=[512, 65, 64], seed=73)
    kp = dev(c["kp"], torch.bfloat16)
    before = kp.float().cpu().numpy()
    a = run_paged(c, "bf16", kp=kp, write=True)
    compare(a, ref(c), ATOL["bf16"], "paged write_new_k")
    after = kp.float().cpu().numpy()
    changed = np.zeros(after.shape[:1] + after.shape[2:3], dtype=bool)   # (page, row)
    for b, L in enumerate(c["lens"]):
        page, row = c["table"][b, (L - 1) // 64], (L - 1) % 64
        want = O.prologue(c["kp"][page][:, row:row + 1], c["gk"], np.array([int(c["pos"][b])]), c["theta"], 1e-6)
        err = np.abs(after[page][:, row] - want[:, 0])
        assert np.all(err <= 2.0 ** -8 * np.abs(want[:, 0]) + 1e-5)
        changed[page, row] = True
    same = np.where(np.isnan(before), np.isnan(after), before == after)
    assert np.all(same.transpose(0, 2, 1, 3)[~changed]), "a row other than the new keys changed"


def test_paged_llama70b_shape_s16384():
    # Llama3-70B-shaped heads (64 / 8, no QK-norm, theta 5e5) over a 16K paged cache
    c = paged(B=1, Hq=64, Hkv=8, S=16384, bs=256, dtype="bf16", lens=[16384], seed=74, norm=False, theta=5e5)
    log("case paged llama70b-shaped S=16384")
    compare(run_paged(c, "bf16", 512), ref(c), ATOL["bf16"], "paged llama70b s16384")
