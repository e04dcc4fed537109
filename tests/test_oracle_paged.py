"""Pins for the paged-cache decode oracle (paged_gather + decode_paged_ref):
paging is addressing only, so a paged cache must give exactly the decode of
the logical cache its block table describes.  Pinned by a scalar-loop
gather into the scalar brute-force decode, by the identity layout against
the contiguous decode, by invariance under a permutation of the physical
pages, and by ignoring table entries past each sequence's last block.
"""

import numpy as np

import oracle as O


def paged_case(B=3, Hq=4, Hkv=2, bs=4, nb=5, d=8, lens=(20, 7, 1), seed=0):
    rng = np.random.default_rng(seed)
    S = nb * bs
    k = rng.standard_normal((B, Hkv, S, d))
    v = rng.standard_normal((B, Hkv, S, d))
    q = rng.standard_normal((B, Hq, d))
    gq, gk = 1 + 0.1 * rng.standard_normal(d), 1 + 0.1 * rng.standard_normal(d)
    # identity layout: page b * nb + i holds rows [i bs, (i+1) bs) of sequence b
    kp = k.reshape(B, Hkv, nb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, d)
    vp = v.reshape(B, Hkv, nb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, d)
    table = np.arange(B * nb).reshape(B, nb)
    lens = np.asarray(lens)
    pos = lens - 1 + 3
    return q, k, v, kp, vp, table, lens, pos, gq, gk


def test_identity_layout_equals_contiguous_decode():
    q, k, v, kp, vp, table, lens, pos, gq, gk = paged_case()
    a = O.decode_paged_ref(q, kp, vp, table, lens, pos, gq, gk, 1e4, block_size=4)
    b = O.decode_ref(q, k, v, lens, pos, gq, gk, 1e4)
    assert np.array_equal(a, b)


def test_page_permutation_invariance_and_unread_entries():
    q, k, v, kp, vp, table, lens, pos, gq, gk = paged_case(seed=1)
    perm = np.random.default_rng(2).permutation(kp.shape[0])
    inv = np.argsort(perm)
    kp2, vp2 = kp[perm], vp[perm]          # physical page p2 holds old page perm[p2]
    table2 = inv[table].copy()             # so old page t lives at inv[t]
    for b, L in enumerate(lens):           # entries past the last block are never read
        table2[b, -(-int(L) // 4):] = -1
    a = O.decode_paged_ref(q, kp, vp, table, lens, pos, gq, gk, 1e4, block_size=4)
    b = O.decode_paged_ref(q, kp2, vp2, table2, lens, pos, gq, gk, 1e4, block_size=4)
    assert np.array_equal(a, b)


def test_scalar_gather_into_brute_force_decode():
    q, k, v, kp, vp, table, lens, pos, gq, gk = paged_case(seed=3)
    perm = np.random.default_rng(4).permutation(kp.shape[0])
    kp2, vp2, table2 = kp[perm], vp[perm], np.argsort(perm)[table]
    bs, (B, Hkv, S, d) = 4, k.shape
    kc = [[[[0.0] * d for _ in range(S)] for _ in range(Hkv)] for _ in range(B)]
    vc = [[[[0.0] * d for _ in range(S)] for _ in range(Hkv)] for _ in range(B)]
    for b in range(B):
        for j in range(int(lens[b])):
            page = int(table2[b][j // bs])
            for h in range(Hkv):
                kc[b][h][j] = [float(x) for x in kp2[page][h][j % bs]]
                vc[b][h][j] = [float(x) for x in vp2[page][h][j % bs]]
    bf = O.brute_decode(q.tolist(), kc, vc, lens, pos, gq.tolist(), gk.tolist(), 1e4)
    ref = O.decode_paged_ref(q, kp2, vp2, table2, lens, pos, gq, gk, 1e4, block_size=4)
    assert np.max(np.abs(ref - np.array(bf))) <= 1e-12
