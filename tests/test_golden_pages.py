"""The pages' printed model dimensions (tests/golden/pages_dims.json) against
the synthetic workloads and the oracle's default scale."""

import json
import math
import os

import numpy as np

import oracle as O
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_dims.json")))


def test_pages_tables_are_self_consistent():
    l70 = GOLD["llama3_70b"]
    assert l70["H_q"] // l70["H_kv"] == l70["G"]
    assert l70["H_q"] * l70["d"] == l70["D"]
    q14 = GOLD["qwen3_14b"]
    assert q14["H_q"] // q14["H_kv"] == q14["G"] and q14["H_q"] % q14["H_kv"] == 0


def test_workloads_use_the_pages_head_shapes():
    q14, l70 = GOLD["qwen3_14b"], GOLD["llama3_70b"]
    for w in (synth.QWEN3_DECODE, synth.QWEN3_RAGGED, synth.QWEN3_PREFILL):
        assert (w.num_q_heads, w.num_kv_heads) == (q14["H_q"], q14["H_kv"])
    assert (synth.LLAMA70B_LONG.num_q_heads, synth.LLAMA70B_LONG.num_kv_heads) == (l70["H_q"], l70["H_kv"])
    assert synth.TINY_DECODE_F32.num_q_heads // synth.TINY_DECODE_F32.num_kv_heads == q14["G"]
    for w in synth.DECODE_WORKLOADS + synth.PREFILL_WORKLOADS:
        assert w.head_dim == l70["d"]


def test_default_scale_is_one_over_sqrt_d():
    # with scale unset the oracle uses 1/sqrt(d): two keys (0 and a e0), query b e0
    d, a, b = 128, 2.0, 3.0
    q = np.zeros((1, 1, d)); q[0, 0, 0] = b
    k = np.zeros((1, 1, 2, d)); k[0, 0, 1, 0] = a
    v = np.zeros((1, 1, 2, d)); v[0, 0, 1, 0] = 1.0
    out = O.decode_ref(q, k, v, np.array([2]), np.array([1]), None, None, 0.0)
    w = 1.0 / (1.0 + math.exp(-a * b / math.sqrt(d)))
    assert math.isclose(out[0, 0, 0], w, rel_tol=1e-14)
