"""Seeded synthetic inputs for grouped-query attention workloads.

Shared by the tests, bench.py and __graft_entry__.smoke().  This module holds
none of the attention method's arithmetic: it only draws random tensors, rounds
them to the storage dtype and poisons unused cache rows.

Recipe (one numpy ``Generator(PCG64(seed))`` per workload):
  draw order lengths (ragged workloads only), q, k, v, gamma_q, gamma_k;
  q, k, v ~ N(0, 1) drawn in float32; gamma ~ N(1, 0.1);
  bf16 workloads round every float tensor to bf16 (round to nearest even);
  ragged lengths are integers uniform on [lo, hi] inclusive;
  cache rows at or past a sequence's length are filled with NaN ("poison"),
  so any read of them shows up in the output.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np

HEAD_DIM = 128


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    max_seq: int
    dtype: str                      # "f32" or "bf16"
    qk_norm: bool
    rope_theta: float
    split_tokens: int               # 0 = library heuristic; >= max_seq = no split
    lengths: Optional[Tuple[int, int]] = None   # ragged: uniform on [lo, hi]; None = full
    seed: int = 0
    head_dim: int = HEAD_DIM
    eps: float = 1e-6


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq: int
    dtype: str
    qk_norm: bool
    rope_theta: float
    causal: bool = True
    position0: int = 0
    lengths: Optional[Tuple[int, int]] = None
    seed: int = 0
    head_dim: int = HEAD_DIM
    eps: float = 1e-6


# The five workloads: shapes of Qwen3-14B (40 query heads over 8 KV heads)
# and of a Llama3-70B-shaped model (64 over 8).
TINY_DECODE_F32 = DecodeWorkload("tiny_gqa_decode_f32_g5_s512", 1, 5, 1, 512, "f32", True, 1e6,
                                 split_tokens=512, seed=1)
QWEN3_DECODE = DecodeWorkload("qwen3_14b_decode_b1_s4096", 1, 40, 8, 4096, "bf16", True, 1e6,
                              split_tokens=0, seed=2)
QWEN3_RAGGED = DecodeWorkload("qwen3_14b_ragged_decode_b32_s256_16384", 32, 40, 8, 16384, "bf16",
                              True, 1e6, split_tokens=1024, lengths=(256, 16384), seed=3)
LLAMA70B_LONG = DecodeWorkload("llama3_70b_decode_b1_s131072", 1, 64, 8, 131072, "bf16", False,
                               5e5, split_tokens=512, seed=4)
QWEN3_PREFILL = PrefillWorkload("qwen3_14b_causal_prefill_s4096", 1, 40, 8, 4096, "bf16", True,
                                1e6, causal=True, position0=0, seed=5)

DECODE_WORKLOADS = [TINY_DECODE_F32, QWEN3_DECODE, QWEN3_RAGGED, LLAMA70B_LONG]
PREFILL_WORKLOADS = [QWEN3_PREFILL]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    arrays whose values are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _lengths(rng, B: int, S: int, lengths) -> np.ndarray:
    if lengths is None:
        return np.full(B, S, dtype=np.int32)
    lo, hi = lengths
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def lengths_of(w) -> np.ndarray:
    """The per-sequence lengths of a workload without drawing its tensors."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    S = w.max_seq if isinstance(w, DecodeWorkload) else w.seq
    return _lengths(rng, w.batch, S, w.lengths)


def make_decode(w: DecodeWorkload, poison: bool = True) -> dict:
    """Inputs of one decode workload as float32 numpy arrays (bf16-exact when
    w.dtype == 'bf16').  Caches are head-major [B, Hkv, max_seq, d]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, Hq, Hkv, S, d = w.batch, w.num_q_heads, w.num_kv_heads, w.max_seq, w.head_dim
    lens = _lengths(rng, B, S, w.lengths)
    q = _store(rng.standard_normal((B, Hq, d), dtype=np.float32), w.dtype)
    k = _store(rng.standard_normal((B, Hkv, S, d), dtype=np.float32), w.dtype)
    v = _store(rng.standard_normal((B, Hkv, S, d), dtype=np.float32), w.dtype)
    gq = _store(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32), w.dtype)
    gk = _store(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32), w.dtype)
    pos = (lens - 1).astype(np.int32)
    if poison:
        for b in range(B):
            k[b, :, lens[b]:] = np.nan
            v[b, :, lens[b]:] = np.nan
    return dict(q=q, k=k, v=v, q_norm_w=gq if w.qk_norm else None, k_norm_w=gk if w.qk_norm else None,
                seq_lens=lens, positions=pos, rope_theta=w.rope_theta, eps=w.eps)


def make_prefill(w: PrefillWorkload, poison: bool = True) -> dict:
    """Inputs of one prefill workload: q [B, Hq, S, d], k/v [B, Hkv, S, d]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, Hq, Hkv, S, d = w.batch, w.num_q_heads, w.num_kv_heads, w.seq, w.head_dim
    lens = _lengths(rng, B, S, w.lengths)
    q = _store(rng.standard_normal((B, Hq, S, d), dtype=np.float32), w.dtype)
    k = _store(rng.standard_normal((B, Hkv, S, d), dtype=np.float32), w.dtype)
    v = _store(rng.standard_normal((B, Hkv, S, d), dtype=np.float32), w.dtype)
    gq = _store(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32), w.dtype)
    gk = _store(1.0 + 0.1 * rng.standard_normal(d, dtype=np.float32), w.dtype)
    pos = np.full(B, w.position0, dtype=np.int32)
    if poison:
        for b in range(B):
            q[b, :, lens[b]:] = np.nan
            k[b, :, lens[b]:] = np.nan
            v[b, :, lens[b]:] = np.nan
    return dict(q=q, k=k, v=v, q_norm_w=gq if w.qk_norm else None, k_norm_w=gk if w.qk_norm else None,
                seq_lens=lens, positions=pos, rope_theta=w.rope_theta, eps=w.eps, causal=w.causal)


def scaled(w, **kw):
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)
