"""Plain, slow, obviously-correct CPU oracle for grouped-query fused attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the ``gqa_attention_attn_amd`` package and its HIP library) never imports,
links or calls anything here, and nothing here imports the product path.

Everything is computed in float64 with materialised score matrices and a
two-pass softmax.  Inputs are upcast exactly from their storage dtype (the
bf16-rounded values the GPU sees are exactly representable in float64).

Sources (the three web pages; no line numbers):

* "ADR-0060: AHBM GQA Fused Attention Kernel (Llama3-70B)"
  - Status / Algorithm lineage: FlashAttention, FlashDecoding (split-KV with a
    log-sum-exp merge) introduce no new math -> the oracle is the plain
    softmax(scale * Q K^T) V definition.
  - §0.5.3 inputs table: ``softmax_scale = 1/sqrt(d)``.
  - §0.5.1 preconditions P2-P4: cached K is post-RoPE and never re-rotated,
    V is raw.
  - §3 per-tile op sequence: the scale multiplies the logits before max/exp.
  - §4 reduction: ``merge(m_a, l_a, O_a, m_b, l_b, O_b)`` and the final O / l.
  - §5.2 decode: the G query heads of one KV head are stacked (M-fold), so
    query head h uses KV head floor(h / G); T_q = 1 attends all past keys.
  - §5.4 prefill: causal classification of (query block, key tile) pairs.
* "Qwen3-14B Optimization"
  - §2.1 "Shape 4" and #796: per-head QK-norm and RoPE are folded into the
    fused attention stage (the prologue).
  - #602 paragraph: RoPE rotates the lo/hi halves of the head dimension; the
    QK-norm reciprocal is a per-row scalar that RoPE is linear in.

Readings taken where the pages are silent:
RMSNorm is x * (mean(x^2) + eps)^-1/2 * gamma over one head's d elements
(gamma shared by all heads); RMSNorm comes before RoPE; RoPE is the textbook
rotation of pairs (i, i + d/2) by angle p * theta^(-2i/d); in decode only the
new token's K row (slot L-1) goes through the prologue; L = 0 gives a zero
output row and L is clamped to the cache capacity; the causal rule includes
the diagonal (key j visible to query i iff j <= i); a prefill chunk of T_q
new tokens after P cached ones is aligned at the bottom right (query t is
token P + t), and P, T_q are clamped to the cache capacity.

Parity status: every function below is pinned by the CPU tests in
``tests/test_oracle.py`` and ``tests/test_oracle_chunk.py`` (closed forms,
worked examples, invariants and a pure-Python brute force).  The composite "whole stage equals the pages' own
kernel" claim is parity unpinned: the pages print no attention outputs.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "rms_norm",
    "rope_frequencies",
    "rope",
    "prologue",
    "attend",
    "partial_state",
    "merge",
    "finalize",
    "decode_ref",
    "decode_split_ref",
    "paged_gather",
    "decode_paged_ref",
    "prefill_ref",
    "prefill_chunk_ref",
    "causal_tile_class",
    "causal_tile_pairs",
    "brute_decode",
    "brute_prefill",
    "brute_prefill_chunk",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Prologue: per-head RMSNorm then RoPE ("Qwen3-14B Optimization", #656/#796/#602)
# --------------------------------------------------------------------------

def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """Per-row RMSNorm over the last axis: x * (mean(x^2) + eps)^-1/2 * gamma.

    The reciprocal r = (mean(x^2) + eps)^-1/2 is a per-row scalar ("Qwen3-14B
    Optimization", #602 paragraph: folding the QK-norm reciprocal).
    """
    x = _f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + float(eps))
    return x * r * _f64(gamma)


def rope_frequencies(d: int, theta: float) -> np.ndarray:
    """Rotation frequency of pair i: theta^(-2i/d) for i in [0, d/2)."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / float(d))


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate the lo/hi halves of the last axis by angle pos * theta^(-2i/d).

    Pair (x_i, x_{i+d/2}) -> (x_i cos a - x_{i+d/2} sin a,
                              x_{i+d/2} cos a + x_i sin a),  a = pos * f_i.
    ``pos`` broadcasts against the leading axes of ``x``.  Angles are formed
    in float64.
    """
    x = _f64(x)
    d = x.shape[-1]
    h = d // 2
    ang = _f64(pos)[..., None] * rope_frequencies(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def prologue(x, gamma, pos, theta: float, eps: float) -> np.ndarray:
    """The fused prologue on projected Q or K rows: RMSNorm (skipped when
    ``gamma`` is None), then RoPE at ``pos`` (skipped when theta <= 0)."""
    y = _f64(x)
    if gamma is not None:
        y = rms_norm(y, gamma, eps)
    if theta is not None and theta > 0:
        y = rope(y, pos, theta)
    return y


# --------------------------------------------------------------------------
# Attention core (ADR-0060 Status: plain softmax attention, no new math)
# --------------------------------------------------------------------------

def attend(q, K, V, scale: float, visible=None):
    """softmax(scale * q K^T) V with a materialised score matrix and a
    two-pass softmax.

    q: [M, d]; K, V: [L, d]; visible: optional bool [M, L] (False = masked).
    Returns (out [M, d], lse [M], probs [M, L]).  Every row must see at
    least one key.
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    s = float(scale) * (q @ K.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)          # pass 1: row max
    e = np.exp(s - m)                               # masked -> exp(-inf) = 0
    z = np.sum(e, axis=-1, keepdims=True)           # pass 2: normaliser
    p = e / z
    return p @ V, (m + np.log(z))[:, 0], p


def partial_state(q, K, V, scale: float):
    """Unnormalised flash state of one KV chunk: (m, l, O) with
    m = max_j s_j, l = sum_j exp(s_j - m), O = sum_j exp(s_j - m) V_j
    (ADR-0060 §3 running state; §4 per-rank partials)."""
    q, K, V = _f64(q), _f64(K), _f64(V)
    s = float(scale) * (q @ K.T)
    m = np.max(s, axis=-1)
    e = np.exp(s - m[:, None])
    return m, np.sum(e, axis=-1), e @ V


def merge(a, b):
    """Union of two flash states over disjoint key sets (ADR-0060 §4 reduction).

    A state (m, l, O) stands for keys whose softmax mass is Z = l * e^m and
    whose normalised output is O / l.  The union has log-mass
    lse = log(e^lse_a + e^lse_b) with lse_i = m_i + log l_i, and its output is
    each side's normalised output weighted by that side's share of the mass,
    e^(lse_i - lse).  The result is returned in the same (m, l, O) form with
    m = lse and l = 1, so merges chain and ``finalize`` applies unchanged.
    """
    m_a, l_a, O_a = (_f64(x) for x in a)
    m_b, l_b, O_b = (_f64(x) for x in b)
    lse_a = m_a + np.log(l_a)
    lse_b = m_b + np.log(l_b)
    lse = np.logaddexp(lse_a, lse_b)
    share_a = np.exp(lse_a - lse)
    share_b = np.exp(lse_b - lse)
    out = (share_a / l_a)[..., None] * O_a + (share_b / l_b)[..., None] * O_b
    return lse, np.ones_like(lse), out


def finalize(state):
    """Normalise once at the end: O / l (ADR-0060 §4)."""
    m, l, O = state
    return O / l[..., None]


def _resolve_scale(scale: Optional[float], d: int) -> float:
    return 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else float(scale)


def _clamp_len(L, cap: int) -> int:
    return int(min(max(int(L), 0), cap))


# --------------------------------------------------------------------------
# Decode (T_q = 1): ADR-0060 §5.2 + the fused prologue of "Qwen3-14B
# Optimization" #796.  Cached rows < L-1 are post-prologue (P2); only the new
# row at slot L-1 is transformed here.
# --------------------------------------------------------------------------

def decode_ref(q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w,
               rope_theta: float, eps: float = 1e-6, scale: Optional[float] = None,
               return_lse: bool = False):
    """q: [B, Hq, d]; k_cache, v_cache: [B, Hkv, S_max, d]; seq_lens,
    positions: [B] ints.  Returns out [B, Hq, d] float64 (and lse [B, Hq])."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    assert Hq % Hkv == 0
    G = Hq // Hkv
    sc = _resolve_scale(scale, d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = _clamp_len(seq_lens[b], S_max)
        if L == 0:
            continue
        p = float(positions[b])
        for h in range(Hkv):
            K = _f64(k_cache[b, h, :L]).copy()
            V = _f64(v_cache[b, h, :L])
            K[L - 1] = prologue(K[L - 1], k_norm_w, p, rope_theta, eps)
            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)
            o, l, _ = attend(Q, K, V, sc)
            out[b, h * G:(h + 1) * G] = o
            lse[b, h * G:(h + 1) * G] = l
    return (out, lse) if return_lse else out


def decode_split_ref(q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w,
                     rope_theta: float, split_tokens: int, eps: float = 1e-6,
                     scale: Optional[float] = None, order: Optional[Sequence[int]] = None):
    """FlashDecoding reference: chunk c covers keys [c*T, min((c+1)*T, L));
    each chunk yields a partial (m, l, O) and the partials are folded with
    ``merge`` in ``order`` (default ascending), then normalised."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    G = Hq // Hkv
    sc = _resolve_scale(scale, d)
    T = int(split_tokens)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = _clamp_len(seq_lens[b], S_max)
        if L == 0:
            continue
        p = float(positions[b])
        n = -(-L // T)
        for h in range(Hkv):
            K = _f64(k_cache[b, h, :L]).copy()
            V = _f64(v_cache[b, h, :L])
            K[L - 1] = prologue(K[L - 1], k_norm_w, p, rope_theta, eps)
            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)
            parts = [partial_state(Q, K[c * T:min((c + 1) * T, L)],
                                   V[c * T:min((c + 1) * T, L)], sc) for c in range(n)]
            seq = list(range(n)) if order is None else [c for c in order if c < n]
            st = parts[seq[0]]
            for c in seq[1:]:
                st = merge(st, parts[c])
            out[b, h * G:(h + 1) * G] = finalize(st)
    return out


def paged_gather(pages, block_table, seq_lens, block_size: int, max_seq: int) -> np.ndarray:
    """Logical cache [B, Hkv, max_seq, d] of a paged cache: logical row j of
    sequence b is pages[block_table[b, j // bs], :, j % bs].  Only the blocks
    that hold rows below seq_lens[b] are read; other rows are NaN."""
    pages = np.asarray(pages)
    _, Hkv, bs, d = pages.shape
    assert bs == block_size and max_seq % bs == 0
    B = len(seq_lens)
    out = np.full((B, Hkv, max_seq, d), np.nan, dtype=np.float64)
    for b in range(B):
        L = _clamp_len(seq_lens[b], max_seq)
        for i in range(-(-L // bs)):
            out[b, :, i * bs:(i + 1) * bs] = pages[int(block_table[b][i])]
    return out


def decode_paged_ref(q, k_pages, v_pages, block_table, seq_lens, positions, q_norm_w, k_norm_w,
                     rope_theta: float, block_size: int, eps: float = 1e-6, scale: Optional[float] = None):
    """Decode over a paged cache: the plain decode of the logical cache that
    the block table describes (paging is addressing only)."""
    max_seq = np.asarray(block_table).shape[1] * block_size
    K = paged_gather(k_pages, block_table, seq_lens, block_size, max_seq)
    V = paged_gather(v_pages, block_table, seq_lens, block_size, max_seq)
    return decode_ref(q, K, V, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, eps, scale)


# --------------------------------------------------------------------------
# Causal prefill: ADR-0060 §5.4 (+ the same prologue on every Q and K row)
# --------------------------------------------------------------------------

def prefill_ref(q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta: float,
                eps: float = 1e-6, scale: Optional[float] = None, causal: bool = True,
                heads: Optional[Sequence[int]] = None, rows: Optional[np.ndarray] = None):
    """q: [B, Hq, S, d]; k, v: [B, Hkv, S, d]; token s of sequence b sits at
    RoPE position positions[b] + s.  Query i sees key j iff j <= i (causal)
    or every key (non-causal), within the first seq_lens[b] tokens.

    ``heads`` restricts the computation to some query heads and ``rows`` to
    some query rows (others stay zero); both exist only to bound the work on
    large cases.  Returns out [B, Hq, S, d] float64; rows >= seq_lens[b] are 0.
    """
    q = np.asarray(q)
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    sc = _resolve_scale(scale, d)
    out = np.zeros((B, Hq, S, d), dtype=np.float64)
    hsel = range(Hq) if heads is None else heads
    for b in range(B):
        n = _clamp_len(seq_lens[b], S)
        if n == 0:
            continue
        pos = float(positions[b]) + np.arange(n, dtype=np.float64)
        rsel = np.arange(n) if rows is None else np.asarray([r for r in rows if r < n], dtype=np.int64)
        if rsel.size == 0:
            continue
        kv_cache = {}
        for hq in hsel:
            h = hq // G
            if h not in kv_cache:
                kv_cache[h] = (prologue(k[b, h, :n], k_norm_w, pos, rope_theta, eps), _f64(v[b, h, :n]))
            K, V = kv_cache[h]
            Q = prologue(q[b, hq, rsel], q_norm_w, pos[rsel], rope_theta, eps)
            vis = (np.arange(n)[None, :] <= rsel[:, None]) if causal else None
            o, _, _ = attend(Q, K, V, sc, vis)
            out[b, hq, rsel] = o
    return out


def prefill_chunk_ref(q, k_cache, v_cache, past_lens, chunk_lens, positions, q_norm_w, k_norm_w,
                      rope_theta: float, eps: float = 1e-6, scale: Optional[float] = None,
                      causal: bool = True, heads: Optional[Sequence[int]] = None,
                      rows: Optional[np.ndarray] = None):
    """Chunked prefill (ADR-0060 §5.4: a query block of T_q tokens that may be
    a chunk of a longer sequence; §0.5.1 P2: cached K is post-RoPE and never
    re-rotated; V is raw).

    q: [B, Hq, T_max, d] raw queries of the chunk; k_cache, v_cache:
    [B, Hkv, S_max, d].  For sequence b with P = past_lens[b] tokens already
    in the cache and T = chunk_lens[b] new tokens (both clamped: P to
    [0, S_max], T to [0, min(T_max, S_max - P)]), cache rows j < P hold
    post-prologue keys, rows P <= j < P + T the raw keys of the chunk, and row
    j sits at RoPE position positions[b] + j.  Query t of the chunk is token
    P + t: it attends keys j <= P + t (causal, aligned at the bottom right of
    the score matrix) or all j < P + T.  Returns out [B, Hq, T_max, d] float64
    (rows t >= T are 0); ``heads`` / ``rows`` restrict the work as in
    ``prefill_ref``.
    """
    q = np.asarray(q)
    B, Hq, T_max, d = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    assert Hq % Hkv == 0
    G = Hq // Hkv
    sc = _resolve_scale(scale, d)
    out = np.zeros((B, Hq, T_max, d), dtype=np.float64)
    hsel = range(Hq) if heads is None else heads
    for b in range(B):
        P = _clamp_len(past_lens[b], S_max)
        T = _clamp_len(chunk_lens[b], min(T_max, S_max - P))
        if T == 0:
            continue
        n = P + T
        pos = float(positions[b]) + np.arange(n, dtype=np.float64)
        tsel = np.arange(T) if rows is None else np.asarray([r for r in rows if r < T], dtype=np.int64)
        if tsel.size == 0:
            continue
        kv = {}
        for hq in hsel:
            h = hq // G
            if h not in kv:
                K = _f64(k_cache[b, h, :n]).copy()
                K[P:] = prologue(K[P:], k_norm_w, pos[P:], rope_theta, eps)
                kv[h] = (K, _f64(v_cache[b, h, :n]))
            K, V = kv[h]
            Q = prologue(q[b, hq, tsel], q_norm_w, pos[P + tsel], rope_theta, eps)
            vis = (np.arange(n)[None, :] <= (P + tsel)[:, None]) if causal else None
            o, _, _ = attend(Q, K, V, sc, vis)
            out[b, hq, tsel] = o
    return out


def causal_tile_class(qs: int, qe: int, ks: int, ke: int) -> str:
    """ADR-0060 §5.4: query block [qs, qe) vs key tile [ks, ke).
    ke <= qs -> 'past' (no mask, full compute); ks >= qe -> 'future' (skip);
    otherwise 'partial' (triangular mask)."""
    if ke <= qs:
        return "past"
    if ks >= qe:
        return "future"
    return "partial"


def causal_tile_pairs(n: int, bm: int, bn: int):
    """Counts of (query block, key tile) classes over an n-token causal
    self-attention: returns dict class -> count."""
    counts = {"past": 0, "partial": 0, "future": 0}
    for qs in range(0, n, bm):
        qe = min(qs + bm, n)
        for ks in range(0, n, bn):
            ke = min(ks + bn, n)
            counts[causal_tile_class(qs, qe, ks, ke)] += 1
    return counts


# --------------------------------------------------------------------------
# Brute force: pure-Python scalar loops (no numpy) for tiny shapes.
# An independent transcription of the same definitions.
# --------------------------------------------------------------------------

def _bf_prologue_row(x: list, gamma, pos: float, theta: float, eps: float) -> list:
    d = len(x)
    y = [float(v) for v in x]
    if gamma is not None:
        ss = 0.0
        for v in y:
            ss += v * v
        r = 1.0 / math.sqrt(ss / d + eps)
        y = [y[i] * r * float(gamma[i]) for i in range(d)]
    if theta is not None and theta > 0:
        h = d // 2
        z = list(y)
        for i in range(h):
            a = pos * (float(theta) ** (-2.0 * i / d))
            z[i] = y[i] * math.cos(a) - y[i + h] * math.sin(a)
            z[i + h] = y[i + h] * math.cos(a) + y[i] * math.sin(a)
        y = z
    return y


def _bf_softmax_weighted(qrow: list, keys: list, vals: list, scale: float) -> list:
    scores = []
    for kr in keys:
        acc = 0.0
        for a, c in zip(qrow, kr):
            acc += a * c
        scores.append(scale * acc)
    mx = max(scores)
    ws = [math.exp(s - mx) for s in scores]
    z = sum(ws)
    d = len(vals[0])
    return [sum(ws[j] * vals[j][t] for j in range(len(vals))) / z for t in range(d)]


def brute_decode(q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w,
                 rope_theta: float, eps: float = 1e-6, scale: Optional[float] = None):
    """Scalar-loop decode; returns nested lists [B][Hq][d]."""
    B, Hq, d = len(q), len(q[0]), len(q[0][0])
    Hkv, S_max = len(k_cache[0]), len(k_cache[0][0])
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else scale
    out = [[[0.0] * d for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = min(max(int(seq_lens[b]), 0), S_max)
        if L == 0:
            continue
        p = float(positions[b])
        for hq in range(Hq):
            h = hq // G
            keys = [[float(v) for v in k_cache[b][h][j]] for j in range(L)]
            keys[L - 1] = _bf_prologue_row(keys[L - 1], k_norm_w, p, rope_theta, eps)
            vals = [[float(v) for v in v_cache[b][h][j]] for j in range(L)]
            qr = _bf_prologue_row(list(q[b][hq]), q_norm_w, p, rope_theta, eps)
            out[b][hq] = _bf_softmax_weighted(qr, keys, vals, sc)
    return out


def brute_prefill(q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta: float,
                  eps: float = 1e-6, scale: Optional[float] = None, causal: bool = True):
    """Scalar-loop prefill; returns nested lists [B][Hq][S][d] (rows past the
    sequence length stay 0)."""
    B, Hq, S, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else scale
    out = [[[[0.0] * d for _ in range(S)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        n = min(max(int(seq_lens[b]), 0), S)
        for hq in range(Hq):
            h = hq // G
            keys = [_bf_prologue_row(list(k[b][h][j]), k_norm_w, float(positions[b]) + j, rope_theta, eps)
                    for j in range(n)]
            vals = [[float(x) for x in v[b][h][j]] for j in range(n)]
            for i in range(n):
                qr = _bf_prologue_row(list(q[b][hq][i]), q_norm_w, float(positions[b]) + i, rope_theta, eps)
                m = i + 1 if causal else n
                out[b][hq][i] = _bf_softmax_weighted(qr, keys[:m], vals[:m], sc)
    return out


def brute_prefill_chunk(q, k_cache, v_cache, past_lens, chunk_lens, positions, q_norm_w, k_norm_w,
                        rope_theta: float, eps: float = 1e-6, scale: Optional[float] = None,
                        causal: bool = True):
    """Scalar-loop chunked prefill; returns nested lists [B][Hq][T_max][d]."""
    B, Hq, T_max, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, S_max = len(k_cache[0]), len(k_cache[0][0])
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(d) if (scale is None or scale <= 0) else scale
    out = [[[[0.0] * d for _ in range(T_max)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        P = min(max(int(past_lens[b]), 0), S_max)
        T = min(max(int(chunk_lens[b]), 0), min(T_max, S_max - P))
        p0 = float(positions[b])
        for hq in range(Hq):
            h = hq // G
            keys = []
            for j in range(P + T):
                row = [float(x) for x in k_cache[b][h][j]]
                keys.append(row if j < P else _bf_prologue_row(row, k_norm_w, p0 + j, rope_theta, eps))
            vals = [[float(x) for x in v_cache[b][h][j]] for j in range(P + T)]
            for t in range(T):
                qr = _bf_prologue_row(list(q[b][hq][t]), q_norm_w, p0 + P + t, rope_theta, eps)
                m = P + t + 1 if causal else P + T
                out[b][hq][t] = _bf_softmax_weighted(qr, keys[:m], vals[:m], sc)
    return out
