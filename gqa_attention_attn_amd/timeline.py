"""Per-workgroup timelines of the decode partition and prefill attention
kernels, read from the timeline build of the library
(libgqa_attn_timeline.so, include/gqa_timeline.h).

    python -m gqa_attention_attn_amd.timeline [--kernel decode|prefill] [--out FILE]

decode: the Qwen3-14B decode step (B = 1, 40 query heads over 8 KV heads, 4096
cached keys, bf16, QK-norm and RoPE at position 4095).  The K/V caches rotate
over 64 buffer sets (1 GiB), so that no call finds its rows in the 256 MB
Infinity Cache.

prefill: the Qwen3-14B causal prefill (B = 1, 4096 tokens, 40 query heads over
8 KV heads, bf16, QK-norm and RoPE, two phases with a workspace).

Inputs are seeded random tensors.  A HIP graph of several calls is replayed
until the shader clock has settled; then the stamps are cleared and the graph
is replayed once more, so the arrays hold the stamps of its last call.  The
script prints, per stamp, the median, minimum and maximum over the kernel's
workgroups of its time after the first workgroup's entry (prefill: also the
per-tile rate by key-range length and the number of workgroups running over
time).  Argument marshalling and bookkeeping only: every step runs in the
library's kernels.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import build as _build

SLOTS = 8          # GQA_TIMELINE_SLOTS
BLOCKS = 4096      # GQA_TIMELINE_BLOCKS
KERNELS = {"decode": 0, "prefill": 1}   # GQA_TIMELINE_DECODE, GQA_TIMELINE_PREFILL
NAMES = {
    "decode": [
        "entry",
        "length and position known",
        "streaming wave 0: first K/V step requested",
        "prologue done (q', RoPE table, new key's score in LDS)",
        "streaming wave 0: sweep starts (after the barrier)",
        "streaming wave 0: sweep done, state handed over",
        "partial stored",
    ],
    "prefill": [
        "entry",
        "q rows landed",
        "query prologue done",
        "first K'/V tiles landed",
        "tile loop done",
        "exit (output rows written)",
    ],
}
TILES_SLOT = 6     # prefill: the workgroup's tile count


def _load(G):
    path = _build.TIMELINE_LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m gqa_attention_attn_amd.build)")
    G.use_library(path)
    G.lib()
    tl = ctypes.CDLL(path)
    tl.gqa_timeline_clear.restype = ctypes.c_int32
    tl.gqa_timeline_read.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t]
    tl.gqa_timeline_read.restype = ctypes.c_int32
    tl.gqa_timeline_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    tl.gqa_timeline_clock_khz.restype = ctypes.c_int32
    return tl


def _decode_calls(torch, G, gen, dev):
    B, Hq, Hkv, S, d = 1, 40, 8, 4096, 128
    sets = 64
    bf = torch.bfloat16
    q = torch.randn(B, Hq, d, generator=gen, device=dev).to(bf)
    ks = [torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(bf) for _ in range(sets)]
    vs = [torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(bf) for _ in range(sets)]
    qw = (1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(bf)
    kw = (1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(bf)
    sl = torch.full((B,), S, dtype=torch.int32, device=dev)
    pos = torch.full((B,), S - 1, dtype=torch.int32, device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    desc = G.decode_desc(q, ks[0], vs[0], out, 0, 1e-6, 0.0)
    ws = G.decode_workspace(desc, dev)
    ws_bytes = 0 if ws is None else ws.numel()

    def call(i, stream):
        st = G.gqa_attn_decode(desc, q.data_ptr(), ks[i].data_ptr(), vs[i].data_ptr(), sl.data_ptr(),
                               pos.data_ptr(), qw.data_ptr(), kw.data_ptr(), 1e6, out.data_ptr(),
                               0 if ws is None else ws.data_ptr(), ws_bytes, stream)
        if st != G.GQA_OK:
            raise G.GqaError(st, "gqa_attn_decode")
    return call, sets


def _prefill_calls(torch, G, gen, dev):
    B, Hq, Hkv, S, d = 1, 40, 8, 4096, 128
    bf = torch.bfloat16
    q = torch.randn(B, Hq, S, d, generator=gen, device=dev).to(bf)
    k = torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(bf)
    v = torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(bf)
    qw = (1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(bf)
    kw = (1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(bf)
    sl = torch.full((B,), S, dtype=torch.int32, device=dev)
    pos = torch.zeros((B,), dtype=torch.int32, device=dev)
    out = torch.empty(B, Hq, S, d, dtype=torch.float32, device=dev)
    desc = G.prefill_desc(q, k, v, out, True, 1e-6, 0.0)
    ws = G.prefill_workspace(desc, dev)

    def call(i, stream):
        st = G.gqa_attn_prefill(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), sl.data_ptr(), pos.data_ptr(),
                                qw.data_ptr(), kw.data_ptr(), 1e6, out.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        if st != G.GQA_OK:
            raise G.GqaError(st, "gqa_attn_prefill")
    return call, 4


def run(kernel: str, settle_ms: float = 200.0):
    import torch
    import gqa_attention_attn_amd as G

    tl = _load(G)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    call, n = (_decode_calls if kernel == "decode" else _prefill_calls)(torch, G, gen, dev)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in range(n):   # warm the launch path outside the capture
            call(i, s.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(n):
            call(i, s.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    per_replay = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(max(1, int(settle_ms / per_replay))):
        graph.replay()
    torch.cuda.synchronize()
    if tl.gqa_timeline_clear() != 0:
        raise RuntimeError("gqa_timeline_clear failed")
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) * 1000.0 / n

    words = np.zeros(BLOCKS * SLOTS, dtype=np.uint64)
    if tl.gqa_timeline_read(KERNELS[kernel], words.ctypes.data, words.size) != 0:
        raise RuntimeError("gqa_timeline_read failed")
    khz = ctypes.c_int32(0)
    if tl.gqa_timeline_clock_khz(ctypes.byref(khz)) != 0 or khz.value <= 0:
        raise RuntimeError("gqa_timeline_clock_khz failed")
    st = words.reshape(BLOCKS, SLOTS).astype(np.int64)
    live = st[st[:, 0] != 0]
    t0 = live[:, 0].min()
    nstamps = len(NAMES[kernel])
    us = (live[:, :nstamps] - t0) * 1000.0 / khz.value
    tiles = live[:, TILES_SLOT] if kernel == "prefill" else None
    return us, tiles, khz.value, call_us, n


def _stamp_table(names, us):
    lines = ["| stamp | median | min | max |", "|---|---|---|---|"]
    for i, name in enumerate(names):
        col = us[:, i]
        lines.append(f"| {i} {name} | {np.median(col):.2f} | {col.min():.2f} | {col.max():.2f} |")
    return lines


def report(kernel, us, tiles, khz, call_us, n, command) -> str:
    names = NAMES[kernel]
    if kernel == "decode":
        lines = [
            "# Decode partition timeline, qwen3_14b_decode_b1_s4096",
            "",
            "Per-workgroup `s_memrealtime` stamps of the partition kernel (timeline build",
            "`libgqa_attn_timeline.so`, stamp points in `include/gqa_timeline.h`), one decode step",
            "(partition + merge) of B = 1, 40 query heads over 8 KV heads, 4096 cached keys, bf16,",
            "QK-norm and RoPE; K/V rotated over 64 sets (1 GiB), clock settled by graph replays.",
            "",
            "Command (from the repository root): `" + command + "`",
            "",
            f"Counter clock {khz} kHz; {len(us)} partition workgroups stamped; step (partition + merge,",
            f"graph of {n} calls) {call_us:.2f} µs per call.  Times in µs after the first workgroup's entry:",
            "",
        ] + _stamp_table(names, us)
        return "\n".join(lines + [""])
    span = us[:, 5].max()
    start = us[:, 3] - us[:, 0]          # entry -> first tiles landed
    loop = us[:, 4] - us[:, 3]
    per_tile = loop / np.maximum(tiles, 1)
    lines = [
        "# Prefill attention timeline, qwen3_14b_causal_prefill_s4096",
        "",
        "Per-workgroup `s_memrealtime` stamps of the attention kernel (second phase; timeline build",
        "`libgqa_attn_timeline.so`, stamp points in `include/gqa_timeline.h`), one causal prefill of",
        "B = 1, 4096 tokens, 40 query heads over 8 KV heads, bf16, QK-norm and RoPE, with a workspace",
        "(key phase, then attention); clock settled by graph replays.",
        "",
        "Command (from the repository root): `" + command + "`",
        "",
        f"Counter clock {khz} kHz; {len(us)} attention workgroups stamped; call (key phase + attention,",
        f"graph of {n} calls) {call_us:.2f} µs.  First entry to last exit {span:.1f} µs.  Times in µs",
        "after the first workgroup's entry:",
        "",
    ] + _stamp_table(names, us) + [
        "",
        "Per workgroup (median, min, max over the workgroups):",
        "",
        "| part | median | min | max |",
        "|---|---|---|---|",
        f"| entry -> q rows landed | {np.median(us[:, 1] - us[:, 0]):.2f} | {(us[:, 1] - us[:, 0]).min():.2f} | "
        f"{(us[:, 1] - us[:, 0]).max():.2f} |",
        f"| q rows landed -> query prologue done | {np.median(us[:, 2] - us[:, 1]):.2f} | "
        f"{(us[:, 2] - us[:, 1]).min():.2f} | {(us[:, 2] - us[:, 1]).max():.2f} |",
        f"| entry -> first tiles landed (the start) | {np.median(start):.2f} | {start.min():.2f} | {start.max():.2f} |",
        f"| tile loop | {np.median(loop):.2f} | {loop.min():.2f} | {loop.max():.2f} |",
        f"| tile loop done -> exit | {np.median(us[:, 5] - us[:, 4]):.2f} | {(us[:, 5] - us[:, 4]).min():.2f} | "
        f"{(us[:, 5] - us[:, 4]).max():.2f} |",
        "",
        "Tile-loop time per 32-key tile by the workgroup's tile count (median µs per tile):",
        "",
        "| tiles | workgroups | µs per tile | loop start (median µs after first entry) |",
        "|---|---|---|---|",
    ]
    for lo, hi in ((1, 32), (33, 64), (65, 96), (97, 128), (129, 1 << 30)):
        m = (tiles >= lo) & (tiles <= hi)
        if m.any():
            label = f"{lo}-{hi}" if hi < (1 << 30) else f">= {lo}"
            lines.append(f"| {label} | {int(m.sum())} | {np.median(per_tile[m]):.3f} | {np.median(us[m, 3]):.1f} |")
    lines += [
        "",
        "Workgroups running (between entry and exit) over time:",
        "",
        "| µs after first entry | running |",
        "|---|---|",
    ]
    step = 10.0
    t = 0.0
    while t <= span:
        running = int(((us[:, 0] <= t) & (us[:, 5] > t)).sum())
        lines.append(f"| {t:.0f} | {running} |")
        t += step
    return "\n".join(lines + [""])


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--kernel", choices=sorted(KERNELS), default="decode")
    ap.add_argument("--out", default=None, help="also write the summary (markdown) to this file")
    a = ap.parse_args(argv)
    us, tiles, khz, call_us, n = run(a.kernel)
    command = "python -m gqa_attention_attn_amd.timeline --kernel " + a.kernel
    text = report(a.kernel, us, tiles, khz, call_us, n, command)
    print(text, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
