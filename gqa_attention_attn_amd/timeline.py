"""Per-workgroup timeline of the decode partition kernel, read from the
timeline build of the library (libgqa_attn_timeline.so, include/gqa_timeline.h).

    python -m gqa_attention_attn_amd.timeline [--out FILE]

Runs the Qwen3-14B decode step (B = 1, 40 query heads over 8 KV heads, 4096
cached keys, bf16, QK-norm and RoPE at position 4095) on seeded random
inputs.  The K/V caches rotate over 64 buffer sets (1 GiB), so that no call
finds its rows in the 256 MB Infinity Cache.  A HIP graph of one call per set
is replayed until the shader clock has settled; then the stamps are cleared
and the graph is replayed once more, so the array holds the stamps of its
last call.  For each stamp the script prints the median, minimum and maximum
over the partition's workgroups of its time after the first workgroup's
entry.  Argument marshalling and bookkeeping only: every step of the decode
runs in the library's kernels.
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
NAMES = [
    "entry",
    "length and position known",
    "streaming wave 0: first K/V step requested",
    "prologue done (q', RoPE table, new key's score in LDS)",
    "streaming wave 0: sweep starts (after the barrier)",
    "streaming wave 0: sweep done, state handed over",
    "partial stored",
]


def run(settle_ms: float = 200.0):
    import torch
    import gqa_attention_attn_amd as G

    path = _build.TIMELINE_LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m gqa_attention_attn_amd.build)")
    G.use_library(path)
    G.lib()
    tl = ctypes.CDLL(path)
    tl.gqa_timeline_clear.restype = ctypes.c_int32
    tl.gqa_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    tl.gqa_timeline_read.restype = ctypes.c_int32
    tl.gqa_timeline_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    tl.gqa_timeline_clock_khz.restype = ctypes.c_int32

    dev = torch.device("cuda")
    B, Hq, Hkv, S, d = 1, 40, 8, 4096, 128
    sets = 64
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
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

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in range(sets):   # warm the launch path outside the capture
            call(i, s.cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for i in range(sets):
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
    step_us = e0.elapsed_time(e1) * 1000.0 / sets

    words = np.zeros(BLOCKS * SLOTS, dtype=np.uint64)
    if tl.gqa_timeline_read(words.ctypes.data, words.size) != 0:
        raise RuntimeError("gqa_timeline_read failed")
    khz = ctypes.c_int32(0)
    if tl.gqa_timeline_clock_khz(ctypes.byref(khz)) != 0 or khz.value <= 0:
        raise RuntimeError("gqa_timeline_clock_khz failed")
    st = words.reshape(BLOCKS, SLOTS)
    live = st[st[:, 0] != 0].astype(np.int64)
    t0 = live[:, 0].min()
    us = (live[:, :len(NAMES)] - t0) * 1000.0 / khz.value
    return us, khz.value, step_us, len(live)


def report(us, khz, step_us, nwg, command) -> str:
    lines = [
        "# Decode partition timeline, qwen3_14b_decode_b1_s4096",
        "",
        "Per-workgroup `s_memrealtime` stamps of the partition kernel (timeline build",
        "`libgqa_attn_timeline.so`, stamp points in `include/gqa_timeline.h`), one decode step",
        "(partition + merge) of B = 1, 40 query heads over 8 KV heads, 4096 cached keys, bf16,",
        "QK-norm and RoPE; K/V rotated over 64 sets (1 GiB), clock settled by graph replays.",
        "",
        "Command (repository root on the GPU box): `" + command + "`",
        "",
        f"Counter clock {khz} kHz; {nwg} partition workgroups stamped; step (partition + merge,",
        f"graph of 64 calls) {step_us:.2f} µs per call.  Times in µs after the first workgroup's entry:",
        "",
        "| stamp | median | min | max |",
        "|---|---|---|---|",
    ]
    for i, name in enumerate(NAMES):
        col = us[:, i]
        lines.append(f"| {i} {name} | {np.median(col):.2f} | {col.min():.2f} | {col.max():.2f} |")
    lines.append("")
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None, help="also write the summary (markdown) to this file")
    a = ap.parse_args(argv)
    us, khz, step_us, nwg = run()
    command = "python -m gqa_attention_attn_amd.timeline"
    text = report(us, khz, step_us, nwg, command)
    print(text, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
