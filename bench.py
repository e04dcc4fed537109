#!/usr/bin/env python3
"""Benchmark of the grouped-query fused attention hot path on one MI355X.

Headline (one JSON line on stdout): decode attention of the Qwen3-14B shape
(B = 1, 40 query heads over 8 KV heads, d = 128, 4096 cached keys, bf16,
fused QK-norm + RoPE, split-KV + log-sum-exp merge).  One step = one full
decode call (partition + merge).  `value` is the achieved HBM bandwidth in
algorithmic bytes (valid K/V rows + q + out) per second.  Inputs are resident
in HBM; K/V rotate over enough distinct buffer sets (>= 1 GiB) that the
256 MB Infinity Cache cannot serve them.  The K timed steps are replayed
from a HIP graph: a graph of the W warmup steps is replayed for at least
50 ms of GPU time first (the shader clock settles), then the median of five
timed replays of the K steps is taken.

Also reported in the same line: per-launch kernel durations (HIP events on the
launch stream) and the roofline of the dominant kernel, the oracle timed on
the host cores, the causal prefill of the Qwen3-14B shape (S = 4096) in
TFLOP/s against the bf16 MFMA peak, and the long-context / ragged decodes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]
"""

import argparse
import dataclasses
import json
import math
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA decode µs/step + achieved HBM GB/s; causal prefill TFLOP/s (1×MI355X)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
LLC_BYTES = 1 << 30            # rotate at least this many bytes of K/V
# rocprofv3 FETCH_SIZE / WRITE_SIZE of the decode partition kernel on the
# headline workload, calibrated on a copy kernel
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partition_qwen3_14b_b1_s4096_hbm_counters.json")
KERNEL_SOURCES = ("gqa_attention_attn_amd/csrc/decode.hip", "gqa_attention_attn_amd/csrc/common.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(lens, Hkv, Hq, B, in_elem=2, out_elem=4, d=128):
    """Algorithmic bytes of one decode call: valid K and V rows, q and out."""
    return int(sum(int(x) for x in lens)) * Hkv * 2 * d * in_elem + B * Hq * d * (in_elem + out_elem)


def prefill_flops(lens, Hq, d=128, causal=True):
    """QK^T and PV multiply-adds over the visible (query, key) pairs, 2 flops each."""
    pairs = sum(n * (n + 1) // 2 if causal else n * n for n in (int(x) for x in lens))
    return 4 * d * Hq * pairs


class DecodeCase:
    """Device buffers (R rotating K/V sets) and raw C-ABI arguments of one decode workload."""

    def __init__(self, w, sets, torch, G, synth, exact_first=True):
        self.w = w
        dev = torch.device("cuda")
        bf = torch.bfloat16
        B, Hq, Hkv, S, d = w.batch, w.num_q_heads, w.num_kv_heads, w.max_seq, w.head_dim
        lens = synth.lengths_of(w)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + w.seed)
        self.q, self.k, self.v = [], [], []
        if exact_first:
            inp = synth.make_decode(w)
            to = lambda x: torch.from_numpy(x).to(dev).to(bf)
            self.q.append(to(inp["q"]))
            self.k.append(to(inp["k"]))
            self.v.append(to(inp["v"]))
            self.qw, self.kw = (to(inp["q_norm_w"]), to(inp["k_norm_w"])) if w.qk_norm else (None, None)
        else:
            self.qw = (1 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(bf) if w.qk_norm else None
            self.kw = (1 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(bf) if w.qk_norm else None
        while len(self.k) < sets:
            self.q.append(torch.randn(B, Hq, d, generator=gen, device=dev).to(bf))
            self.k.append(torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(bf))
            self.v.append(torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(bf))
        self.lens = lens
        self.sl = torch.from_numpy(lens).to(dev)
        self.pos = torch.from_numpy((lens - 1).astype("int32")).to(dev)
        self.out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
        self.desc = G.decode_desc(self.q[0], self.k[0], self.v[0], self.out, w.split_tokens, w.eps, 0.0)
        st, self.T, self.n = G.gqa_attn_decode_plan(self.desc)
        assert st == G.GQA_OK
        self.ws = G.decode_workspace(self.desc, dev)
        self.ws_bytes = 0 if self.ws is None else self.ws.numel()
        self.bytes = decode_bytes(lens, Hkv, Hq, B)
        self.G = G

    def args(self, i):
        j = i % len(self.k)
        p = lambda t: None if t is None else t.data_ptr()
        return (self.desc, p(self.q[j]), p(self.k[j]), p(self.v[j]), p(self.sl), p(self.pos), p(self.qw),
                p(self.kw), self.w.rope_theta, p(self.out), p(self.ws), self.ws_bytes)

    def call(self, i, stream):
        st = self.G.gqa_attn_decode(*self.args(i), stream)
        assert st == self.G.GQA_OK, self.G.gqa_attn_status_string(st)

    def partition(self, i, stream):
        st = self.G.gqa_attn_decode_partition(*self.args(i), stream)
        assert st == self.G.GQA_OK

    def merge(self, i, stream):
        a = self.args(i)
        st = self.G.gqa_attn_decode_merge(a[0], a[4], a[9], a[10], a[11], stream)
        assert st == self.G.GQA_OK


def kernel_source_digest():
    """sha256 over the sources of the decode kernels (the counters file records it)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_key") != kernel or rec.get("source_sha256") != kernel_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def graph_time_ms(torch, fn, steps, warmup, trials=5, settle_ms=50.0):
    """Capture `steps` calls of fn(i, stream) in a HIP graph and return the GPU
    time of one replay (ms): the median of `trials` timed replays, taken after a
    warmup graph of `warmup` calls has been replayed for at least `settle_ms`
    of GPU time (the shader clock ramps up over the first tens of ms of
    sustained work; timing before it settles measures the ramp)."""
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for i in range(2):                         # eager warm-up before capture
            fn(i, s.cuda_stream)
    torch.cuda.synchronize()
    gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw, stream=s):
        for i in range(max(warmup, 1)):
            fn(i, s.cuda_stream)
    with torch.cuda.graph(gt, stream=s):
        for i in range(steps):
            fn(i, s.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    settled = 0.0
    while True:
        with torch.cuda.stream(s):
            e0.record(s)
            gw.replay()
            e1.record(s)
        torch.cuda.synchronize()
        settled += e0.elapsed_time(e1)
        if settled >= settle_ms:
            break
    times = []
    for _ in range(max(trials, 1)):
        with torch.cuda.stream(s):
            e0.record(s)
            gt.replay()
            e1.record(s)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return statistics.median(times)


def launch_time_us(torch, fn, steps, warmup):
    """Average duration (us) of one launch of fn(i, stream): `steps` back-to-back
    launches replayed from a HIP graph, bracketed by HIP events on the launch
    stream (each launch's time includes its share of the dispatch gap)."""
    return 1000.0 * graph_time_ms(torch, fn, steps, warmup) / steps


def cpu_baseline(case_inputs, bytes_per_call, budget_s=12.0):
    """The oracle as it stands, on the host cores, over the same decode workload."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    inp = case_inputs
    with threadpool_limits(cores):
        info = threadpool_info()
        threads = max([x.get("num_threads", 1) for x in info] or [1])
        t0 = time.perf_counter()
        reps = 0
        while True:
            O.decode_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["positions"], inp["q_norm_w"],
                         inp["k_norm_w"], inp["rope_theta"], inp["eps"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 1000:
                break
    per = el / reps
    return {"value": bytes_per_call / per / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full oracle decode calls of the headline workload ({el:.1f} s, "
                      f"{per * 1e3:.1f} ms each, host cores available {cores})"}


def prefill_case(torch, G, synth, np, two_phase=True):
    """Device inputs and a call closure of the causal prefill workload."""
    pw = synth.QWEN3_PREFILL
    pin = synth.make_prefill(pw)
    bf = torch.bfloat16
    to = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda().to(bf)
    t = dict(q=to(pin["q"]), k=to(pin["k"]), v=to(pin["v"]), qw=to(pin["q_norm_w"]), kw=to(pin["k_norm_w"]),
             sl=torch.from_numpy(pin["seq_lens"]).cuda(), pos=torch.from_numpy(pin["positions"]).cuda())
    t["out"] = torch.empty(t["q"].shape, dtype=torch.float32, device="cuda")
    desc = G.prefill_desc(t["q"], t["k"], t["v"], t["out"], True, pw.eps)
    t["ws"] = G.prefill_workspace(desc, "cuda") if two_phase else None
    ws_ptr = t["ws"].data_ptr() if two_phase else None
    ws_bytes = t["ws"].numel() if two_phase else 0

    def call(i, stream):
        st = G.gqa_attn_prefill(desc, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["sl"].data_ptr(),
                                t["pos"].data_ptr(), t["qw"].data_ptr(), t["kw"].data_ptr(), pw.rope_theta,
                                t["out"].data_ptr(), ws_ptr, ws_bytes, stream)
        assert st == G.GQA_OK
    return pw, pin, t, call


def prefill_chunk_case(torch, G, synth, np, past=3072, chunk=1024, bs=0):
    """The last `chunk` tokens of the Qwen3-14B prefill prompt as one chunk after
    `past` cached tokens (a cache of past + chunk rows; seeded synthetic rows).
    bs > 0: the same cache as a shuffled pool of bs-row pages."""
    pw = synth.QWEN3_PREFILL
    rng = np.random.Generator(np.random.PCG64(pw.seed + 100))
    bf = torch.bfloat16
    S = past + chunk
    mk = lambda *shape: torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).cuda().to(bf)
    t = dict(q=mk(1, pw.num_q_heads, chunk, 128), k=mk(1, pw.num_kv_heads, S, 128), v=mk(1, pw.num_kv_heads, S, 128),
             qw=(1 + 0.1 * mk(128).float()).to(bf), kw=(1 + 0.1 * mk(128).float()).to(bf),
             past=torch.tensor([past], dtype=torch.int32, device="cuda"),
             cl=torch.tensor([chunk], dtype=torch.int32, device="cuda"),
             pos=torch.tensor([0], dtype=torch.int32, device="cuda"))
    t["out"] = torch.empty(t["q"].shape, dtype=torch.float32, device="cuda")
    desc = G.prefill_chunk_desc(t["q"], t["k"], t["v"], t["out"], True, pw.eps)
    if bs:
        nb = S // bs
        perm = torch.from_numpy(rng.permutation(nb)).cuda()
        pages = lambda x: x[0].reshape(pw.num_kv_heads, nb, bs, 128).transpose(0, 1)   # [nb, Hkv, bs, 128]
        t["kp"] = torch.empty_like(pages(t["k"])).contiguous()
        t["vp"] = torch.empty_like(t["kp"])
        t["kp"][perm] = pages(t["k"])
        t["vp"][perm] = pages(t["v"])
        t["table"] = perm.to(torch.int32).reshape(1, nb).contiguous()
        kp, vp = t["kp"], t["vp"]
        desc.k_stride_b, desc.k_stride_h, desc.k_stride_s = kp.stride(0), kp.stride(1), kp.stride(2)
        desc.v_stride_b, desc.v_stride_h, desc.v_stride_s = vp.stride(0), vp.stride(1), vp.stride(2)
        desc.block_size = bs
        del t["k"], t["v"]
    t["ws"] = G.prefill_workspace(desc, "cuda")
    flops = 4 * 128 * pw.num_q_heads * sum(past + i + 1 for i in range(chunk))

    def call(i, stream):
        if bs:
            st = G.gqa_attn_prefill_chunk_paged(desc, t["q"].data_ptr(), t["kp"].data_ptr(), t["vp"].data_ptr(),
                                                t["table"].data_ptr(), t["past"].data_ptr(), t["cl"].data_ptr(),
                                                t["pos"].data_ptr(), t["qw"].data_ptr(), t["kw"].data_ptr(),
                                                pw.rope_theta, t["out"].data_ptr(), t["ws"].data_ptr(),
                                                t["ws"].numel(), stream)
        else:
            st = G.gqa_attn_prefill_chunk(desc, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                          t["past"].data_ptr(), t["cl"].data_ptr(), t["pos"].data_ptr(),
                                          t["qw"].data_ptr(), t["kw"].data_ptr(), pw.rope_theta, t["out"].data_ptr(),
                                          t["ws"].data_ptr(), t["ws"].numel(), stream)
        assert st == G.GQA_OK
    return t, call, flops


def paged_decode_case(torch, G, synth, np, w, bs):
    """A decode workload over a paged cache of bs-row pages (shuffled pool with
    exactly the pages the lengths need; seeded synthetic rows)."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 200))
    lens = synth.lengths_of(w)
    nb = w.max_seq // bs
    used = [-(-int(L) // bs) for L in lens]
    npages = sum(used)
    bf = torch.bfloat16
    kp = torch.randn(npages, w.num_kv_heads, bs, 128, device="cuda", dtype=bf)
    vp = torch.randn(npages, w.num_kv_heads, bs, 128, device="cuda", dtype=bf)
    perm = rng.permutation(npages)
    table = np.full((w.batch, nb), -1, dtype=np.int32)
    k = 0
    for b, u in enumerate(used):
        table[b, :u] = perm[k:k + u]
        k += u
    t = dict(q=torch.randn(w.batch, w.num_q_heads, 128, device="cuda", dtype=bf), kp=kp, vp=vp,
             table=torch.from_numpy(table).cuda(), sl=torch.from_numpy(lens).cuda(),
             pos=torch.from_numpy(np.maximum(lens, 1) - 1).cuda(),
             qw=(1 + 0.1 * torch.randn(128, device="cuda")).to(bf) if w.qk_norm else None,
             kw=(1 + 0.1 * torch.randn(128, device="cuda")).to(bf) if w.qk_norm else None)
    t["out"] = torch.empty(w.batch, w.num_q_heads, 128, device="cuda", dtype=torch.float32)
    q, out = t["q"], t["out"]
    desc = G.GqaDecodeDesc(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=128,
                           max_seq=w.max_seq, in_dtype=G.GQA_BF16, out_dtype=G.GQA_F32,
                           kv_split_tokens=w.split_tokens, q_stride_b=q.stride(0), q_stride_h=q.stride(1),
                           k_stride_b=kp.stride(0), k_stride_h=kp.stride(1), k_stride_s=kp.stride(2),
                           v_stride_b=vp.stride(0), v_stride_h=vp.stride(1), v_stride_s=vp.stride(2),
                           out_stride_b=out.stride(0), out_stride_h=out.stride(1), eps=w.eps, scale=0.0,
                           block_size=bs)
    st, nbytes = G.gqa_attn_decode_workspace_size(desc)
    assert st == G.GQA_OK
    t["ws"] = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    ptr = lambda x: None if x is None else x.data_ptr()

    def call(i, stream):
        st = G.gqa_attn_decode_paged(desc, q.data_ptr(), kp.data_ptr(), vp.data_ptr(), t["table"].data_ptr(),
                                     t["sl"].data_ptr(), t["pos"].data_ptr(), ptr(t["qw"]), ptr(t["kw"]),
                                     w.rope_theta, out.data_ptr(), t["ws"].data_ptr(), t["ws"].numel(), stream)
        assert st == G.GQA_OK
    return t, call, decode_bytes(lens, w.num_kv_heads, w.num_q_heads, w.batch)


def profile_calls(args, torch, G, synth, np):
    """Plain back-to-back calls of one workload, for profiler runs."""
    if args.only in ("prefill", "prefill_fused"):
        _, _, _, call = prefill_case(torch, G, synth, np, two_phase=args.only == "prefill")
    else:
        w = {"decode": synth.QWEN3_DECODE, "long": synth.LLAMA70B_LONG, "ragged": synth.QWEN3_RAGGED}[args.only or "decode"]
        if args.group:   # the same shape with G query heads per KV head (K/V bytes do not depend on G)
            w = dataclasses.replace(w, name=f"{w.name}_g{args.group}", num_q_heads=w.num_kv_heads * args.group)
        call = DecodeCase(w, 1, torch, G, synth, exact_first=(w is synth.QWEN3_DECODE)).call
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read, {args.copy_probe_mib} MiB written")
    s = torch.cuda.current_stream().cuda_stream
    for i in range(args.eager_calls):
        call(i, s)
    torch.cuda.synchronize()
    log(f"[bench] {args.eager_calls} calls of {args.only} done")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill and long-context decode fields")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "prefill_fused", "long", "ragged"],
                    help="with --eager-calls: the workload to run")
    ap.add_argument("--eager-calls", type=int, default=0,
                    help="profiling mode: run this many plain calls of --only's workload (no timing, no JSON)")
    ap.add_argument("--group", type=int, default=0,
                    help="profiling mode, decode workloads: G query heads per KV head instead of the workload's")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="profiling mode: first copy a device buffer of this many MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this build has "
              "no multi-GPU path; the sharding design is described in DESIGN.md.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import gqa_attention_attn_amd as G
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    G.lib()
    K, W = args.steps, args.warmup
    if args.eager_calls:
        return profile_calls(args, torch, G, synth, np)

    # ---------------- headline: Qwen3-14B decode, B = 1, S = 4096
    w = synth.QWEN3_DECODE
    per_set = decode_bytes(synth.lengths_of(w), w.num_kv_heads, w.num_q_heads, w.batch)
    sets = max(1, math.ceil(LLC_BYTES / per_set))
    log(f"[bench] {w.name}: {per_set} B per call, rotating {sets} K/V sets")
    case = DecodeCase(w, sets, torch, G, synth)
    t_ms = graph_time_ms(torch, case.call, K, W)
    us_step = 1000.0 * t_ms / K
    gbs = case.bytes / (us_step * 1e-6) / 1e9
    log(f"[bench] decode step {us_step:.2f} us  -> {gbs:.1f} GB/s (split T={case.T}, n={case.n})")
    t_part = launch_time_us(torch, case.partition, K, W)
    t_merge = launch_time_us(torch, case.merge, K, W)
    log(f"[bench] per-launch durations: partition {t_part:.2f} us, merge {t_merge:.2f} us")
    ach = case.bytes / (t_part * 1e-6) / 1e9
    traffic = measured_traffic("decode_partition:" + w.name)
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(us_step / 1000.0, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "seq_len": w.max_seq,
                   "kv_split_tokens": case.T, "num_splits": case.n, "qk_norm": w.qk_norm,
                   "rope_theta": w.rope_theta, "kv_sets_rotated": sets, "hip_graph": True},
        "us_per_step": round(us_step, 3),
        "kernel_us": {"decode_partition": round(t_part, 3), "decode_merge": round(t_merge, 3)},
        "roofline": {"bound": "hbm", "kernel": "decode_partition", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": case.bytes},
    }
    cb_inputs = synth.make_decode(w) if not args.no_cpu_baseline else None
    del case
    torch.cuda.empty_cache()

    # ---------------- extras: causal prefill and the other decode shapes
    if not args.no_extra:
        extra = {}
        pw, pin, pt_inputs, pcall = prefill_case(torch, G, synth, np)
        pk_steps = max(5, K // 10)
        flops = prefill_flops(pin["seq_lens"], pw.num_q_heads)
        pt = graph_time_ms(torch, pcall, pk_steps, max(2, W // 10))
        us_p = 1000.0 * pt / pk_steps
        tf = flops / (us_p * 1e-6) / 1e12
        extra["prefill"] = {"workload": pw.name, "path": "two_phase", "us_per_call": round(us_p, 2),
                            "tflops": round(tf, 2),
                            "roofline": {"bound": "mfma", "kernel": "prefill (key prologue + attention)",
                                         "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                                         "algorithmic_flops": flops}}
        log(f"[bench] prefill two-phase {us_p:.1f} us -> {tf:.1f} TFLOP/s")
        del pt_inputs, pcall
        torch.cuda.empty_cache()
        _, _, pt_inputs, pcall = prefill_case(torch, G, synth, np, two_phase=False)
        pt = graph_time_ms(torch, pcall, pk_steps, max(2, W // 10))
        us_f = 1000.0 * pt / pk_steps
        extra["prefill_single_kernel"] = {"workload": pw.name, "path": "single_kernel", "us_per_call": round(us_f, 2),
                                          "tflops": round(flops / (us_f * 1e-6) / 1e12, 2)}
        log(f"[bench] prefill single-kernel {us_f:.1f} us -> {flops / (us_f * 1e-6) / 1e12:.1f} TFLOP/s")
        del pt_inputs, pcall
        torch.cuda.empty_cache()

        ct, ccall, cflops = prefill_chunk_case(torch, G, synth, np)
        pt = graph_time_ms(torch, ccall, pk_steps, max(2, W // 10))
        us_c = 1000.0 * pt / pk_steps
        tf_c = cflops / (us_c * 1e-6) / 1e12
        extra["prefill_chunk"] = {"workload": "qwen3_14b_prefill_chunk_3072_cached_1024_new", "us_per_call": round(us_c, 2),
                                  "tflops": round(tf_c, 2), "frac_of_bf16_peak": round(tf_c / BF16_PEAK_TFLOPS, 4),
                                  "algorithmic_flops": cflops}
        log(f"[bench] prefill chunk (3072 cached + 1024 new) {us_c:.1f} us -> {tf_c:.1f} TFLOP/s")
        del ct, ccall
        torch.cuda.empty_cache()

        ct, ccall, cflops = prefill_chunk_case(torch, G, synth, np, bs=64)
        pt = graph_time_ms(torch, ccall, pk_steps, max(2, W // 10))
        us_c = 1000.0 * pt / pk_steps
        tf_c = cflops / (us_c * 1e-6) / 1e12
        extra["prefill_chunk_paged"] = {"workload": "qwen3_14b_prefill_chunk_3072_cached_1024_new", "block_size": 64,
                                        "us_per_call": round(us_c, 2), "tflops": round(tf_c, 2),
                                        "frac_of_bf16_peak": round(tf_c / BF16_PEAK_TFLOPS, 4)}
        log(f"[bench] prefill chunk over 64-row pages {us_c:.1f} us -> {tf_c:.1f} TFLOP/s")
        del ct, ccall
        torch.cuda.empty_cache()

        for dw, bs in ((synth.LLAMA70B_LONG, 256), (synth.QWEN3_RAGGED, 64)):
            pt_, pcall_, pbytes = paged_decode_case(torch, G, synth, np, dw, bs)
            steps = max(5, K // 10)
            t = graph_time_ms(torch, pcall_, steps, 2)
            us = 1000.0 * t / steps
            extra[dw.name + "_paged"] = {"block_size": bs, "us_per_step": round(us, 2),
                                         "gbs": round(pbytes / (us * 1e-6) / 1e9, 1), "algorithmic_bytes": pbytes}
            log(f"[bench] {dw.name} paged (bs={bs}): {us:.1f} us/step, {pbytes / (us * 1e-6) / 1e9:.0f} GB/s")
            del pt_, pcall_
            torch.cuda.empty_cache()

        for dw in (synth.LLAMA70B_LONG, synth.QWEN3_RAGGED):
            nb = decode_bytes(synth.lengths_of(dw), dw.num_kv_heads, dw.num_q_heads, dw.batch)
            dsets = max(1, math.ceil(LLC_BYTES / nb))
            c = DecodeCase(dw, dsets, torch, G, synth, exact_first=False)
            steps = max(5, K // 10)
            t = graph_time_ms(torch, c.call, steps, 2)
            us = 1000.0 * t / steps
            tp = launch_time_us(torch, c.partition, steps, 2)
            tm = launch_time_us(torch, c.merge, steps, 2)
            extra[dw.name] = {"us_per_step": round(us, 2), "gbs": round(c.bytes / (us * 1e-6) / 1e9, 1),
                              "kernel_us": {"decode_partition": round(tp, 2), "decode_merge": round(tm, 2)},
                              "partition_frac_of_hbm_peak": round(c.bytes / (tp * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                              "kv_split_tokens": c.T, "num_splits": c.n, "kv_sets_rotated": dsets,
                              "algorithmic_bytes": c.bytes}
            log(f"[bench] {dw.name}: {us:.1f} us/step, {c.bytes / (us * 1e-6) / 1e9:.0f} GB/s "
                f"(partition {tp:.1f} us, merge {tm:.1f} us)")
            del c
            torch.cuda.empty_cache()

        # what a plain device copy reaches on this machine (torch copy_ of 1 GiB: 1 GiB read + 1 GiB written)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        t = graph_time_ms(torch, lambda i, stream: dst.copy_(src), 10, 2)
        probe = 2.0 * src.numel() * 4 * 10 / (t * 1e-3) / 1e9
        extra["hbm_copy_probe"] = {"kernel": "torch copy_ of 1 GiB (read + write)", "gbs": round(probe, 1),
                                   "frac_of_hbm_peak": round(probe / HBM_PEAK_GBS, 4),
                                   "decode_partition_frac_of_probe": round(ach / probe, 4)}
        log(f"[bench] copy probe {probe:.0f} GB/s")
        del src, dst
        torch.cuda.empty_cache()
        result["extra"] = extra

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cb_inputs, result["roofline"]["algorithmic_bytes"])
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
