#!/usr/bin/env python3
"""Benchmark of the grouped-query fused attention hot path on one MI355X.

Headline (one JSON line on stdout): decode attention of the Llama3-70B-shaped
long-context workload (B = 1, 64 query heads over 8 KV heads, d = 128,
131072 cached keys, bf16, RoPE theta 5e5 without QK-norm, split-KV into 256
chunks of 512 keys + log-sum-exp merge), the longest-context decode workload.
One step = one full decode call (partition + merge).  `value` is the achieved
HBM bandwidth in algorithmic bytes (valid K/V rows + q + out) per second.
Inputs are resident in HBM; K/V rotate over enough distinct buffer sets
(>= 1 GiB) that the 256 MB Infinity Cache cannot serve them.  The K timed
steps are replayed from a HIP graph: a graph of the W warmup steps is replayed
for at least 50 ms of GPU time first (the shader clock settles), then the
median of five timed replays of the K steps is taken.

Every workload (the tiny f32 decode, the Qwen3-14B B=1 decode, the Qwen3-14B
ragged B=32 decode, the Llama3-70B-shaped decode, the Qwen3-14B causal
prefill) is reported in `extra.workloads` with its time, bandwidth or
TFLOP/s, the roofline of its dominant kernel (algorithmic work over that
kernel's average launch duration, HIP events on its launch stream), the
largest absolute error against the oracle on the same seeded inputs, and the
oracle's own time on the host cores.  `extra.probes` holds what plain kernels
reach on the same GPU in the same run: a streaming HBM read of 16 MiB and of
1 GiB, a 1 GiB device copy and the dispatch floor of one graph node.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-oracle]
Profiling: python bench.py --only WORKLOAD --eager-calls N [--copy-probe-mib M]
Counter records: python bench.py --summarize-counters FETCH_DIR WRITE_DIR --workload NAME --kernel KERNEL
"""

import argparse
import dataclasses
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA decode µs/step + achieved HBM GB/s; causal prefill TFLOP/s (1×MI355X)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA, published
LLC_BYTES = 1 << 30            # rotate at least this many bytes of K/V

# Kernels with a counter record in profiles/: the rocprofv3 kernel-name
# fragment and the sources the record was measured on.
DECODE_SOURCES = ("gqa_attention_attn_amd/csrc/decode.hip", "gqa_attention_attn_amd/csrc/common.hpp")
PREFILL_SOURCES = ("gqa_attention_attn_amd/csrc/prefill_phased.hip", "gqa_attention_attn_amd/csrc/common.hpp")
KERNELS = {
    "decode_partition": ("decode_partition_kernel", DECODE_SOURCES),
    "decode_merge": ("decode_merge_kernel", DECODE_SOURCES),
    "key_prologue": ("key_prologue_kernel", PREFILL_SOURCES),
    "attention": ("attention_kernel", PREFILL_SOURCES),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(lens, Hkv, Hq, B, in_elem=2, out_elem=4, d=128):
    """Algorithmic bytes of one decode call: valid K and V rows, q and out."""
    return int(sum(int(x) for x in lens)) * Hkv * 2 * d * in_elem + B * Hq * d * (in_elem + out_elem)


def prefill_flops(lens, Hq, d=128, causal=True):
    """QK^T and PV multiply-adds over the visible (query, key) pairs, 2 flops each."""
    pairs = sum(n * (n + 1) // 2 if causal else n * n for n in (int(x) for x in lens))
    return 4 * d * Hq * pairs


# ----------------------------------------------------------------- counter records

def counter_file(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.json")


def source_digest(files):
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from its committed counter
    record, or None when there is none or its sources changed since."""
    try:
        with open(counter_file(kernel, workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(rec.get("source_files", [])):
        return None
    return rec.get("traffic_bytes_per_launch")


def read_counter_csv(d, counter):
    """(kernel name, grid size, value) of every dispatch in a rocprofv3 csv directory."""
    import csv
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def summarize_counters(args):
    """Write profiles/<kernel>_<workload>_hbm_counters.json from one FETCH_SIZE
    and one WRITE_SIZE pass of `--only <workload> --eager-calls N
    --copy-probe-mib M`: the kernel's mean KiB per dispatch, each scaled by
    what the same counter reads for the probe copy of M MiB (M MiB read and M
    MiB written)."""
    fetch_dir, write_dir = args.summarize_counters
    frag, sources = KERNELS[args.kernel]
    mib = args.copy_probe_mib
    out = {"kernel_key": f"{args.kernel}:{args.workload}", "workload": args.workload, "kernel_name_fragment": frag}
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = read_counter_csv(d, counter)
        cal = [v for k, g, v in rows if k.startswith("(anonymous namespace)::copy_kernel(")]   # the probe copy
        vals = [v for k, g, v in rows if frag in k]
        if not cal or not vals:
            raise SystemExit(f"{d}: no {counter} rows for the probe copy or for {frag}")
        out[f"{name}_kib_per_dispatch"] = statistics.mean(vals)
        out[f"{name}_dispatches"] = len(vals)
        out[f"{name}_copy_kib"] = statistics.mean(cal)
        out[f"{name}_scale"] = mib * 1024.0 / statistics.mean(cal)
    out["copy_calibration"] = f"gqa_probe_copy of {mib} MiB ({mib * 1024} KiB read, {mib * 1024} KiB written)"
    out["traffic_bytes_per_launch"] = int(round(1024.0 * (out["fetch_kib_per_dispatch"] * out["fetch_scale"] +
                                                           out["write_kib_per_dispatch"] * out["write_scale"])))
    if args.algorithmic_bytes:
        out["algorithmic_bytes_per_launch"] = args.algorithmic_bytes
        out["traffic_over_algorithmic"] = round(out["traffic_bytes_per_launch"] / args.algorithmic_bytes, 4)
    out["commands"] = [
        f"cd /tmp && timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d $REPO/{d} -o p "
        f"-- python3 $REPO/bench.py --only {args.workload_arg or args.workload} --eager-calls 3 --copy-probe-mib {mib}"
        for c, d in (("FETCH_SIZE", os.path.relpath(fetch_dir, ROOT)), ("WRITE_SIZE", os.path.relpath(write_dir, ROOT)))]
    out["summary_command"] = (f"python3 bench.py --summarize-counters {os.path.relpath(fetch_dir, ROOT)} "
                              f"{os.path.relpath(write_dir, ROOT)} --workload {args.workload} --kernel {args.kernel} "
                              f"--workload-arg {args.workload_arg or args.workload} --copy-probe-mib {mib}"
                              + (f" --algorithmic-bytes {args.algorithmic_bytes}" if args.algorithmic_bytes else ""))
    out["source_files"] = list(sources)
    out["source_sha256"] = source_digest(sources)
    path = counter_file(args.kernel, args.workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


# ----------------------------------------------------------------- timing

def graph_times_ms(torch, fn, steps, warmup, trials=5, settle_ms=50.0):
    """Capture `steps` calls of fn(i, stream) in a HIP graph and return the GPU
    times (ms) of `trials` timed replays, taken after a warmup graph of
    `warmup` calls has been replayed for at least `settle_ms` of GPU time (the
    shader clock ramps up over the first tens of ms of sustained work; timing
    before it settles measures the ramp)."""
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
    return times


def graph_time_ms(torch, fn, steps, warmup):
    return statistics.median(graph_times_ms(torch, fn, steps, warmup))


def launch_time_us(torch, fn, steps, warmup):
    """Average duration (us) of one launch of fn(i, stream): `steps` back-to-back
    launches replayed from a HIP graph, bracketed by HIP events on the launch
    stream (each launch's time includes its share of the dispatch gap)."""
    return 1000.0 * graph_time_ms(torch, fn, steps, warmup) / steps


def roofline_hbm(kernel, nbytes, us, traffic):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "algorithmic_bytes": nbytes,
            "kernel_us": round(us, 3)}


def roofline_mfma(kernel, flops, us, traffic):
    tf = flops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": traffic, "algorithmic_flops": flops,
            "kernel_us": round(us, 3)}


# ----------------------------------------------------------------- the oracle on the host

def host_cores():
    return len(os.sched_getaffinity(0))


def time_oracle(fn, budget_s, max_runs=3, min_runs=1):
    """Run the oracle call fn() until `budget_s` of wall time (at least
    min_runs, at most max_runs calls); returns (last result, median seconds
    per call, BLAS threads used, calls)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    with threadpool_limits(host_cores()):
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
        times, out = [], None
        while len(times) < max_runs:
            t0 = time.perf_counter()
            out = fn()
            times.append(time.perf_counter() - t0)
            if len(times) >= min_runs and sum(times) >= budget_s:
                break
    return out, statistics.median(times), int(threads), len(times)


def max_abs_err(got, ref):
    import numpy as np
    g = np.asarray(got, dtype=np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - np.asarray(ref, dtype=np.float64))))


# ----------------------------------------------------------------- decode workloads

class DecodeCase:
    """Device buffers (R rotating K/V sets) and raw C-ABI arguments of one decode
    workload.  Set 0 holds the seeded synthetic inputs the oracle sees (kept in
    self.inp); the other sets are drawn on the GPU with the same distributions."""

    def __init__(self, w, sets, torch, G, synth):
        self.w = w
        dev = torch.device("cuda")
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        B, Hq, Hkv, S, d = w.batch, w.num_q_heads, w.num_kv_heads, w.max_seq, w.head_dim
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 + w.seed)
        self.inp = synth.make_decode(w)
        to = lambda x: torch.from_numpy(x).to(dev).to(dt)
        self.q, self.k, self.v = [to(self.inp["q"])], [to(self.inp["k"])], [to(self.inp["v"])]
        self.qw, self.kw = (to(self.inp["q_norm_w"]), to(self.inp["k_norm_w"])) if w.qk_norm else (None, None)
        while len(self.k) < sets:
            self.q.append(torch.randn(B, Hq, d, generator=gen, device=dev).to(dt))
            self.k.append(torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(dt))
            self.v.append(torch.randn(B, Hkv, S, d, generator=gen, device=dev).to(dt))
        lens = self.inp["seq_lens"]
        self.sl = torch.from_numpy(lens).to(dev)
        self.pos = torch.from_numpy(self.inp["positions"]).to(dev)
        self.out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
        self.desc = G.decode_desc(self.q[0], self.k[0], self.v[0], self.out, w.split_tokens, w.eps, 0.0)
        st, self.T, self.n = G.gqa_attn_decode_plan(self.desc)
        assert st == G.GQA_OK
        self.ws = G.decode_workspace(self.desc, dev)
        self.ws_bytes = 0 if self.ws is None else self.ws.numel()
        self.bytes = decode_bytes(lens, Hkv, Hq, B, in_elem=2 if w.dtype == "bf16" else 4)
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

    def oracle(self):
        import oracle as O
        x = self.inp
        return O.decode_ref(x["q"], x["k"], x["v"], x["seq_lens"], x["positions"], x["q_norm_w"], x["k_norm_w"],
                            x["rope_theta"], x["eps"])


def measure_decode(ctx, w, steps, warmup, oracle_budget_s):
    """Step time, kernel durations, roofline of the partition kernel, the max
    error against the oracle on set 0 and the oracle's time on the host."""
    torch, G, synth = ctx["torch"], ctx["G"], ctx["synth"]
    lens = synth.lengths_of(w)
    per_set = decode_bytes(lens, w.num_kv_heads, w.num_q_heads, w.batch, in_elem=2 if w.dtype == "bf16" else 4)
    # the tiny workload is a latency case: one warm set
    sets = 1 if per_set < (8 << 20) else max(1, math.ceil(LLC_BYTES / per_set))
    log(f"[bench] {w.name}: {per_set} B per call, {sets} K/V sets")
    case = DecodeCase(w, sets, torch, G, synth)
    us = 1000.0 * graph_time_ms(torch, case.call, steps, warmup) / steps
    t_part = launch_time_us(torch, case.partition, steps, warmup)
    t_merge = launch_time_us(torch, case.merge, steps, warmup) if case.n > 1 else 0.0
    gbs = case.bytes / (us * 1e-6) / 1e9
    rec = {"workload": w.name, "us_per_step": round(us, 3), "gbs": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "kernel_us": {"decode_partition": round(t_part, 3), "decode_merge": round(t_merge, 3)},
           "roofline": roofline_hbm("decode_partition", case.bytes, t_part,
                                    measured_traffic("decode_partition", w.name)),
           "kv_split_tokens": case.T, "num_splits": case.n, "kv_sets_rotated": sets, "dtype": w.dtype,
           "algorithmic_bytes": case.bytes}
    log(f"[bench] {w.name}: {us:.2f} us/step -> {gbs:.1f} GB/s (partition {t_part:.2f} us, merge {t_merge:.2f} us, "
        f"T={case.T}, n={case.n})")
    if ctx["oracle"]:
        s = torch.cuda.current_stream().cuda_stream
        case.out.fill_(float("nan"))
        case.call(0, s)
        torch.cuda.synchronize()
        got = case.out.cpu().numpy()
        ref, sec, threads, runs = time_oracle(case.oracle, oracle_budget_s)
        rec["max_abs_err"] = max_abs_err(got, ref)
        rec["tolerance"] = 1e-5 if w.dtype == "f32" else 1e-2
        rec["oracle"] = {"s_per_call": round(sec, 4), "cores": threads, "runs": runs,
                         "gbs": round(case.bytes / sec / 1e9, 3)}
        log(f"[bench] {w.name}: max|err| vs oracle {rec['max_abs_err']:.3e}; oracle {sec:.3f} s per call "
            f"on {threads} threads")
    del case
    torch.cuda.empty_cache()
    return rec


# ----------------------------------------------------------------- prefill workloads

def prefill_case(ctx, two_phase=True):
    """Device inputs and call closures of the causal prefill workload."""
    torch, G, synth, np = ctx["torch"], ctx["G"], ctx["synth"], ctx["np"]
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

    def args():
        return (desc, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["sl"].data_ptr(),
                t["pos"].data_ptr(), t["qw"].data_ptr(), t["kw"].data_ptr(), pw.rope_theta, t["out"].data_ptr(),
                ws_ptr, ws_bytes)

    def call(i, stream):
        assert G.gqa_attn_prefill(*args(), stream) == G.GQA_OK

    def keys(i, stream):
        assert G.gqa_attn_prefill_keys(*args(), stream) == G.GQA_OK

    def attend(i, stream):
        assert G.gqa_attn_prefill_attend(*args(), stream) == G.GQA_OK
    return pw, pin, t, call, keys, attend


def measure_prefill(ctx, steps, warmup):
    torch = ctx["torch"]
    pw, pin, t, call, keys, attend = prefill_case(ctx)
    flops = prefill_flops(pin["seq_lens"], pw.num_q_heads)
    times = [1000.0 * x / steps for x in graph_times_ms(torch, call, steps, warmup)]
    us = statistics.median(times)
    t_keys = launch_time_us(torch, keys, steps, warmup)
    keys(0, torch.cuda.current_stream().cuda_stream)   # the attention phase reads the key phase's workspace
    t_att = launch_time_us(torch, attend, steps, warmup)
    tf = flops / (us * 1e-6) / 1e12
    # key phase: K and V rows read (bf16), K' and V rows written (fp16)
    key_bytes = 4 * int(pin["k"][0].size) * 2
    rec = {"workload": pw.name, "path": "two_phase (key prologue, then attention)",
           "us_per_call": {"median": round(us, 2), "min": round(min(times), 2), "max": round(max(times), 2),
                           "replays": len(times), "calls_per_replay": steps},
           "tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
           "kernel_us": {"key_prologue": round(t_keys, 2), "attention": round(t_att, 2)},
           "roofline": roofline_mfma("attention", flops, t_att, measured_traffic("attention", pw.name)),
           "key_prologue_roofline": roofline_hbm("key_prologue", key_bytes, t_keys,
                                                 measured_traffic("key_prologue", pw.name)),
           "algorithmic_flops": flops}
    log(f"[bench] prefill two-phase {us:.1f} us (min {min(times):.1f}) -> {tf:.1f} TFLOP/s; "
        f"key phase {t_keys:.2f} us, attention {t_att:.2f} us")
    if ctx["oracle"]:
        import oracle as O
        t["out"].fill_(float("nan"))
        call(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got = t["out"].cpu().numpy()
        ref, sec, threads, runs = time_oracle(
            lambda: O.prefill_ref(pin["q"], pin["k"], pin["v"], pin["seq_lens"], pin["positions"], pin["q_norm_w"],
                                  pin["k_norm_w"], pin["rope_theta"], pin["eps"]), 0.0, max_runs=1)
        rec["max_abs_err"] = max_abs_err(got, ref)
        rec["tolerance"] = 1e-2
        rec["oracle"] = {"s_per_call": round(sec, 3), "cores": threads, "runs": runs,
                         "tflops": round(flops / sec / 1e12, 5)}
        log(f"[bench] prefill: max|err| vs oracle {rec['max_abs_err']:.3e} over every element; oracle {sec:.1f} s "
            f"on {threads} threads")
        del ref, got
    del t
    torch.cuda.empty_cache()
    return rec


def prefill_chunk_case(ctx, past=3072, chunk=1024, bs=0):
    """The last `chunk` tokens of the Qwen3-14B prefill prompt as one chunk after
    `past` cached tokens (a cache of past + chunk rows; seeded synthetic rows).
    bs > 0: the same cache as a shuffled pool of bs-row pages."""
    torch, G, synth, np = ctx["torch"], ctx["G"], ctx["synth"], ctx["np"]
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


def paged_decode_case(ctx, w, bs):
    """A decode workload over a paged cache of bs-row pages (shuffled pool with
    exactly the pages the lengths need; seeded synthetic rows).  Calls rotate
    over enough pools (>= LLC_BYTES of K/V) that the Infinity Cache cannot
    serve one call's rows to the next, as for the contiguous workloads."""
    torch, G, synth, np = ctx["torch"], ctx["G"], ctx["synth"], ctx["np"]
    rng = np.random.Generator(np.random.PCG64(w.seed + 200))
    lens = synth.lengths_of(w)
    nb = w.max_seq // bs
    used = [-(-int(L) // bs) for L in lens]
    npages = sum(used)
    bf = torch.bfloat16
    pool_bytes = 2 * npages * w.num_kv_heads * bs * 128 * 2
    sets = max(1, math.ceil(LLC_BYTES / pool_bytes))
    kps = [torch.randn(npages, w.num_kv_heads, bs, 128, device="cuda", dtype=bf) for _ in range(sets)]
    vps = [torch.randn(npages, w.num_kv_heads, bs, 128, device="cuda", dtype=bf) for _ in range(sets)]
    kp, vp = kps[0], vps[0]
    perm = rng.permutation(npages)
    table = np.full((w.batch, nb), -1, dtype=np.int32)
    k = 0
    for b, u in enumerate(used):
        table[b, :u] = perm[k:k + u]
        k += u
    t = dict(q=torch.randn(w.batch, w.num_q_heads, 128, device="cuda", dtype=bf), kp=kps, vp=vps,
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
        j = i % sets
        st = G.gqa_attn_decode_paged(desc, q.data_ptr(), kps[j].data_ptr(), vps[j].data_ptr(), t["table"].data_ptr(),
                                     t["sl"].data_ptr(), t["pos"].data_ptr(), ptr(t["qw"]), ptr(t["kw"]),
                                     w.rope_theta, out.data_ptr(), t["ws"].data_ptr(), t["ws"].numel(), stream)
        assert st == G.GQA_OK
    return t, call, decode_bytes(lens, w.num_kv_heads, w.num_q_heads, w.batch)


# ----------------------------------------------------------------- probes

def measure_probes(ctx):
    """What plain kernels reach on this GPU in this run (libgqa_probe.so)."""
    torch = ctx["torch"]
    from gqa_attention_attn_amd import probe as P
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {}
    for mib in (16, 1024):
        nbytes = mib << 20
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
                for _ in range(max(2, LLC_BYTES // nbytes))]

        def rd(i, stream, bufs=bufs, nbytes=nbytes):
            assert P.read(bufs[i % len(bufs)].data_ptr(), nbytes, sink.data_ptr(), stream) == 0
        steps = 64 if mib == 16 else 8
        us = launch_time_us(torch, rd, steps, 4)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"hbm_read_{mib}mib"] = {"us_per_launch": round(us, 3), "gbs": round(gbs, 1),
                                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "buffers_rotated": len(bufs)}
        log(f"[bench] probe read {mib} MiB: {us:.2f} us per launch -> {gbs:.0f} GB/s")
        del bufs
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def cp(i, stream):
        assert P.copy(src.data_ptr(), dst.data_ptr(), 1 << 30, stream) == 0
    us = launch_time_us(torch, cp, 8, 2)
    res["hbm_copy_1gib"] = {"us_per_launch": round(us, 2), "gbs": round(2 * (1 << 30) / (us * 1e-6) / 1e9, 1),
                            "bytes": "1 GiB read + 1 GiB written"}
    log(f"[bench] probe copy 1 GiB: {us:.1f} us -> {2 * (1 << 30) / (us * 1e-6) / 1e9:.0f} GB/s (read + write)")
    del src, dst

    def em(i, stream):
        assert P.empty(stream) == 0
    us = launch_time_us(torch, em, 256, 16)
    res["graph_node_empty_kernel_us"] = round(us, 3)
    log(f"[bench] probe empty kernel: {us:.2f} us per graph node")
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------- profiling mode

def profile_calls(args, ctx):
    """Plain back-to-back calls of one workload, for profiler runs."""
    torch, synth = ctx["torch"], ctx["synth"]
    if args.copy_probe_mib:
        from gqa_attention_attn_amd import probe as P
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        assert P.copy(src.data_ptr(), dst.data_ptr(), args.copy_probe_mib << 20,
                      torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        log(f"[bench] probe copy: {args.copy_probe_mib} MiB read, {args.copy_probe_mib} MiB written")
        del src, dst
    if args.only in ("prefill", "prefill_fused"):
        _, _, _, call, _, _ = prefill_case(ctx, two_phase=args.only == "prefill")
    elif args.only == "chunk":
        _, call, _ = prefill_chunk_case(ctx)
    else:
        w = {"tiny": synth.TINY_DECODE_F32, "decode": synth.QWEN3_DECODE, "long": synth.LLAMA70B_LONG,
             "ragged": synth.QWEN3_RAGGED}[args.only or "decode"]
        if args.group:   # the same shape with G query heads per KV head (K/V bytes do not depend on G)
            w = dataclasses.replace(w, name=f"{w.name}_g{args.group}", num_q_heads=w.num_kv_heads * args.group)
        call = DecodeCase(w, 1, torch, ctx["G"], synth).call
    s = torch.cuda.current_stream().cuda_stream
    for i in range(args.eager_calls):
        call(i, s)
    torch.cuda.synchronize()
    log(f"[bench] {args.eager_calls} calls of {args.only} done")


# ----------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload (and its oracle)")
    ap.add_argument("--no-oracle", action="store_true", help="skip the oracle runs (errors and host timings)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="same as --no-oracle")
    ap.add_argument("--only", choices=["tiny", "decode", "ragged", "long", "prefill", "prefill_fused", "chunk"],
                    help="with --eager-calls: the workload to run")
    ap.add_argument("--eager-calls", type=int, default=0,
                    help="profiling mode: run this many plain calls of --only's workload (no timing, no JSON)")
    ap.add_argument("--group", type=int, default=0,
                    help="profiling mode, decode workloads: G query heads per KV head instead of the workload's")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="profiling mode: first copy this many MiB with the probe copy (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write a counter record to profiles/ from two rocprofv3 --pmc csv directories")
    ap.add_argument("--workload", help="with --summarize-counters: the workload name of the record")
    ap.add_argument("--workload-arg", help="with --summarize-counters: the --only value the passes used")
    ap.add_argument("--kernel", choices=sorted(KERNELS), help="with --summarize-counters: the kernel")
    ap.add_argument("--algorithmic-bytes", type=int, default=0, help="with --summarize-counters")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this build has "
              "no multi-GPU path (sharding across GPUs is designed, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import gqa_attention_attn_amd as G
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    G.lib()
    ctx = dict(torch=torch, G=G, synth=synth, np=np, oracle=not (args.no_oracle or args.no_cpu_baseline))
    K, W = args.steps, args.warmup
    if args.eager_calls:
        return profile_calls(args, ctx)

    # ---------------- headline: Llama3-70B-shaped decode, B = 1, S = 131072
    w = synth.LLAMA70B_LONG
    head = measure_decode(ctx, w, K, W, oracle_budget_s=2.0)
    us_step = head["us_per_step"]
    result = {
        "metric": METRIC, "value": head["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(us_step / 1000.0, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "seq_len": w.max_seq,
                   "kv_split_tokens": head["kv_split_tokens"], "num_splits": head["num_splits"],
                   "qk_norm": w.qk_norm, "rope_theta": w.rope_theta, "kv_sets_rotated": head["kv_sets_rotated"],
                   "hip_graph": True},
        "us_per_step": us_step,
        "kernel_us": head["kernel_us"],
        "roofline": head["roofline"],
    }
    if "max_abs_err" in head:
        result["max_abs_err"] = head["max_abs_err"]

    if ctx["oracle"]:
        # the oracle as it stands on the host cores, over the headline workload:
        # whole decode calls for about 12 s
        import oracle as O
        inp = synth.make_decode(w)
        _, sec, threads, runs = time_oracle(
            lambda: O.decode_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"], inp["positions"], inp["q_norm_w"],
                                 inp["k_norm_w"], inp["rope_theta"], inp["eps"]), 12.0, max_runs=1000, min_runs=3)
        result["cpu_baseline"] = {
            "value": round(head["algorithmic_bytes"] / sec / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{runs} whole oracle decode calls of {w.name} ({sec:.2f} s each, median; fp64 numpy, "
                      f"{host_cores()} host cores available)"}
        log(f"[bench] cpu baseline {result['cpu_baseline']}")
        del inp

    if not args.no_extra:
        extra = {"workloads": {w.name: head}}
        for dw in (synth.TINY_DECODE_F32, synth.QWEN3_DECODE, synth.QWEN3_RAGGED):
            extra["workloads"][dw.name] = measure_decode(ctx, dw, K, W, oracle_budget_s=3.0)
        pk = max(5, K // 10)
        extra["workloads"][synth.QWEN3_PREFILL.name] = measure_prefill(ctx, pk, max(2, W // 5))

        _, _, t, call, _, _ = prefill_case(ctx, two_phase=False)
        us_f = 1000.0 * graph_time_ms(torch, call, pk, max(2, W // 5)) / pk
        flops = extra["workloads"][synth.QWEN3_PREFILL.name]["algorithmic_flops"]
        extra["prefill_single_kernel"] = {"workload": synth.QWEN3_PREFILL.name, "path": "single kernel, no workspace",
                                          "us_per_call": round(us_f, 2),
                                          "tflops": round(flops / (us_f * 1e-6) / 1e12, 2)}
        log(f"[bench] prefill single kernel {us_f:.1f} us -> {flops / (us_f * 1e-6) / 1e12:.1f} TFLOP/s")
        del t, call
        torch.cuda.empty_cache()

        for key, past, chunk, bs in (("prefill_chunk", 3072, 1024, 0), ("prefill_chunk_paged", 3072, 1024, 64),
                                     ("prefill_chunk_short", 4000, 96, 0)):
            t, call, cflops = prefill_chunk_case(ctx, past, chunk, bs=bs)
            us_c = 1000.0 * graph_time_ms(torch, call, pk, max(2, W // 5)) / pk
            tf_c = cflops / (us_c * 1e-6) / 1e12
            extra[key] = {"workload": f"qwen3_14b_prefill_chunk_{past}_cached_{chunk}_new", "block_size": bs,
                          "us_per_call": round(us_c, 2), "tflops": round(tf_c, 2),
                          "frac_of_bf16_peak": round(tf_c / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": cflops}
            log(f"[bench] {key} ({past} cached + {chunk} new) {us_c:.1f} us -> {tf_c:.1f} TFLOP/s")
            del t, call
            torch.cuda.empty_cache()

        for dw, bs in ((synth.LLAMA70B_LONG, 256), (synth.QWEN3_RAGGED, 64)):
            t, call, nbytes = paged_decode_case(ctx, dw, bs)
            steps = max(5, K // 5)
            us = 1000.0 * graph_time_ms(torch, call, steps, 2) / steps
            extra[dw.name + "_paged"] = {"block_size": bs, "us_per_step": round(us, 2),
                                         "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "algorithmic_bytes": nbytes}
            log(f"[bench] {dw.name} paged (bs={bs}): {us:.1f} us/step, {nbytes / (us * 1e-6) / 1e9:.0f} GB/s")
            del t, call
            torch.cuda.empty_cache()

        extra["probes"] = measure_probes(ctx)
        rd = extra["probes"]["hbm_read_1024mib"]["gbs"]
        result["roofline"]["frac_of_read_probe"] = round(result["roofline"]["achieved"] / rd, 4)
        result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
