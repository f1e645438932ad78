#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one kvq_decode_attn call (one kernel: split attention, then the
log-sum-exp combine by the last workgroup of each sequence and KV head) over
the whole batch of one layer, the hot path of single-query decode attention
over a quantized KV cache.  The cache is built on the device by
kvq_quantize_append from seeded synthetic inputs before timing; inputs are
resident in HBM when the timed region starts.  Caches smaller than 1 GiB are
replicated and the steps rotate over the replicas so that the 256 MB
Infinity Cache cannot hold the working set.

Prints one JSON line: metric, value (effective KV GB/s = algorithmic cache
bytes per step / time per step), ms_per_step, roofline of the split kernel
(algorithmic bytes per launch / its average duration, measured with HIP
events around that kernel on its stream; HBM traffic per launch from the
committed rocprofv3 counter summary when it matches the kernel sources), a
warm single-replica step time, the decode-append time for one token per
sequence, the time of append + attention back to back (the whole decode step
of one layer), and the CPU oracle baseline.

The default workload is 4 (paged_mixed: 64 sequences of 1024-32768 tokens,
64 query / 8 KV heads, int8 with a 128-token bf16 window in 16-token pages),
the largest that fits one GPU.  The same run also times the decode of the
other int8 / int4 workloads (2, 3 and 5) and records them under "also".

Before the W warm-up steps the decode runs untimed for --settle-ms of GPU
time: the GPU's clocks take some tens of milliseconds of sustained decode to
settle (on one MI355X, after 20 warm-up steps the timed steps ran 7-14 %
slower than after 500).

  python bench.py [--config 4] [--steps 200] [--warmup 20] [--also 2,3,5]
  python bench.py --copy-probe 1073741824   (plain copy kernel, for counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + effective KV HBM GB/s (% of MI355X peak), 1 GPU"
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20, help="untimed steps before the timed region")
    # untimed decode before the warm-up steps, in milliseconds of GPU time
    # (clock settling; measured on one MI355X: after 20 steps the VALU-heavy
    # 2-bit step ran 45.8 us, after 500 steps 39.3 us)
    p.add_argument("--settle-ms", type=float, default=300.0)
    p.add_argument("--config", type=int, default=4,
                   help="workload 1..8 (default 4: paged int8 with a bf16 window, the largest)")
    p.add_argument("--also", default="2,3,5",
                   help="other workloads whose decode is timed in the same run ('' = none)")
    p.add_argument("--replicas", type=int, default=0, help="cache copies (0 = enough for 1 GiB)")
    p.add_argument("--split", type=int, default=0, help="split_tokens (0 = library choice)")
    p.add_argument("--query-bits", type=int, default=0,
                   help="0: exact query; 8: the integer-query path")
    p.add_argument("--ab", action="store_true",
                   help="also time the dequantize-into-temporary-storage path")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU baseline time budget")
    p.add_argument("--phases", action="store_true",
                   help="per-workgroup phase breakdown of the decode kernel, from the instrumented "
                        "build (python -m decode_attention_quantized_kvq_amd.build --phase-stamps)")
    p.add_argument("--copy-probe", type=int, default=0,
                   help="run only a plain device copy of this many bytes (counter calibration)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The sources that define the decode kernel and its launch (split plan, grid,
# workspace layout): the counter summaries are valid while these are unchanged.
DECODE_SOURCES = ("kvq_decode.hip", "kvq_decode_kernel.h", "kvq_decode_w4.hip", "kvq_decode_mixed.hip",
                  "kvq_decode_w2.hip", "kvq_host.cpp", "kvq_internal.h", "kvq_quantize.h")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_quantized_kvq_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def copy_probe(nbytes: int, steps: int):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "steps": steps}))


def build_cache(wl, lens, K, synth, torch):
    """One cache of the workload built on the device by kvq_quantize_append."""
    table = None
    nb = mb = 0
    if wl["block_tokens"]:
        table, pool = synth.block_table(wl, lens)
        nb, mb = pool, table.shape[1]
    cfg = K.make_config(batch=wl["batch"], num_q_heads=wl["hq"], num_kv_heads=wl["hkv"],
                        head_dim=wl["d"], max_tokens=wl["tokens"], key=wl["key"],
                        value=wl["value"], window=wl["window"], block_tokens=wl["block_tokens"],
                        num_blocks=nb, max_blocks_per_seq=mb, in_dtype=wl["in_dtype"],
                        group_tokens=wl.get("group", 1), mid_tokens=wl.get("mid", 0))
    st = K.validate(cfg)
    if st != K.KVQ_OK:
        raise SystemExit(f"workload not supported: {K.status_string(st)}")
    cache = K.KvqCache(cfg, "cuda", None if table is None else torch.from_numpy(table))
    k, v = synth.kv_device(wl, lens)
    cache.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
    K.quantize_append(cache, 0, k, v, torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    del k, v
    return cfg, cache


def replicate(cache, K, torch):
    c = K.KvqCache(cache.cfg, "cuda", cache.block_table)
    for name, buf in cache.buffers.items():
        if buf is not None:
            c.buffers[name].copy_(buf)
    c.seq_lens.copy_(cache.seq_lens)
    return c


def cpu_baseline(wl, lens, seconds: float):
    """The oracle as it stands, timed on the host: dequantize-then-attend of
    one decode step over whole (sequence, KV head) groups of the same
    workload, as many groups as fit the time budget, scaled to the full step."""
    import numpy as np
    from decode_attention_quantized_kvq_amd import synth
    from oracle import kvq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    host_cpus = len(os.sched_getaffinity(0))
    fmt = lambda s: O.TensorFormat(s["bits"], s.get("axis", "token"), bool(s.get("zero_point")),
                                   s.get("scale", "f32"))
    G = wl["hq"] // wl["hkv"]
    groups = [(b, h) for b in range(wl["batch"]) for h in range(wl["hkv"])]
    # the same groups in the same order every run; quantization is not timed
    rng = np.random.default_rng(12345)
    order = rng.permutation(len(groups))
    keep = sum(lens) * wl["hkv"] <= (1 << 20)   # small caches are built once
    built = {}
    done_tokens = done_bytes = n_groups = passes = 0
    elapsed = 0.0
    wall0 = time.perf_counter()
    while elapsed < seconds and time.perf_counter() - wall0 < 3 * seconds:
        for gi in order:
            b, h = groups[gi]
            n = lens[b]
            if gi in built:
                cache = built[gi]
            else:
                k, v = synth.kv_tokens(wl, b, h, n)
                cache = O.OracleCache(1, 1, wl["d"], fmt(wl["key"]), fmt(wl["value"]), wl["window"],
                                      group=wl.get("group", 1), mid=wl.get("mid", 0))
                cache.append(0, k[None], v[None])
                if keep:
                    built[gi] = cache
            q = synth.queries(wl, b)[h * G:(h + 1) * G]
            t0 = time.perf_counter()
            cache.attend(0, q)               # dequantize + attend, fp64
            elapsed += time.perf_counter() - t0
            done_bytes += O.decode_traffic(fmt(wl["key"]), fmt(wl["value"]), 1, wl["d"], [n],
                                           wl["window"], wl.get("group", 1), wl.get("mid", 0))
            done_tokens += n
            n_groups += 1
            if elapsed >= seconds:
                break
        passes += 1
    total_bytes = O.decode_traffic(fmt(wl["key"]), fmt(wl["value"]), wl["hkv"], wl["d"], lens,
                                   wl["window"], wl.get("group", 1), wl.get("mid", 0))
    step_s = elapsed * total_bytes / done_bytes
    return {
        "value": round(total_bytes / step_s / 1e9, 3), "unit": "GB/s",
        "us_per_step": round(step_s * 1e6, 1), "cores": threads, "kind": "oracle",
        "host_cpus": host_cpus, "cpu": cpu_model(),
        "cores_note": "cores = BLAS threads the oracle's matrix products ran on; host_cpus = "
                      "CPUs this process may use (sched_getaffinity)",
        "sample": f"{n_groups} (sequence, KV head) group attends ({len(groups)} per step, "
                  f"{passes} pass(es) over them), {done_tokens} tokens, {elapsed:.2f} s of fp64 "
                  f"dequantize-then-attend, scaled by bytes to one full step",
    }


def load_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    profiles/<kernel>_<workload>_counters.md (its `key: value` lines), or None
    when it is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("|", "#", " ", "`")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha") != sha or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentile(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))]


def ab_path(args, wl, caches, q, out, max_len, K, torch):
    """The dequantize-into-temporary-storage alternative: kvq_dequantize writes
    each replica as a bf16 cache (one bf16 copy per replica, so the copies do
    not sit in the Infinity Cache either), then the decode kernel reads that.
    Times the dequantize, the bf16 decode and the two in sequence per step."""
    reps = len(caches)
    T16 = -(-max_len // 16) * 16
    tmps = [K.bf16_cache_like(c, T16) for c in caches]
    ws = torch.zeros(max(K.decode_workspace_bytes(tmps[0].cfg, max_len, args.split), 1),
                     dtype=torch.uint8, device="cuda")
    deq = lambda i: K.dequantize(caches[i % reps], 0, T16, out=tmps[i % reps])
    dec = lambda i: K.decode_attn(tmps[i % reps], 0, q, max_len, out=out, workspace=ws,
                                  split_tokens=args.split, query_bits=args.query_bits)
    for i in range(reps + 3):
        deq(i)
        dec(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("dequantize_us", lambda i: deq(i)), ("bf16_decode_us", lambda i: dec(i)),
                     ("dequantize_then_decode_us", lambda i: (deq(i), dec(i)))):
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / args.steps * 1e3, 2)
    lens = [int(x) for x in caches[0].seq_lens.cpu().tolist()]
    res["bf16_bytes_per_step"] = K.decode_traffic_bytes(tmps[0].cfg, lens)
    log(f"[bench] dequantize-then-decode: {res}")
    return res


def setup_workload(wid, args, K, synth, torch):
    """Cache (and replicas), query, output and workspace of one workload."""
    import numpy as np
    wl = synth.workload(wid)
    lens = synth.seq_lengths(wl)
    max_len = max(lens)
    log(f"[bench] workload {wid} {wl['name']}: building cache")
    t0 = time.time()
    cfg, cache = build_cache(wl, lens, K, synth, torch)
    traffic = K.decode_traffic_bytes(cfg, lens)
    reps = args.replicas
    if reps <= 0:
        reps = 1 if traffic < (16 << 20) else max(1, math.ceil((1 << 30) / traffic))
    caches = [cache] + [replicate(cache, K, torch) for _ in range(reps - 1)]
    torch.cuda.synchronize()
    log(f"[bench] {reps} replica(s) of {traffic / 1e6:.1f} MB built in {time.time() - t0:.1f} s")
    q = torch.from_numpy(np.stack([synth.queries(wl, b) for b in range(wl["batch"])]))
    q = q.to(torch.bfloat16 if wl["in_dtype"] == "bf16" else torch.float32).cuda()
    out = torch.empty((wl["batch"], wl["hq"], wl["d"]), dtype=torch.float32, device="cuda")
    # sized for the timed plan and for the library's own plan (the decode
    # step takes no split option)
    ws = torch.zeros(max(K.decode_workspace_bytes(cfg, max_len, args.split),
                         K.decode_workspace_bytes(cfg, max_len), 1),
                     dtype=torch.uint8, device="cuda")

    def step(i, events=None):
        K.decode_attn(caches[i % reps], 0, q, max_len, out=out, workspace=ws,
                      split_tokens=args.split, split_events=events, query_bits=args.query_bits)

    return dict(wl=wl, lens=lens, max_len=max_len, cfg=cfg, caches=caches, reps=reps,
                traffic=traffic, q=q, out=out, ws=ws, step=step)


def time_decode(w, args, torch):
    """Settles the clocks, runs the warm-up steps, then times exactly
    args.steps decode steps between two events (ms per step), and the split
    kernel's own duration per launch with dispatch-stamped events."""
    step = w["step"]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # clock settling: untimed decode for about args.settle_ms of GPU time,
    # measured in batches of steps
    i = 0
    if args.settle_ms > 0:
        settled = 0.0
        n = 8
        while settled < args.settle_ms:
            e0.record()
            for _ in range(n):
                step(i)
                i += 1
            e1.record()
            torch.cuda.synchronize()
            settled += e0.elapsed_time(e1)
            n = min(n * 2, 4096)
        log(f"[bench] settle: {i} steps, {settled:.1f} ms")
    for _ in range(args.warmup):
        step(i)
        i += 1
    torch.cuda.synchronize()
    # timed region: K steps between two events on the stream
    e0.record()
    for k in range(args.steps):
        step(k)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    # split-kernel duration: events stamped by the dispatch itself
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a, b in pairs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k, pairs[k])
    torch.cuda.synchronize()
    split_each = [a.elapsed_time(b) for a, b in pairs]
    split_ms = sum(split_each) / args.steps
    return ms_step, split_ms, split_each


PHASE_STAMP_BYTES = 65536 * 64   # the instrumented build's stamp region (end of the workspace)


def phase_breakdown(w, args, torch, launches: int = 5):
    """Per-workgroup phases of `launches` decode launches of the instrumented
    build (times in us from the first workgroup's start, 100 MHz counter).
    Each workgroup's first thread stamps: 0 start, 1 work item known, 2 query
    ready (its first tiles in flight), 3 its wave's tiles done, 4 partial
    stored, 5 arrival counted, 6 end; 7 holds the hardware ids."""
    import numpy as np
    ws = w["ws"]
    reg = ws[ws.numel() - PHASE_STAMP_BYTES:]
    out = []
    for i in range(launches):
        reg.zero_()
        torch.cuda.synchronize()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        ev[0].record()
        ev[1].record()
        torch.cuda.synchronize()
        w["step"](i, ev)
        torch.cuda.synchronize()
        st = reg.cpu().numpy().view(np.uint64).reshape(-1, 8).astype(np.int64)
        n = int(np.nonzero(st[:, 0])[0].max()) + 1
        st = st[:n]
        t0 = st[:, 0].min()
        rel = lambda c: (st[:, c] - t0) / 100.0
        streamed = st[:, 3] > 0
        end = np.where(st[:, 6] > 0, ((st[:, 6] >> 1) - t0) / 100.0, np.maximum(rel(1), rel(4)))
        combined = (st[:, 6] & 1) == 1
        hw, xcc = st[:, 7] & 0xFFFFFFFF, (st[:, 7] >> 32) & 0xF
        cu = xcc * 1000 + ((hw >> 13) & 7) * 100 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
        cus = np.unique(cu)
        cu_end = np.array([rel(3)[streamed & (cu == c)].max() for c in cus if (streamed & (cu == c)).any()])
        pct = lambda x, p: round(float(np.percentile(x, p)), 2) if len(x) else None
        out.append({
            "kernel_us_events": round(ev[0].elapsed_time(ev[1]) * 1e3, 2),
            "span_us": round(float(end.max()), 2), "workgroups": n, "cus": int(len(cus)),
            "start_p50_max": [pct(rel(0), 50), pct(rel(0), 100)],
            "item_known_after_start_p50": pct(rel(1) - rel(0), 50),
            "query_ready_after_item_p50_p90": [pct((rel(2) - rel(1))[streamed], p) for p in (50, 90)],
            "tiles_us_p10_p50_p90": [pct((rel(3) - rel(2))[streamed], p) for p in (10, 50, 90)],
            "cu_tiles_done_min_p50_max": [round(float(cu_end.min()), 2), pct(cu_end, 50),
                                          round(float(cu_end.max()), 2)],
            "partial_stored_after_tiles_p50_p90": [pct((rel(4) - rel(3))[streamed], p) for p in (50, 90)],
            "arrival_after_store_p50_p90": [pct((rel(5) - rel(4))[streamed & (st[:, 5] > 0)], p)
                                            for p in (50, 90)],
            "combine_us_p50_p90": [pct((end - rel(5))[combined], p) for p in (50, 90)],
            "end_p50_p90_max": [pct(end, p) for p in (50, 90, 100)],
        })
        j = int(np.argmax(end))
        out[-1]["last_workgroup"] = {k: round(float(v), 2) for k, v in (
            ("start", rel(0)[j]), ("item_known", rel(1)[j]), ("query_ready", rel(2)[j]),
            ("tiles_done", rel(3)[j]), ("partial_stored", rel(4)[j]), ("arrived", rel(5)[j]),
            ("end", end[j]))}
        log(f"[bench] phases launch {i}: {json.dumps(out[-1])}")
    return out


def main():
    args = parse()
    if args.phases:
        from decode_attention_quantized_kvq_amd import build as B
        if not os.path.exists(B.PHASES_LIB):
            raise SystemExit(f"{B.PHASES_LIB} is missing: build it with "
                             "python -m decode_attention_quantized_kvq_amd.build --phase-stamps")
        os.environ["KVQ_LIB"] = B.PHASES_LIB
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the decode "
              "path has no multi-GPU mode (sequences and KV heads are independent, so several "
              "GPUs would each run this same single-GPU kernel on their share).", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps, 1))
        return
    import torch
    from decode_attention_quantized_kvq_amd import kvq as K
    from decode_attention_quantized_kvq_amd import synth

    w = setup_workload(args.config, args, K, synth, torch)
    wl, lens, max_len, caches, reps = w["wl"], w["lens"], w["max_len"], w["caches"], w["reps"]
    q, out, ws, step, traffic = w["q"], w["out"], w["ws"], w["step"], w["traffic"]
    ms_step, split_ms, split_each = time_decode(w, args, torch)
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.2f} us/step; split kernel "
        f"{split_ms * 1e3:.2f} us/launch")
    if args.phases:
        ph = phase_breakdown(w, args, torch)
        print(json.dumps({"workload": wl["name"], "avg_launch_us": round(split_ms * 1e3, 2),
                          "kernel_sources": kernel_source_sha(), "phases": ph}), flush=True)
        return
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    # warm: the same replica every step (working set may sit in the 256 MB
    # Infinity Cache; context only)
    e0.record()
    for i in range(args.steps):
        step(0)
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / args.steps

    # decode-append: one new token per sequence (rewrites each sequence's
    # last position of replica 0, after all timing that reads it; repeating
    # it rewrites the same positions).  Eager calls are bound by the host's
    # launch path (the kernels take a few microseconds), so the append is
    # also captured once in a HIP graph and replayed: that is its GPU time.
    # The graph comes last: on this platform eager decode launches after a
    # graph capture ran 4-6 % slower (measured: 412.9 us before, 428-438
    # after, also once the graph is freed), so every eager timing precedes it.
    k1, v1 = (torch.randn((wl["batch"], wl["hkv"], 1, wl["d"]), device="cuda").to(q.dtype)
              for _ in range(2))
    ones = torch.ones(wl["batch"], dtype=torch.int32, device="cuda")
    append = lambda: K.quantize_append(caches[0], 0, k1, v1, ones)
    for _ in range(3):
        append()
    e0.record()
    for _ in range(20):
        append()
    e1.record()
    torch.cuda.synchronize()
    append_eager_us = e0.elapsed_time(e1) / 20 * 1e3

    # the whole decode step of one layer: quantize-append one token per
    # sequence, then attend (each step rewrites the last position of the
    # replica it attends; the work is the same every step)
    # (the start event follows the warm-up launches on the stream without a
    # host synchronization, so the host's launch path of the first timed
    # step overlaps the warm-up's GPU time, as it does in a serving loop)
    for i in range(max(reps, 10)):
        K.quantize_append(caches[i % reps], 0, k1, v1, ones)
        step(i)
    e0.record()
    for i in range(args.steps):
        K.quantize_append(caches[i % reps], 0, k1, v1, ones)
        step(i)
    e1.record()
    torch.cuda.synchronize()
    full_step_us = e0.elapsed_time(e1) / args.steps * 1e3
    # the same step through kvq_decode_step (one kernel for formats it fuses)
    for i in range(max(reps, 10)):
        K.decode_step(caches[i % reps], 0, k1, v1, q, max_len, out=out, workspace=ws)
    e0.record()
    for i in range(args.steps):
        K.decode_step(caches[i % reps], 0, k1, v1, q, max_len, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    decode_step_us = e0.elapsed_time(e1) / args.steps * 1e3

    ab = ab_path(args, wl, caches, q, out, max_len, K, torch) if args.ab else None

    def graph_append_us():
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(10):
                append()
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 100 * 1e3

    value = traffic / (ms_step * 1e-3) / 1e9
    achieved = traffic / (split_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    hbm = load_traffic("decode_split", wl["name"], sha)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8,f16",  # matrix-core operands: int8 query limbs x int8 key codes
                            # (int32 sums), fp16 weights x exact fp16 value codes;
                            # fp32 scales, softmax and accumulation
        "data": "synthetic (seeded; no dataset on the pages)",
        "config": {"workload": wl["name"], "batch": wl["batch"], "q_heads": wl["hq"],
                   "kv_heads": wl["hkv"], "head_dim": wl["d"], "tokens": max_len,
                   "total_tokens": int(sum(lens)),
                   "key": wl["key"], "value": wl["value"], "window": wl["window"],
                   "block_tokens": wl["block_tokens"], "group_tokens": wl.get("group", 1),
                   "mid_tokens": wl.get("mid", 0), "replicas": reps,
                   "split_tokens": args.split or "auto", "query_bits": args.query_bits,
                   "settle_ms": args.settle_ms, "kernel_sources": sha},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": hbm, "kernel": "decode_split",
                     "algorithmic_bytes_per_launch": traffic,
                     "avg_launch_us": round(split_ms * 1e3, 2),
                     "launch_us_p10_p50_p90": [round(percentile(split_each, p) * 1e3, 2)
                                               for p in (10, 50, 90)]},
        "warm_us_per_step": round(warm_ms * 1e3, 2),
        "decode_append_us": None,                          # GPU time (graph replay), below
        "decode_append_eager_us": round(append_eager_us, 2),  # per eager call
        "step_with_append_us": round(full_step_us, 2),  # append one token, then attend
        "decode_step_us": round(decode_step_us, 2),     # the same through kvq_decode_step
    }
    if ab is not None:
        result["ab_dequantize_then_decode"] = ab
    # the decode of the other int8 / int4 workloads, timed the same way
    # (the main workload's first cache stays for the graph-replayed append)
    also = {}
    del w, q, out, ws, step
    caches = caches[:1]
    torch.cuda.empty_cache()
    for wid in [int(x) for x in args.also.split(",") if x.strip()]:
        if wid == args.config:
            continue
        o = setup_workload(wid, args, K, synth, torch)
        ms_o, split_o, _ = time_decode(o, args, torch)
        frac = o["traffic"] / (split_o * 1e-3) / 1e9 / PEAK_HBM_GBS
        also[o["wl"]["name"]] = {
            "us_per_step": round(ms_o * 1e3, 2), "avg_launch_us": round(split_o * 1e3, 2),
            "algorithmic_bytes_per_launch": o["traffic"], "frac": round(frac, 4),
            "value_gbs": round(o["traffic"] / (ms_o * 1e-3) / 1e9, 1),
            "traffic": load_traffic("decode_split", o["wl"]["name"], sha)}
        log(f"[bench] also {o['wl']['name']}: {ms_o * 1e3:.2f} us/step, split kernel "
            f"{split_o * 1e3:.2f} us, frac {frac:.4f}")
        del o
        torch.cuda.empty_cache()
    if also:
        result["also"] = also
    result["decode_append_us"] = round(graph_append_us(), 2)
    if not args.no_cpu:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(wl, lens, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
