#!/usr/bin/env python3
"""Benchmark: one paged decode step (KV append + decode attention) on one MI355X.

A step is ``paged_kv_write`` (one new token per sequence) followed by
``paged_attn_decode`` over every sequence of the batch, on torch's current
stream, inputs resident in HBM.  The default workload is the high-concurrency
batch: 256 sequences, 32 query / 8 KV heads, head_dim 128, bf16, 16-token
blocks, lognormal context lengths (median 1024, sigma 1, clamp [1, 8192]),
pool ~90% full with the free blocks interleaved.

Output: one JSON line (rank 0).  ``value`` is decode sequences per second of the
whole step (wall clock over the K timed steps, synchronised on both sides);
``roofline`` prices the decode call (partition + combine kernels, timed with
HIP events on the launch stream) against 8 TB/s with the algorithmic bytes of
one launch: sum(ctx) * 2 * Hkv * head_dim * elem (K and V rows read once) plus
q, out, the block-table entries and the lengths.  ``cpu_baseline`` is the fp64
CPU oracle timed on the host cores (the same step, write + attention).
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode seqs/s and achieved KV-read HBM GB/s (% of peak), 1 MI355X"
PEAK_HBM_GBS = 8000.0


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="hc_b256",
                   choices=["tiny", "llama8b_b64", "hc_b256", "long32k", "shared_prefix",
                            "multi_spec4", "multi_chunk64"],
                   help="multi_* are steps with several new tokens per sequence (paged_attn_decode_multi)")
    p.add_argument("--partition-tokens", type=int, default=0)
    p.add_argument("--kernel", type=int, default=0, help="0 auto, 1 generic, 2 fast")
    p.add_argument("--grid-waves", type=int, default=0, help="fast kernel: waves sharing the work (0 = library choice)")
    p.add_argument("--xcd-balance", type=int, default=0,
                   help="fast kernel: share of a wave on an odd XCD in 64ths (64 = equal, 0 = library choice)")
    p.add_argument("--cold-steps", type=int, default=10,
                   help="after the timed steps, time this many decode calls each preceded by "
                        "reading --flush-mib of scratch (no KV bytes left in L2 or MALL)")
    p.add_argument("--flush-mib", type=int, default=512)
    p.add_argument("--block-size", type=int, default=0,
                   help="redraw the workload's lengths into blocks of this many tokens (block-size sweep)")
    p.add_argument("--heads", default="",
                   help="Hq,Hkv,d: the same batch with another head layout (e.g. 128,8,128 or 32,8,256)")
    p.add_argument("--prefix", action="store_true",
                   help="decode with paged_attn_decode_prefix (workloads whose sequences share prefix blocks): "
                        "each shared block is read once per group")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-achievable", action="store_true",
                   help="skip the same-run streaming-read ceiling (2 GiB read by a plain HIP kernel)")
    p.add_argument("--no-parity", action="store_true")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="HBM bytes per launch measured by rocprofv3 counters (optional)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after the timed steps, copy a buffer of this many MiB three times "
                        "(a plain copy of known size for scaling hardware byte counters)")
    p.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: read two rocprofv3 --pmc runs of this script (FETCH_SIZE, "
                        "WRITE_SIZE; each directory also holds the run's JSON line as bench.json) "
                        "and record the decode call's HBM bytes per launch in --traffic-json")
    return p.parse_args(argv)


def algorithmic_bytes(w) -> dict:
    """Bytes one decode call must move.  `kv` counts every sequence's tokens (the
    logical attention input); `kv_unique` counts each physical block's used
    tokens once (what a path that reads a shared block once per batch moves)."""
    ctx = w.context_lens.astype(np.int64)
    e = w.elem_bytes
    B = w.block_size
    per_token = 2 * w.num_kv_heads * w.head_dim * e
    kv = int(ctx.sum()) * per_token
    used = {}
    for i, n in enumerate(ctx):
        for b in range(-(-int(n) // B)):
            phys = int(w.block_tables[i, b])
            used[phys] = max(used.get(phys, 0), min(B, int(n) - b * B))
    kv_unique = sum(used.values()) * per_token
    q = w.num_seqs * w.num_q_heads * w.head_dim * e
    out = w.num_seqs * w.num_q_heads * w.head_dim * 4
    tables = int(((ctx + B - 1) // B).sum()) * 4 + w.num_seqs * 4
    return {"kv": kv, "kv_unique": kv_unique, "q": q, "out": out, "tables": tables,
            "total": kv + q + out + tables, "total_unique": kv_unique + q + out + tables}


def cpu_baseline(w) -> dict:
    import oracle

    o = oracle.Oracle()
    kc = oracle._bits(w.k_cache).copy()
    vc = oracle._bits(w.v_cache).copy()
    # Repeat the whole batch until about 10 s of host work is spent (at least
    # three runs), then take the median run.
    times = []
    budget = 10.0
    while True:
        t0 = time.perf_counter()
        o.kv_write(w.k_new, w.v_new, w.slot_mapping, kc, vc, w.block_size)
        o.attn_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, num_kv_heads=w.num_kv_heads)
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 and sum(times) >= budget:
            break
    med = statistics.median(times)
    return {
        "value": w.num_seqs / med,
        "unit": "seqs/s",
        "cores": o.num_threads(),
        "kind": "oracle",
        "sample": f"whole batch ({w.num_seqs} seqs, write + attention), median of {len(times)} runs "
                  f"of {med:.2f} s",
        "kv_GBps": algorithmic_bytes(w)["kv"] / med / 1e9,
        "cpu": cpu_model(),
        "os_cpu_count": os.cpu_count(),
        "threads_used": o.num_threads(),
    }


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (the machine name where that is missing)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


DECODE_KERNELS = ("decode_prefix_kernel", "decode_fast_kernel", "merge_fast_kernel", "decode_generic_kernel", "combine_kernel",
                  "multi_query_kernel", "multi_pipe_kernel", "multi_merge_kernel", "multi_sk_kernel", "multi_sk_merge_kernel")


def _counter_rows(run_dir: str):
    import csv
    import glob

    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {run_dir}, found {files}")
    with open(files[0]) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _per_dispatch(rows, counter: str):
    """(kernel name, value) per dispatch; a counter read per XCD or SE is summed."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        name, val = acc.get(key, (r["Kernel_Name"], 0.0))
        acc[key] = (name, val + float(r["Counter_Value"]))
    return [acc[k] for k in sorted(acc)]


def ingest_counters(args) -> int:
    """Turn FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per decode call.

    Each counter is scaled by what it reads for the plain device-to-device copy
    of known size that the profiled run made last (three copies of
    ``copy_calibration_bytes``), so that the figure is in real HBM bytes."""
    out = {}
    meta = None
    for counter, run_dir in (("FETCH_SIZE", args.ingest_counters[0]), ("WRITE_SIZE", args.ingest_counters[1])):
        with open(os.path.join(run_dir, "bench.json")) as f:
            line = [ln for ln in f if ln.startswith("{")][-1]
        rec = json.loads(line)
        disp = _per_dispatch(_counter_rows(run_dir), counter)
        copies = [v for n, v in disp if "copyBuffer" in n][-3:]
        nbytes = rec.get("copy_calibration_bytes")
        if not nbytes or len(copies) != 3:
            raise SystemExit(f"{run_dir}: the run made no calibration copies (--copy-calibration-mib)")
        factor = nbytes / (statistics.mean(copies) * 1024.0)
        per_kernel = {}
        for name in DECODE_KERNELS:
            vals = [v for n, v in disp if name in n]
            if vals:
                per_kernel[name] = statistics.mean(vals) * 1024.0 * factor
        if not per_kernel:
            raise SystemExit(f"{run_dir}: no decode kernel dispatches")
        out[counter] = {"factor": factor, "per_kernel_bytes": per_kernel, "bytes": sum(per_kernel.values())}
        cfg = rec["config"]
        this = (cfg["workload"], cfg["kernel"], cfg["partition_tokens"], rec["algorithmic_bytes"]["total"])
        if meta is not None and meta != this:
            raise SystemExit("the two runs profiled different workloads")
        meta = this
    key = f"{meta[0]}/{meta[1]}/T{meta[2]}"
    table = {}
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            table = json.load(f)
    table[key] = {
        "source_sha": _kernel_source_sha(),
        "bytes_per_launch": out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"],
        "read_bytes": out["FETCH_SIZE"]["bytes"],
        "write_bytes": out["WRITE_SIZE"]["bytes"],
        "read_per_kernel": out["FETCH_SIZE"]["per_kernel_bytes"],
        "write_per_kernel": out["WRITE_SIZE"]["per_kernel_bytes"],
        "fetch_factor": out["FETCH_SIZE"]["factor"],
        "write_factor": out["WRITE_SIZE"]["factor"],
        "algorithmic_bytes": meta[3],
    }
    os.makedirs(os.path.dirname(args.traffic_json), exist_ok=True)
    with open(args.traffic_json, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({key: table[key]}))
    return 0


class _HipEvents:
    """Timing events made with hipEventCreateWithFlags(hipEventDisableSystemFence): a timing
    event does not need the system-scope release that torch's events ask for, which flushes
    L2 and leaves the stream idle for microseconds around the kernels it brackets.  Falls back
    to torch's events if the HIP runtime cannot be loaded by name."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self.ct = ctypes
        self.lib = None
        try:
            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            self.lib = lib
        except OSError:
            pass
        self.kind = "hip, no system fence" if self.lib else "torch"

    def new(self):
        if not self.lib:
            return torch.cuda.Event(enable_timing=True)
        e = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def record(self, e):
        if not self.lib:
            e.record()
            return
        rc = self.lib.hipEventRecord(e, self.ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        if not self.lib:
            return a.elapsed_time(b)
        f = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def free(self, events):
        if self.lib:
            for e in events:
                self.lib.hipEventDestroy(e)


def timed_steps(write, decode, K: int) -> dict:
    """The timed region: K steps of write() then decode() between two synchronisations, with
    nothing between the kernels (an event between two kernels idles the stream for
    microseconds).  Then the per-launch durations: K decode launches back to back, and K write
    launches back to back, each run bracketed by one pair of HIP events on the current stream
    (where both launch), so each figure is the run's length over K."""
    he = _HipEvents()
    whole = [he.new() for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    he.record(whole[0])
    for _ in range(K):
        write()
        decode()
    he.record(whole[1])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    def per_launch(fn, lead: int = 0) -> float:
        # `lead` decode calls go first so that the GPU is still busy while the host queues K
        # short launches: a kernel shorter than its host-side call would otherwise be timed
        # with the host's gaps between launches.
        e = [he.new() for _ in range(2)]
        torch.cuda.synchronize()
        for _ in range(lead):
            decode()
        he.record(e[0])
        for _ in range(K):
            fn()
        he.record(e[1])
        torch.cuda.synchronize()
        ms = he.elapsed_ms(e[0], e[1]) / K
        he.free(e)
        return ms

    decode_ms = per_launch(decode)
    # ~20 us of host time per queued write, covered by decode calls in front.
    lead = min(1000, int(K * 0.02 / max(decode_ms, 1e-3)) + 2)
    res = {
        "ms_per_step": (t1 - t0) * 1e3 / K,
        "gpu_ms_per_step": he.elapsed_ms(whole[0], whole[1]) / K,
        "decode_ms": decode_ms,
        "write_ms": per_launch(write, lead),
        "event_kind": he.kind,
    }
    he.free(whole)
    return res


def achievable_read(dev, gib: int = 2, reps: int = 10) -> dict:
    """Same-run ceiling: the hand-written streaming-read kernels of libpkvprobe.so over a `gib` GiB
    buffer, three access patterns at four grid sizes; the best one's median of `reps` launches (each
    between its own pair of HIP events)."""
    import ctypes

    from paged_kv_cache_276_amd import build as pkv_build

    if not os.path.exists(pkv_build.PROBE_LIBRARY):
        raise RuntimeError(f"{pkv_build.PROBE_LIBRARY} is not built (python -m paged_kv_cache_276_amd.build)")
    lib = ctypes.CDLL(pkv_build.PROBE_LIBRARY)
    lib.pkv_probe_stream_read.restype = ctypes.c_int
    lib.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(cus * 16, dtype=torch.int32, device=dev)
    he = _HipEvents()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    names = {0: "grid stride", 1: "contiguous per workgroup", 2: "contiguous per workgroup, non-temporal"}
    best = None
    tried = []
    for variant, per_cu in [(v, p) for v in (0, 1, 2) for p in (2, 4, 8, 16)]:
        blocks = cus * per_cu

        def launch():
            rc = lib.pkv_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks, variant,
                                           ctypes.c_void_p(sink.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError(f"pkv_probe_stream_read failed ({rc})")

        launch()
        launch()
        ev = [(he.new(), he.new()) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            he.record(e0)
            launch()
            he.record(e1)
        torch.cuda.synchronize()
        ms = statistics.median(he.elapsed_ms(e0, e1) for e0, e1 in ev)
        he.free([e for pair in ev for e in pair])
        gbs = nbytes / (ms * 1e-3) / 1e9
        tried.append({"variant": names[variant], "workgroups": blocks, "GBps": round(gbs, 1)})
        if best is None or gbs > best["GBps"]:
            best = {"GBps": gbs, "bytes": nbytes, "workgroups": blocks, "us": ms * 1e3, "variant": names[variant]}
    del buf, sink
    best["probe"] = "stream_read_kernel (libpkvprobe.so): 16-byte loads, 8 in flight per thread, 256 threads"
    best["tried"] = tried
    return best


def per_call_percentiles(fn, calls: int) -> dict:
    """Durations of `calls` single calls, each between its own pair of HIP events (outside the timed
    region): p10 / p50 / p90 in microseconds."""
    he = _HipEvents()
    ev = [(he.new(), he.new()) for _ in range(calls)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        he.record(e0)
        fn()
        he.record(e1)
    torch.cuda.synchronize()
    us = sorted(he.elapsed_ms(e0, e1) * 1e3 for e0, e1 in ev)
    he.free([e for pair in ev for e in pair])
    return {"p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
            "p90": float(np.percentile(us, 90)), "calls": calls}


PEAK_BF16_TFLOPS = 2500.0


def multi_roofline(flops: float, nbytes: float, seconds: float) -> dict:
    """The roof of a call with `flops` of bf16 matrix work over `nbytes` of algorithmic bytes: HBM below
    the ridge (8 TB/s x intensity < 2.5 PFLOP/s), the matrix cores above it; `frac` against that roof."""
    intensity = flops / nbytes
    if intensity * PEAK_HBM_GBS * 1e9 < PEAK_BF16_TFLOPS * 1e12:
        achieved = nbytes / seconds / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops / seconds / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof.update({"kernel": "paged_attn_decode_multi (one call)", "traffic": None,
                 "intensity_flop_per_byte": intensity,
                 "ridge_flop_per_byte": PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)})
    return roof


def bench_multi(args) -> int:
    """A step with several new tokens per sequence: paged_kv_write of the new tokens, then the causal
    multi-token attention.  value = new tokens per second; the roofline prices the attention call on the
    KV bytes read once per (sequence, KV head) plus q and out, and reports its matrix-core rate."""
    import paged_kv_cache_276_amd as pkv
    from workloads import make_multi_config

    dev = torch.device("cuda", 0)
    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    w = make_multi_config(args.config)
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, kn, vn = w.q.to(dev), w.k_new.to(dev), w.v_new.to(dev)
    sm = torch.from_numpy(w.slot_mapping).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    cl = torch.from_numpy(w.context_lens).to(dev)
    cu = torch.from_numpy(w.cu_q).to(dev)
    TQ = int(w.cu_q[-1])
    mq = int(np.max(np.diff(w.cu_q)))
    plan = pkv.paged_attn_multi_plan(w.num_seqs, TQ, mq, w.num_q_heads, w.max_blocks_per_seq, kc,
                                     chunk_tokens=args.partition_tokens, grid_waves=args.grid_waves)
    out = torch.empty((TQ, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = pkv.new_workspace(plan["workspace_bytes"], dev)  # zero-filled (the counter region)

    def write():
        pkv.paged_kv_write(kn, vn, sm, kc, vc)

    def attend():
        pkv.paged_attn_decode_multi(q, kc, vc, bt, cl, cu, mq, w.scale, out=out, workspace=ws,
                                    chunk_tokens=args.partition_tokens, grid_waves=args.grid_waves)

    for _ in range(args.warmup):
        write()
        attend()
    torch.cuda.synchronize()
    K = args.steps
    tm = timed_steps(write, attend, K)
    ms_per_step = tm["ms_per_step"]
    att = tm["decode_ms"] * 1e-3
    ctx = w.context_lens.astype(np.int64)
    ql = np.diff(w.cu_q).astype(np.int64)
    kv = int(ctx.sum()) * 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    qo = TQ * w.num_q_heads * w.head_dim * (w.elem_bytes + 4)
    # q.K and P.V over the visible tokens of every (new token, query head): 4 * head_dim flops per pair
    visible = int(sum(int(ql[i]) * int(ctx[i]) - int(ql[i]) * (int(ql[i]) - 1) // 2 for i in range(w.num_seqs)))
    flops = 4 * w.head_dim * visible * w.num_q_heads
    rec = {
        "metric": "multi-token attention new tokens/s (several new tokens per sequence, causal), 1 MI355X",
        "value": TQ / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.config, "num_seqs": w.num_seqs, "new_tokens": TQ, "max_q_len": mq,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "context_tokens": int(ctx.sum()),
                   "lengths": w.meta.get("lengths"), "chunk_tokens": plan["chunk_tokens"],
                   "kernel": "multi", "partition_tokens": plan["chunk_tokens"]},
        "roofline": multi_roofline(flops, kv + qo, att),
        "algorithmic_bytes": {"kv": kv, "q_out": qo, "total": kv + qo},
        "attention_us": att * 1e6,
        "mfma_TFLOPs": flops / att / 1e12,
        "mfma_frac_of_bf16_peak": flops / att / 2.5e15,
        "write_us": tm["write_ms"] * 1e3,
        "timing": {"gpu_us_per_step": tm["gpu_ms_per_step"] * 1e3, "events": tm["event_kind"],
                   "per_launch": "K launches back to back / K"},
    }
    rec["attention_us_per_call"] = per_call_percentiles(attend, min(K, 200))
    rec["roofline"]["traffic"] = _traffic_for(args, f"{args.config}/multi/T{plan['chunk_tokens']}")
    if args.copy_calibration_mib > 0:
        rec["copy_calibration_bytes"] = _calibration_copy(dev, args.copy_calibration_mib)
    if not args.no_parity:
        import oracle

        fresh = make_multi_config(args.config)
        o = oracle.Oracle()
        rk, rv = oracle._bits(fresh.k_cache).copy(), oracle._bits(fresh.v_cache).copy()
        o.kv_write(fresh.k_new, fresh.v_new, fresh.slot_mapping, rk, rv, fresh.block_size)
        ref = o.attn_multi(fresh.q, rk, rv, fresh.block_tables, fresh.context_lens, fresh.cu_q, fresh.scale)
        g = out.double().cpu().numpy()
        rec["parity"] = {"max_err_over_allowed": float(np.max(np.abs(g - ref) / (2e-3 + 1e-2 * np.abs(ref)))),
                         "finite": bool(np.isfinite(g).all())}
    rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def _traffic_for(args, key: str):
    """HBM bytes per launch that rocprofv3 counters measured for this workload and kernel family
    (profiles/traffic.json), or None when there is none for the current kernel sources."""
    if not os.path.exists(args.traffic_json):
        return None
    with open(args.traffic_json) as f:
        t = json.load(f)
    if key in t and t[key].get("source_sha") == _kernel_source_sha():
        return t[key]["bytes_per_launch"]
    return None


def _calibration_copy(dev, mib: int) -> int:
    """Three device-to-device copies of `mib` MiB (a copy of known size that scales byte counters)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return n


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.ingest_counters:
        return ingest_counters(args)
    if args.config.startswith("multi_"):
        if args.gpus != 1:
            print(json.dumps({"error": "this benchmark runs on exactly one GPU"}))
            return 2
        return bench_multi(args)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   "the multi-GPU path is a design note, not a measured configuration"}))
        return 2
    assert torch.cuda.is_available(), "no GPU visible"
    import paged_kv_cache_276_amd as pkv
    from workloads import make_config

    dev = torch.device("cuda", 0)
    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    heads = tuple(int(x) for x in args.heads.split(",")) if args.heads else None
    w = make_config(args.config, block_size=args.block_size or None, heads=heads)
    d = {
        "q": w.q.to(dev), "k_new": w.k_new.to(dev), "v_new": w.v_new.to(dev),
        "k_cache": w.k_cache.to(dev), "v_cache": w.v_cache.to(dev),
        "block_tables": torch.from_numpy(w.block_tables).to(dev),
        "context_lens": torch.from_numpy(w.context_lens).to(dev),
        "slot_mapping": torch.from_numpy(w.slot_mapping).to(dev),
    }
    if args.prefix:
        groups = w.meta.get("prefix_groups")
        if not groups:
            print(json.dumps({"error": f"--prefix needs a workload with shared prefixes, not {args.config}"}))
            return 2
        start = np.zeros(w.num_seqs, dtype=np.int32)
        grows = []
        for ptok, members in groups:
            start[members] = ptok
            for k in range(0, len(members), 8):
                grows.append((members[k], len(members[k:k + 8])))
        d["seq_prefix"] = torch.from_numpy(start).to(dev)
        d["groups"] = torch.from_numpy(np.array(grows, dtype=np.int32)).to(dev)
        max_prefix = int(start.max())
        plan = pkv.paged_attn_prefix_plan(w.num_seqs, w.num_q_heads, w.max_blocks_per_seq, len(grows), max_prefix,
                                          d["k_cache"], chunk_tokens=args.partition_tokens,
                                          grid_waves=args.grid_waves, xcd_balance=args.xcd_balance)
        plan["partition_tokens"] = plan["chunk_tokens"]
        plan["grid_blocks"] = args.grid_waves
        plan["kernel"] = "prefix"
    else:
        plan = pkv.paged_attn_plan(w.num_seqs, w.num_q_heads, w.max_blocks_per_seq, d["k_cache"],
                                   partition_tokens=args.partition_tokens, kernel=args.kernel,
                                   grid_waves=args.grid_waves, xcd_balance=args.xcd_balance)
    out = torch.empty((w.num_seqs, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    ws = pkv.new_workspace(plan["workspace_bytes"], dev)

    def write():
        pkv.paged_kv_write(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"])

    def decode():
        if args.prefix:
            pkv.paged_attn_decode_prefix(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                         d["seq_prefix"], d["groups"], max_prefix, w.scale, out=out, workspace=ws,
                                         chunk_tokens=args.partition_tokens, grid_waves=args.grid_waves,
                                         xcd_balance=args.xcd_balance)
        else:
            pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                                  w.scale, out=out, workspace=ws, partition_tokens=args.partition_tokens,
                                  kernel=args.kernel, grid_waves=args.grid_waves, xcd_balance=args.xcd_balance)

    print(f"[bench] warmup {args.warmup} steps, plan {plan}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        write()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    tm = timed_steps(write, decode, K)
    print(f"[bench] timed {K} steps", file=sys.stderr, flush=True)
    launched = pkv.last_launch_info()  # the grid and XCD shares the library chose
    ms_per_step = tm["ms_per_step"]
    dec_avg = tm["decode_ms"]
    nbytes = algorithmic_bytes(w)
    # The prefix path has to move each shared block once: it is priced on the unique bytes.
    moved = nbytes["total_unique"] if args.prefix else nbytes["total"]
    achieved = moved / (dec_avg * 1e-3) / 1e9
    kv_gbs = nbytes["kv"] / (dec_avg * 1e-3) / 1e9

    key = (f"{args.config}/{plan['kernel']}/T{plan['partition_tokens']}" + (f"/B{w.block_size}" if args.block_size else "")
           + (f"/H{w.num_q_heads}-{w.num_kv_heads}-{w.head_dim}" if heads else ""))
    traffic = _traffic_for(args, key)

    rec = {
        "metric": METRIC,
        "value": w.num_seqs / (ms_per_step * 1e-3),
        "unit": "seqs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.config,
            "num_seqs": w.num_seqs,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "context_tokens": int(w.context_lens.sum()),
            "lengths": w.meta.get("lengths", "fixed"),
            "slack_tokens": int(((w.context_lens.astype(np.int64) + w.block_size - 1) // w.block_size).sum()
                                * w.block_size - w.context_lens.astype(np.int64).sum()),
            "table_entries": int(((w.context_lens.astype(np.int64) + w.block_size - 1) // w.block_size).sum()),
            "kernel": plan["kernel"],
            "partition_tokens": plan["partition_tokens"],
            "grid_waves": launched["grid"] if launched["kernel"] == "fast" else plan["grid_blocks"],
            "xcd_balance": launched["xcd_balance"] if launched["kernel"] == "fast" else None,
            "k_loads": (("streamed" if launched["k_stream"] else "cached") if launched["kernel"] == "fast" else None),
        },
        "roofline": {
            "kernel": ("paged_attn_decode_prefix (prefix, suffix and merge kernels, one call; unique bytes)"
                       if args.prefix else "paged_attn_decode (partition + merge kernels, one call)"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
        },
        "kv_read_GBps": kv_gbs,
        "kv_unique_GBps": nbytes["kv_unique"] / (dec_avg * 1e-3) / 1e9,
        "kv_read_pct_of_peak": 100.0 * kv_gbs / PEAK_HBM_GBS,
        "decode_us": dec_avg * 1e3,
        "write_us": tm["write_ms"] * 1e3,
        "timing": {"gpu_us_per_step": tm["gpu_ms_per_step"] * 1e3, "events": tm["event_kind"],
                   "per_launch": "K launches back to back / K"},
        "algorithmic_bytes": nbytes,
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "hip": torch.version.hip,
    }

    rec["decode_us_per_call"] = per_call_percentiles(decode, min(K, 200))
    if not args.no_achievable:
        ach = achievable_read(dev)
        rec["achievable_GBps"] = ach["GBps"]
        rec["achievable_read"] = ach
        rec["roofline"]["pct_of_achievable"] = 100.0 * achieved / ach["GBps"]

    if args.cold_steps > 0:
        # The flush only reads: a written flush would leave dirty lines whose write-back
        # lands inside the timed call.
        scratch = torch.zeros(args.flush_mib << 18, dtype=torch.float32, device=dev)
        decode()  # evicts the zero fill's dirty lines before the first timed call
        cold = []
        he = _HipEvents()
        for i in range(args.cold_steps):
            sink = scratch.sum()
            e0, e1 = he.new(), he.new()
            he.record(e0)
            decode()
            he.record(e1)
            torch.cuda.synchronize()
            cold.append(he.elapsed_ms(e0, e1) * 1e3)
            he.free([e0, e1])
        rec["decode_us_cold"] = statistics.median(cold)
        rec["kv_read_GBps_cold"] = nbytes["kv"] / (rec["decode_us_cold"] * 1e-6) / 1e9
        del scratch, sink

    if args.copy_calibration_mib > 0:
        rec["copy_calibration_bytes"] = _calibration_copy(dev, args.copy_calibration_mib)

    if not args.no_parity:
        import oracle
        from workloads import make_config as _mk

        fresh = _mk(args.config, block_size=args.block_size or None, heads=heads)  # pre-write state; the pool was rewritten K+W times (same slots)
        ref = oracle.decode_step(fresh)
        g = out.double().cpu().numpy()
        err = np.abs(g - ref.out)
        rec["parity"] = {
            "max_err_over_allowed": float(np.max(err / (2e-3 + 1e-2 * np.abs(ref.out)))),
            "finite": bool(np.isfinite(g).all()),
        }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


def _strip_comments(text: str) -> str:
    """C/C++ source without comments and blank space, so that comment edits keep the stamp.
    Naive about comment markers inside string literals, which the kernel sources do not use."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _kernel_source_sha(csrc: str = None) -> str:
    """Stamp of the kernel sources (their code, comments and layout excluded)."""
    import hashlib

    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "paged_kv_cache_276_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
