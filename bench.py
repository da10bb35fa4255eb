"""Benchmark of the paged-attention hot path on one GPU.

Default workload (the metric's configuration), one step = reshape_and_cache of
the 256 newest tokens, then paged decode of 256 sequences at Llama-2-13B shape
(40 query heads = 40 kv heads, head_dim 128, bf16 cache, block size 16,
lognormal context lengths with median 1024 clipped to [16, 4096], 65536-block
shuffled pool) with split-K partitions and their merge.

--workload selects the other shapes the hot path is measured on:
  llama7b   decode of 64 sequences, 32 = 32 heads, lengths U[128, 2048], 2048-token
            split-K partitions + merge
  gqa       decode of 32 sequences, 32 query heads over 8 kv heads, lengths
            U[8192, 32768], 512-token split-K partitions + merge
  mixed     chunked prefill of 4 x 512-token chunks over paged prefixes, then
            decode of 192 sequences sharing 2048-token prefixes in groups of 3
            (also timed with prefill and decode on two streams)
  mixed_gqa, mixed_gqa_fp8
            the mixed step with 32 query heads over 8 kv heads (Llama-3-8B shape);
            mixed_gqa splits the prefill into 2048-key runs
  llama13b_fp8, gqa_fp8, mixed_fp8
            the llama13b, gqa and mixed steps over an FP8 (OCP E4M3) cache with
            one scale per pool: quantising scatter (llama13b), chunked prefill
            (mixed), decode, merge; KV bytes count one byte per element
  prefill_long  4 chunks of 128 tokens over 16384-token paged prefixes (40
            heads): the split prefill (runs of 5504 keys) against one workgroup
            per query tile; with one 128-row query tile per (sequence, kv head)
            the K/V stream bounds it, so its roofline is HBM (K/V bytes read
            once), the TFLOP/s metric beside it
  prefix_cache  32 prompts at Llama-2-13B shape sharing a 2048-token system
            prompt, each with 256 tokens of its own: the chunked prefill of
            all 32 with prefix-cache hits (256 query tokens each over the
            cached 2048) against the same prompts prefilled whole, and the
            block manager's host time to look the prompts up
  sampler   the next-token draw for 256 rows of a 32000-token vocabulary (Llama 2),
            fp32 logits, temperature / top-k / top-p cycling through the
            pages' example (0.7, 50, 0.9) and other settings
  block_moves  the data movement around the step at the Llama-2-13B pool shape:
            copy-on-write block copies (pa_copy_blocks, 1024 pairs in one call;
            the metric of that line is its read + write GB/s), swaps to and
            from pinned host memory (pa_swap_blocks), and the native block
            manager's host time for one decode step of 256 sequences
  stream_read  the part's achievable HBM read rate: plain 16-byte loads over a
            4 GiB buffer (pa_stream_read), the ceiling the HBM-bound kernels
            are compared with; the default line reports it too

Inputs are seeded synthetic data already resident in GPU memory before timing
starts.  Prints one JSON line: KV GB/s over the whole step (the metric), % of
the 8 TB/s HBM peak, tokens/s for one layer, the dominant kernel's roofline
position (algorithmic bytes or flops / its own launch time, from HIP events on
the launch stream), and the fp64 CPU oracle timed on a sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged-attn decode KV GB/s (% of HBM peak) + tokens/s at Llama-2-13B shape"
_CSRC = os.path.join(ROOT, "paged_kv_cache_453_amd", "csrc")
# kernels whose HBM traffic comes from committed counter runs: the summary file,
# the kernel name prefix in the rocprofv3 CSVs, the sources the kernel is built
# from, and the bench command the counter runs profiled
_DECODE_SOURCES = [os.path.join(_CSRC, f) for f in
                   ("decode_valu.h", "decode_groups.h", "decode_valu_bf16.hip", "pa_device.h",
                    "decode.hip", "pa_launch.h")]
COUNTED = {
    "decode": {
        "json": os.path.join(ROOT, "profiles", "decode_llama13b_counters.json"),
        # told apart by its grid from the Llama-2-7B-shaped launch of the same kernel
        "kernel": [("void pa::decode_valu_dealt_kernel<unsigned short, unsigned short, 128, 1>",
                    5648384)],
        "sources": _DECODE_SOURCES,
        "bench": "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline",
        "dir": "pmc", "out": "bench"},
    # one pa_decode_shared_prefix call on the mixed workload's decoders: the grouped
    # pass and the regular pass, summed per call
    "mixed_decode": {
        "json": os.path.join(ROOT, "profiles", "decode_mixed_counters.json"),
        "kernel": ["void pa::decode_valu_kernel<unsigned short, unsigned short, 128, 3, false, true>",
                   "void pa::decode_valu_kernel<unsigned short, unsigned short, 128, 1, true, false>"],
        "sources": _DECODE_SOURCES,
        "bench": "python3 bench.py --workload mixed --decode-only --steps 3 --warmup 1",
        "dir": "pmc_mixed", "out": "mixed"},
    # the same decoders through pa_decode (each sample reads the shared prefix itself)
    "mixed_decode_plain": {
        "json": os.path.join(ROOT, "profiles", "decode_mixed_plain_counters.json"),
        "kernel": ["void pa::decode_valu_kernel<unsigned short, unsigned short, 128, 1, true, false>"],
        "sources": _DECODE_SOURCES,
        "bench": "python3 bench.py --workload mixed --decode-only --no-prefix-groups --steps 3 "
                 "--warmup 1",
        "dir": "pmc_mixed_plain", "out": "mixed"},
    # the Llama-2-7B-shaped batch (the headline kernel, other lengths and partitions)
    "decode_7b": {
        "json": os.path.join(ROOT, "profiles", "decode_llama7b_counters.json"),
        "kernel": [("void pa::decode_valu_dealt_kernel<unsigned short, unsigned short, 128, 1>",
                    573440)],
        "sources": _DECODE_SOURCES,
        "bench": "python3 bench.py --workload llama7b --decode-only --steps 3 --warmup 1",
        "dir": "pmc_7b", "out": "l7b"},
    # the GQA long-context batch on the matrix-core decode
    "decode_gqa": {
        "json": os.path.join(ROOT, "profiles", "decode_gqa_counters.json"),
        "kernel": "void pa::decode_gqa_mfma_kernel<unsigned short, false, false, true>",
        "sources": [os.path.join(_CSRC, f) for f in
                    ("decode_mfma.hip", "decode_groups.h", "pa_device.h")],
        "bench": "python3 bench.py --workload gqa --decode-only --steps 3 --warmup 1",
        "dir": "pmc_gqa", "out": "gqa"},
    # the long-prefix split prefill: the key-run launch (told apart from the
    # unsplit comparison launch of the same kernel by its grid) and the merge
    "prefill_long": {
        "json": os.path.join(ROOT, "profiles", "prefill_long_counters.json"),
        "kernel": [("void pa::prefill_x32_kernel<128, 4, true>", 122880),
                   "void pa::prefill_merge_kernel<128, 128>"],
        "sources": [os.path.join(_CSRC, f) for f in ("prefill.hip", "pa_device.h", "pa_launch.h")],
        "bench": "python3 bench.py --workload prefill_long --steps 3 --warmup 1 --no-cpu-baseline",
        "dir": "pmc_pl", "out": "pl"},
    "copy": {
        "json": os.path.join(ROOT, "profiles", "copy_blocks_13b_counters.json"),
        "kernel": "void pa::move_blocks_kernel<unsigned int __vector(4), pa::DeviceMapping>",
        "sources": [os.path.join(_CSRC, f) for f in ("copy_blocks.hip", "pa_device.h")],
        "bench": "python3 bench.py --workload block_moves --steps 3 --warmup 1 "
                 "--no-cpu-baseline",
        "dir": "pmc_bm", "out": "bm"},
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(kind: str) -> str:
    h = hashlib.sha256()
    for path in COUNTED[kind]["sources"]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch of the counted kernel from committed rocprofv3 counter
    runs, or None when they are missing or were taken on a different source."""
    try:
        with open(COUNTED[kind]["json"]) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256_16") != source_digest(kind):
        return None
    return c.get("hbm_bytes_per_launch")


FP8_K_SCALE, FP8_V_SCALE = 0.07, 0.11


def cpu_baseline(w, budget_s: float = 10.0, fp8_pools=None, threads: int = 1):
    """The fp64 oracle on a bounded sample of the same workload, with its BLAS
    limited to `threads` host threads.

    Decode: the first sequences in order (scatter included where the workload
    has one) until budget_s of CPU time.  Prefill (mixed workload): the first
    chunk first, then decode sequences.  Reported in the metric's unit, KV GB/s
    of decode over the sample.  fp8_pools: (k codes, v codes) of an FP8 cache,
    run through the FP8 oracle instead.
    """
    from threadpoolctl import threadpool_limits

    import oracle
    from oracle import kv_fp8
    from workloads import accounting

    fp8 = fp8_pools is not None
    k, v = fp8_pools if fp8 else (w.k_host, w.v_host)
    t_total = 0.0
    notes = []
    with threadpool_limits(threads):
        if w.slot_mapping is not None:
            t0 = time.perf_counter()
            if fp8:
                k, v = kv_fp8.reshape_and_cache(k, v, w.new_k, w.new_v, w.host_slots(), w.dtype,
                                                FP8_K_SCALE, FP8_V_SCALE)
            else:
                k, v = oracle.reshape_and_cache(k, v, w.new_k, w.new_v, w.host_slots())
            t_total += time.perf_counter() - t0
            notes.append(f"scatter of {len(w.slot_mapping)} tokens")
        if w.prefill is not None:
            p = w.prefill
            qsl = p.query_start_loc
            t0 = time.perf_counter()
            if fp8:
                kv_fp8.prefill(p.query[qsl[0]:qsl[1]], k, v, w.host_tables(p.block_tables[:1]),
                               qsl[:2] - qsl[0], p.context_lens[:1], w.scale, FP8_K_SCALE,
                               FP8_V_SCALE, w.dtype)
            else:
                oracle.prefill(p.query[qsl[0]:qsl[1]], k, v, w.host_tables(p.block_tables[:1]),
                               qsl[:2] - qsl[0], p.context_lens[:1], w.scale, w.dtype)
            dt = time.perf_counter() - t0
            t_total += dt
            notes.append(f"prefill of the first {int(qsl[1] - qsl[0])}-token chunk "
                         f"({dt:.1f} s)")
        g = w.decode
        tables = w.host_tables(g.block_tables)
        done, t_dec = 0, 0.0
        while done < g.num_seqs and t_total + t_dec < budget_s:
            hi = min(g.num_seqs, done + 8)
            t0 = time.perf_counter()
            if fp8:
                kv_fp8.decode(g.query[done:hi], k, v, tables[done:hi], g.context_lens[done:hi],
                              w.scale, FP8_K_SCALE, FP8_V_SCALE, w.dtype)
            else:
                oracle.decode(g.query[done:hi], k, v, tables[done:hi], g.context_lens[done:hi],
                              w.scale, w.dtype)
            t_dec += time.perf_counter() - t0
            done = hi
    kv = accounting.decode_kv_bytes(g.context_lens[:done], w.num_kv_heads, w.head_dim,
                                    1 if fp8 else w.elem_bytes)
    notes.append(f"decode of the first {done} of {g.num_seqs} sequences "
                 f"({int(g.context_lens[:done].sum())} tokens, {t_dec:.1f} s)")
    return {"value": round(kv / t_dec / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fp64 numpy oracle, BLAS limited to {threads} host thread(s): " +
                      "; ".join(notes) + "; value = decode KV bytes / decode time"}


def host_description():
    """The host the CPU baseline runs on: cores this process may use (its
    affinity mask), capped by OMP_NUM_THREADS where the box sets its CPU share
    there; the CPU model; the BLAS numpy calls."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    threads = affinity
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        threads = min(threads, int(omp))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy  # noqa: F401  (loads its BLAS so threadpoolctl can see it)
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in libs)
    except Exception:  # pragma: no cover
        pass
    return {"affinity_cores": affinity, "threads": threads, "cpu_model": model, "blas": blas}


def cpu_baseline_report(w, fp8_pools=None):
    """The oracle baseline on every core this process may use (the reported
    value), and again on one thread for reference."""
    host = host_description()
    allc = cpu_baseline(w, budget_s=10.0, fp8_pools=fp8_pools, threads=host["threads"])
    one = cpu_baseline(w, budget_s=6.0, fp8_pools=fp8_pools, threads=1)
    allc.update({"affinity_cores": host["affinity_cores"], "cpu_model": host["cpu_model"],
                 "blas": host["blas"],
                 "one_thread": {"value": one["value"], "unit": one["unit"],
                                "sample": one["sample"]}})
    return allc


def other_configs(args, torch, dev, lib):
    """The other decode configurations, each timed like the headline step:
    the Llama-2-7B-shaped batch, the GQA long-context batch (512-token split-K
    partitions as configured) and the mixed prefill + decode step."""
    out = {}
    for name, ps in (("llama7b", 2048), ("gqa", 512), ("mixed", 2048)):
        r = bench_attention(args, torch, dev, lib, name, partition_size=ps, with_cpu=False)
        torch.cuda.empty_cache()
        rf = r["roofline"]
        entry = {"workload": r["config"]["workload"], "num_seqs": r["config"]["num_seqs"],
                 "partition_size": ps, "ms_per_step": r["ms_per_step"],
                 "ms_per_step_p10_p50_p90": r["ms_per_step_p10_p50_p90"],
                 "kv_gbs": r["value"], "pct_hbm_peak": r["pct_hbm_peak"],
                 "tokens_per_s": r["tokens_per_s"], "kernel_us": r["kernel_us"],
                 "kv_bytes_per_step": r["kv_bytes_per_step"],
                 "decode_roofline": {"achieved": rf["achieved"], "frac": rf["frac"],
                                     "unit": rf["unit"], "kernel": rf["kernel"],
                                     "traffic": rf["traffic"]}}
        if "roofline_prefill" in r:
            pf = r["roofline_prefill"]
            entry["value_note"] = r["value_note"]
            entry["kv_gbs_logical"] = r["kv_gbs_logical"]
            entry["kv_bytes_unique_per_step"] = r["kv_bytes_unique_per_step"]
            entry["decode_roofline"]["logical_gbs"] = rf.get("logical_gbs")
            entry["prefill_roofline"] = {"achieved": pf["achieved"], "frac": pf["frac"],
                                         "unit": pf["unit"], "kernel": pf["kernel"]}
            entry["overlapped_two_streams"] = r["overlapped_two_streams"]
        out[name] = entry
        log(f"bench: {name}: {json.dumps(entry)}")
    return out


def _counter_rows(path: str, kernel):
    """Counter values of the dispatches of `kernel`: a name prefix, or a
    (name prefix, grid size in threads) pair."""
    import csv
    prefix, grid = kernel if isinstance(kernel, tuple) else (kernel, None)
    with open(path) as f:
        return [float(r["Counter_Value"]) for r in csv.DictReader(f)
                if r["Kernel_Name"].startswith(prefix)
                and (grid is None or int(r["Grid_Size"]) == grid)]


def digest_counters(kind: str, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                    copy_write_csv: str, copy_bytes: int = 1 << 30) -> int:
    """Turn four rocprofv3 --pmc runs into HBM bytes per launch of a kernel.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Each is scaled by
    what the same counter reads for a plain copy of copy_bytes (which reads and
    writes exactly copy_bytes), so the result is in true bytes whatever share of
    the memory channels the counter sees.  Writes the committed summary that
    bench.py reports as roofline.traffic while the kernel's sources are
    unchanged.
    """
    import statistics
    spec = COUNTED[kind]
    k = spec["kernel"]
    copy = "__amd_rocclr_copyBuffer"
    # several kernels: one launch of each per call, the call's traffic is their sum
    ks = k if isinstance(k, list) else [k]
    f_k = sum(statistics.mean(_counter_rows(fetch_csv, x)) for x in ks)
    w_k = sum(statistics.mean(_counter_rows(write_csv, x)) for x in ks)
    f_copy = statistics.mean(_counter_rows(copy_fetch_csv, copy))
    w_copy = statistics.mean(_counter_rows(copy_write_csv, copy))
    f_scale = copy_bytes / (f_copy * 1024)
    w_scale = copy_bytes / (w_copy * 1024)
    hbm = f_k * 1024 * f_scale + w_k * 1024 * w_scale
    d, o = spec["dir"], spec["out"]
    out = {"kernel": k if isinstance(k, str) else
           [x if isinstance(x, str) else f"{x[0]} (grid {x[1]})" for x in ks],
           "source_sha256_16": source_digest(kind),
           "fetch_kib_per_launch": round(f_k, 1), "write_kib_per_launch": round(w_k, 1),
           "copy_bytes": copy_bytes, "copy_fetch_kib": round(f_copy, 1),
           "copy_write_kib": round(w_copy, 1), "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "hbm_bytes_per_launch": int(round(hbm)),
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/{d}_fetch -o {o} -- "
               + spec["bench"],
               f"rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/{d}_write -o {o} -- "
               + spec["bench"],
               "rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/pmc_copy_fetch -o copy -- "
               "python3 bench.py --copy-calibration",
               "rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/pmc_copy_write -o copy -- "
               "python3 bench.py --copy-calibration"]}
    os.makedirs(os.path.dirname(spec["json"]), exist_ok=True)
    with open(spec["json"], "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration(torch, dev, nbytes: int = 1 << 30, reps: int = 3) -> int:
    """A plain copy of known size: reads nbytes, writes nbytes per launch."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "ms_per_copy": round(ms, 4),
                      "gbs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


class StepTimer:
    """Times launches with HIP events recorded on the stream each launch uses."""

    def __init__(self, torch):
        self.torch = torch

    def per_step(self, step, steps: int, streams) -> float:
        """Milliseconds per step of `step()` over `steps` calls, all streams joined.
        Events between the steps (on the first stream) also give each step's own
        time; their 10th, 50th and 90th percentiles are kept in `self.spread`."""
        torch = self.torch
        main = streams[0]
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        a.record(main)
        for i in range(steps):
            step()
            if len(streams) == 1:
                marks[i].record(main)
        for s in streams[1:]:
            e = torch.cuda.Event()
            e.record(s)
            main.wait_event(e)
        b.record(main)
        torch.cuda.synchronize()
        if len(streams) == 1:
            each = sorted([a.elapsed_time(marks[0])] +
                          [marks[i - 1].elapsed_time(marks[i]) for i in range(1, steps)])
            pick = lambda q: each[min(len(each) - 1, int(q * len(each)))]
            self.spread = [round(pick(0.1), 5), round(pick(0.5), 5), round(pick(0.9), 5)]
        return a.elapsed_time(b) / steps

    def per_launch(self, launches, steps: int, stream):
        """Average milliseconds of each launch in `launches` (name, fn) run in order
        on one stream, from events recorded on that stream around each launch."""
        torch = self.torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
               for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            evs[i][0].record(stream)
            for k, (_, fn) in enumerate(launches):
                fn()
                evs[i][k + 1].record(stream)
        torch.cuda.synchronize()
        return {name: sum(e[k].elapsed_time(e[k + 1]) for e in evs) / steps
                for k, (name, _) in enumerate(launches)}


STREAM_BYTES = 4 << 30
STREAM_METRIC = "achievable HBM read GB/s (plain 16-byte loads over a 4 GiB buffer)"
WORKLOADS = ("llama13b", "llama7b", "gqa", "mixed", "llama13b_fp8", "gqa_fp8", "mixed_fp8",
             "mixed_gqa", "mixed_gqa_fp8", "prefix_cache", "prefill_long",
             "sampler", "block_moves", "stream_read")
SAMPLER_BUFFERS = 9
SAMPLER_METRIC = "next-token sampling rows/s (temperature + top-k + top-p + draw), 32000-token vocabulary"
PREFIX_METRIC = ("prefill us for 32 prompts sharing a 2048-token system prompt, with prefix-cache "
                 "hits, at Llama-2-13B shape")
LONG_PREFILL_METRIC = ("chunked prefill TFLOP/s, 4 chunks of 128 tokens over 16384-token paged "
                       "prefixes at Llama-2-13B head shape, split over the keys")
COPY_METRIC = "paged KV block copy GB/s (copy-on-write, read + write bytes) at Llama-2-13B pool shape"


def build_workload(name: str, ps: int):
    from workloads import config1, config2, config3, config4
    if name == "llama13b":
        return config2(partition_size=ps), {
            "workload": "llama2-13b-shaped paged decode (scatter + decode + split-K merge)",
            "context_lens": "lognormal median 1024 sigma 0.5 clipped [16,4096]", "seed": 455}
    if name == "llama7b":
        return config1(partition_size=ps), {
            "workload": "llama2-7b-shaped paged decode (decode + split-K merge)",
            "context_lens": "uniform [128,2048]", "seed": 454}
    if name == "gqa":
        return config3(partition_size=ps), {
            "workload": "llama3-8b-shaped GQA long-context paged decode (decode + split-K merge)",
            "context_lens": "uniform [8192,32768]", "seed": 456}
    if name == "mixed_gqa":
        return config4(partition_size=ps, heads=32, kv_heads=8), {
            "workload": "mixed chunked prefill + shared-prefix paged decode, grouped-query "
                        "heads (Llama-3-8B shape: 32 query heads over 8 kv heads)",
            "prefill": "4 x 512-token causal chunks over paged prefixes U{0..3584}",
            "decode": "64 prompts x 3 samples sharing 2048-token prefixes + U{0..512} private",
            "seed": 457}
    return config4(partition_size=ps), {
        "workload": "mixed chunked prefill + shared-prefix paged decode",
        "prefill": "4 x 512-token causal chunks over paged prefixes U{0..3584}",
        "decode": "64 prompts x 3 samples sharing 2048-token prefixes + U{0..512} private",
        "seed": 457}


def stream_read_gbs(torch, dev, lib, timer, launches: int = 20) -> float:
    """The part's achievable read rate: pa_stream_read over a 4 GiB buffer
    (GB/s, 1e9), the ceiling the HBM-bound kernels are compared with."""
    buf = torch.ones(STREAM_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(lib.pa_stream_read_sink_words(), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    run = lambda: lib.pa_stream_read(buf, sink, stream=stream)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ms = timer.per_launch([("read", run)], launches, stream)["read"]
    del buf
    return STREAM_BYTES / (ms * 1e-3) / 1e9


def bench_stream_read(args, torch, dev, lib, timer) -> int:
    """The stream-read calibration as its own line."""
    log(f"bench: timing {args.steps} stream-read launches over {STREAM_BYTES >> 30} GiB")
    gbs = stream_read_gbs(torch, dev, lib, timer, args.steps)
    ms = STREAM_BYTES / gbs / 1e6
    result = {
        "metric": STREAM_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": 3, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "read of a 4 GiB device buffer, nontemporal 16-byte loads, "
                               "grid-stride, a 32-bit fold per workgroup"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "stream_read_kernel", "algorithmic_bytes_per_launch": STREAM_BYTES},
        "cpu_baseline": None,
        "cpu_baseline_note": "a calibration of the GPU's memory, with no CPU counterpart",
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_block_moves(args, torch, dev, lib, timer) -> int:
    """pa_copy_blocks / pa_swap_blocks throughput and block-manager host time."""
    import numpy as np

    nb, hkv, d, bs, pairs_n = 65536, 40, 128, 16, 1024
    block_bytes = hkv * bs * d * 2
    log("bench: allocating two 10 GiB bf16 pools")
    g = torch.Generator(device=dev).manual_seed(453)
    kc = torch.randint(-2**15, 2**15, (nb, hkv, bs, d), dtype=torch.int16, device=dev,
                       generator=g).view(torch.bfloat16)
    vc = torch.randint(-2**15, 2**15, (nb, hkv, bs, d), dtype=torch.int16, device=dev,
                       generator=g).view(torch.bfloat16)
    rng = np.random.default_rng(453)
    ids = rng.permutation(nb)
    pairs = np.stack([rng.choice(ids[pairs_n:], pairs_n), ids[:pairs_n]], 1).astype(np.int32)
    mapping = torch.from_numpy(pairs).to(dev)
    stream = torch.cuda.current_stream()

    def copy():
        lib.pa_copy_blocks(kc, vc, mapping, stream=stream)

    for _ in range(args.warmup):
        copy()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} copy launches")
    ms = timer.per_launch([("copy_blocks", copy)], args.steps, stream)["copy_blocks"]
    algo = 2 * 2 * pairs_n * block_bytes              # K and V, read + write
    gbs = algo / (ms * 1e-3) / 1e9

    # swaps: 256 scattered blocks, and one run of 256 consecutive blocks
    nh, sw = 1024, 256
    hk = torch.empty((nh, hkv, bs, d), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((nh, hkv, bs, d), dtype=torch.bfloat16, pin_memory=True)
    scattered = np.stack([rng.choice(nb, sw, replace=False),
                          rng.choice(nh, sw, replace=False)], 1).astype(np.int32)
    run = np.stack([np.arange(4096, 4096 + sw), np.arange(sw)], 1).astype(np.int32)
    swaps = {}
    for name, m in (("scattered", scattered), ("one_run", run)):
        for direction, (a, b) in (("out", ((kc, vc), (hk, hv))), ("in", ((hk, hv), (kc, vc)))):
            src_m = m if direction == "out" else m[:, ::-1].copy()

            def sw_call(a=a, b=b, src_m=src_m):
                lib.pa_swap_blocks(a[0], a[1], b[0], b[1], src_m, stream=stream)

            sw_call()
            torch.cuda.synchronize()
            t = timer.per_step(sw_call, max(3, args.steps // 5), [stream])
            swaps[f"{direction}_{name}"] = {
                "ms": round(t, 4), "gbs": round(2 * sw * block_bytes / (t * 1e-3) / 1e9, 2)}
    log("bench: swaps " + ", ".join(f"{k} {v['gbs']} GB/s" for k, v in swaps.items()))

    # block manager host time for one decode step of 256 sequences
    bm = lib.BlockManager(nb, bs, 0)
    seqs = np.arange(256, dtype=np.int64)
    lens = np.clip(np.round(rng.lognormal(np.log(1024), 0.5, 256)), 16, 4096).astype(np.int32)
    for s_, n_ in zip(seqs, lens):
        bm.add_sequence(int(s_))
        bm.append_slots(int(s_), int(n_) - 1)
    bm.take_moves()
    ones = np.ones(256, dtype=np.int32)
    reps = 200
    t0 = time.perf_counter()
    for _ in range(reps):
        slots, done, st = bm.append_batch(seqs, ones)
        bm.take_moves()
        tables, cl, sh = bm.build_batch(seqs, 320)
    host_us = (time.perf_counter() - t0) / reps * 1e6

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("bench: timing the CPU oracle block copy on a sample")
        nbs = 2048
        kp = np.zeros((nbs, hkv, bs, d), dtype=np.uint16)
        sp = pairs[:64] % nbs
        sp = sp[np.unique(sp[:, 1], return_index=True)[1]]
        t0 = time.perf_counter()
        n_calls = 0
        while time.perf_counter() - t0 < 10.0:
            oracle.copy_blocks(kp, sp)
            n_calls += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(2 * len(sp) * block_bytes * n_calls / el / 1e9, 3),
               "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"oracle.copy_blocks on one {nbs}-block 13B-shaped pool, {len(sp)} "
                         f"pairs, {n_calls} calls in {el:.1f} s (the oracle returns a copied "
                         "pool, so each call also copies the whole pool)"}

    result = {
        "metric": COPY_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "copy-on-write block copies, 1024 pairs, Llama-2-13B pools "
                               "(65536 blocks x 40 kv heads x 16 x 128 bf16, 10 GiB each)",
                   "pairs": pairs_n, "block_bytes_per_pool": block_bytes, "seed": 453},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("copy"),
                     "kernel": "move_blocks_kernel<u32x4, DeviceMapping>",
                     "algorithmic_bytes_per_launch": int(algo)},
        "swap_blocks_256": swaps,
        "swap_note": "pa_swap_blocks between the device pools and pinned host pools, K and V "
                     "(2 x 256 x 160 KiB), GB/s over PCIe, one kernel launch per call; "
                     "scattered = 256 random block ids, one_run = 256 consecutive ids",
        "block_manager_host_us_per_step": round(host_us, 1),
        "block_manager_note": "append_batch (1 token x 256 sequences) + take_moves + "
                              "build_batch (256 x 320 table) through the C ABI from Python",
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_prefix_cache(args, torch, dev, lib, timer) -> int:
    """Chunked prefill with and without prefix-cache hits, and the lookups."""
    import numpy as np

    from workloads import accounting

    hq = hkv = 40
    d, n, sys_len, own = 128, 32, 2048, 256
    total = sys_len + own
    scale = float(np.float32(1 / np.sqrt(d)))
    rng = np.random.default_rng(453)
    system = rng.integers(0, 32000, sys_len).astype(np.int32)
    prompts = [np.concatenate([system, rng.integers(0, 32000, own).astype(np.int32)])
               for _ in range(n + 1)]

    # the block manager: an earlier request with the same system prompt fills
    # the cache, then the 32 prompts are looked up
    nb = 16384
    bm = lib.BlockManager(nb)
    bm.add_prompt(0, prompts[n])
    bm.append_tokens(0, prompts[n])
    bm.take_moves()
    t0 = time.perf_counter()
    cached = []
    for i in range(1, n + 1):
        c = bm.add_prompt(i, prompts[i - 1])
        bm.append_tokens(i, prompts[i - 1][c:])
        cached.append(c)
    bm.take_moves()
    host_us = (time.perf_counter() - t0) * 1e6
    mb = total // 16
    hit_tables, hit_lens, _ = bm.build_batch(list(range(1, n + 1)), mb)
    assert all(c == sys_len for c in cached), cached

    # pools of random bf16 contents, every block any table names
    g = torch.Generator(device=dev).manual_seed(453)
    kc = torch.randn((nb, hkv, 16, d), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((nb, hkv, 16, d), generator=g, device=dev).to(torch.bfloat16)
    # whole prompts: each its own 144 blocks
    whole_tables = np.arange(n * mb, dtype=np.int32).reshape(n, mb) + 1024

    def batch(tables, chunk):
        qsl = np.arange(n + 1, dtype=np.int32) * chunk
        lens = np.full(n, total, dtype=np.int32)
        q = torch.randn((n * chunk, hq, d), generator=g, device=dev).to(torch.bfloat16)
        return (q, torch.empty_like(q), torch.from_numpy(np.ascontiguousarray(tables)).to(dev),
                torch.from_numpy(qsl).to(dev), torch.from_numpy(lens).to(dev), qsl, lens)

    hit = batch(hit_tables, own)
    whole = batch(whole_tables, total)
    stream = torch.cuda.current_stream()

    def run(b, chunk):
        lib.pa_prefill_chunk(b[1], b[0], kc, vc, b[2], b[3], b[4], scale, chunk, stream=stream)

    for _ in range(args.warmup):
        run(hit, own)
        run(whole, total)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} prefills with and without prefix hits")
    ms = timer.per_launch([("with_hits", lambda: run(hit, own)),
                           ("whole", lambda: run(whole, total))], args.steps, stream)
    flops_hit = accounting.prefill_flops(hit[5], hit[6], hq, d)
    flops_whole = accounting.prefill_flops(whole[5], whole[6], hq, d)
    tf = flops_hit / (ms["with_hits"] * 1e-3) / 1e12
    result = {
        "metric": PREFIX_METRIC, "value": round(ms["with_hits"] * 1e3, 2), "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms["with_hits"], 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "32 prompts sharing a 2048-token system prompt + 256 own tokens, "
                               "40 query and 40 kv heads, head_dim 128, bf16, block size 16",
                   "cached_tokens_per_prompt": sys_len, "seed": 453},
        "whole_prompt_prefill_us": round(ms["whole"] * 1e3, 2),
        "prefill_speedup": round(ms["whole"] / ms["with_hits"], 2),
        "prefill_tokens_per_step": {"with_hits": n * own, "whole": n * total},
        "kv_blocks": {"with_hits": int(len(set(hit_tables[hit_tables >= 0].tolist()))),
                      "whole": n * mb},
        "block_manager_host_us": round(host_us, 1),
        "block_manager_note": "add_prompt + append_tokens of 32 prompts of 2304 tokens (hashing, "
                              "lookup, slots) and the batch's take_moves, through the C ABI",
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "prefill_x32_kernel<128,4>",
                     "algorithmic_flops_per_launch": int(flops_hit),
                     "whole_prompt_flops": int(flops_whole)},
        "cpu_baseline": None if args.no_cpu_baseline else prefix_cpu_baseline(d, hq, own, total),
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_prefill_long(args, torch, dev, lib, timer) -> int:
    """Chunks over long paged prefixes: few query tiles with long causal key
    ranges, where one workgroup per query tile leaves most of the part idle;
    pa_prefill_chunk_split against pa_prefill_chunk."""
    import numpy as np

    from workloads import accounting, make_prefill
    from workloads.device import to_device

    nseq, prefix, chunk, h, d = 4, 16384, 128, 40, 128
    # runs of 5504 keys: 3 even runs per query tile (86 tiles each), 480
    # workgroups, one round of the part's 512 workgroup slots; with the K/V
    # streamed past the caches this beats 6 runs of 3072 (235 vs 278 us) and
    # the other sizes of 1536-5632
    split = args.prefill_split or 5504
    w = make_prefill("prefill-long", 453, "bf16", [prefix] * nseq, [chunk] * nseq, h, h, d,
                     nseq * ((prefix + chunk) // 16 + 1))
    dw = to_device(w, device=dev)
    g = dw.prefill
    maxc = prefix + chunk
    ws = torch.empty(lib.pa_prefill_workspace_bytes(nseq * chunk, h, d, maxc, split),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def split_run():
        lib.pa_prefill_chunk_split(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                                   g.query_start_loc, g.context_lens, w.scale, g.max_query_len,
                                   maxc, split, ws, stream=stream)

    def plain_run():
        lib.pa_prefill_chunk(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                             g.query_start_loc, g.context_lens, w.scale, g.max_query_len,
                             stream=stream)

    for _ in range(args.warmup):
        split_run()
        plain_run()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} long-prefix prefills, split and whole")
    ms = timer.per_launch([("split", split_run), ("unsplit", plain_run)], args.steps, stream)
    flops = accounting.prefill_flops(w.prefill.query_start_loc, w.prefill.context_lens, h, d)
    tf = flops / (ms["split"] * 1e-3) / 1e12
    tf_plain = flops / (ms["unsplit"] * 1e-3) / 1e12
    # each (sequence, kv head) has one 128-row query tile: its K and V rows are
    # read once, 4·D·128 flops per 2·2·D bytes = 128 flop/B, below the 312
    # flop/B where the bf16 matrix-core and HBM peaks meet, so the K/V stream
    # bounds the launch
    kv_bytes = nseq * (prefix + chunk) * h * d * 2 * 2
    gbs = kv_bytes / (ms["split"] * 1e-3) / 1e9
    gbs_plain = kv_bytes / (ms["unsplit"] * 1e-3) / 1e9
    result = {
        "metric": LONG_PREFILL_METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms["split"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{nseq} chunks of {chunk} query tokens over {prefix}-token paged "
                               f"prefixes, 40 query and 40 kv heads, head_dim 128, bf16, block size 16",
                   "split_tokens": split, "seed": 453},
        "prefill_us": {"split": round(ms["split"] * 1e3, 2),
                       "unsplit": round(ms["unsplit"] * 1e3, 2)},
        "speedup_over_unsplit": round(ms["unsplit"] / ms["split"], 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("prefill_long") if split == 5504 else None,
                     "kernel": f"prefill_x32_kernel<128,4> in runs of {split} keys + "
                               "prefill_merge_kernel (one pa_prefill_chunk_split call)",
                     "algorithmic_bytes_per_launch": int(kv_bytes),
                     "note": "one 128-row query tile per (sequence, kv head): 128 flop per K/V "
                             "byte, under the 312 flop/B ridge of the bf16 matrix cores and HBM",
                     "mfma_achieved_tflops": round(tf, 2),
                     "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_launch": int(flops),
                     "unsplit_achieved": round(gbs_plain, 2),
                     "unsplit_frac": round(gbs_plain / HBM_PEAK_GBS, 4),
                     "unsplit_mfma_frac": round(tf_plain / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        cpu = prefix_cpu_baseline(d, h, chunk, prefix + chunk, n=nseq)
        cpu.update(value=round(flops / (cpu["value"] * 1e-6) / 1e12, 6), unit="TFLOP/s")
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


def prefix_cpu_baseline(d: int, hq: int, own: int, total: int, n: int = 32):
    """The fp64 prefill oracle on one prompt's chunk (own query tokens over a
    total-token context), BLAS on every core the process may use, scaled to the
    32-prompt batch."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads.generate import f32_to_bf16_bits

    rng = np.random.default_rng(454)
    nblk = total // 16
    k = f32_to_bf16_bits(rng.standard_normal((nblk, hq, 16, d)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((nblk, hq, 16, d)).astype(np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((own, hq, d)).astype(np.float32))
    host = host_description()
    with threadpool_limits(host["threads"]):
        t0 = time.perf_counter()
        oracle.prefill(q, k, v, np.arange(nblk)[None, :], np.array([0, own], dtype=np.int32),
                       np.array([total], dtype=np.int32), np.float32(1 / np.sqrt(d)), "bf16")
        t = time.perf_counter() - t0
    return {"value": round(t * n * 1e6, 1), "unit": "us", "cores": host["threads"],
            "kind": "oracle", "cpu_model": host["cpu_model"], "blas": host["blas"],
            "sample": f"fp64 numpy prefill oracle, BLAS on {host['threads']} thread(s): one "
                      f"prompt's {own}-token chunk over {total} tokens of context, {hq} heads "
                      f"({t:.2f} s), times {n} prompts"}


def bench_sampler(args, torch, dev, lib, timer) -> int:
    """pa_sample over 256 rows of 32000 fp32 logits."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from workloads import sampler_inputs

    s, v = 256, 32000
    logits, t, k, p, u = sampler_inputs(s, v, 453)
    f = lambda a: torch.from_numpy(np.asarray(a)).to(dev)
    # Launches cycle through SAMPLER_BUFFERS distinct logits batches (295 MB in
    # all, more than the GPU's 256 MB last-level cache), so that every launch
    # reads its logits from HBM.
    host = [logits] + [sampler_inputs(s, v, 453 + i)[0] for i in range(1, SAMPLER_BUFFERS)]
    lgs = [f(x) for x in host]
    tt, kk, pp, uu = f(t), f(k), f(p), f(u)
    tok = torch.empty(s, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    turn = [0]

    def run():
        lib.pa_sample(tok, lgs[turn[0] % SAMPLER_BUFFERS], tt, kk, pp, uu, stream=stream)
        turn[0] += 1

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} sampler launches")
    ms = timer.per_launch([("sample", run)], args.steps, stream)["sample"]
    algo = s * v * 4 + s * 20                        # logits, per-row parameters and the token
    gbs = algo / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle.sampler as osamp
        host = host_description()
        with threadpool_limits(host["threads"]):
            t0 = time.perf_counter()
            rows = 0
            while rows < 4 * s * SAMPLER_BUFFERS and time.perf_counter() - t0 < 10.0:
                b, r = (rows // s) % SAMPLER_BUFFERS, rows % s
                osamp.sample(host[b][r], float(t[r]), int(k[r]), float(p[r]), float(u[r]))
                rows += 1
            el = time.perf_counter() - t0
        cpu = {"value": round(rows / el, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
               "cpu_model": host["cpu_model"], "blas": host["blas"],
               "sample": f"reference sampler (numpy float64, sorts the row) on {rows} rows "
                         f"taken in turn from the {SAMPLER_BUFFERS} logits batches, {el:.2f} s; "
                         f"it runs row by row in one thread (BLAS allowed {host['threads']})"}
    result = {
        "metric": SAMPLER_METRIC, "value": round(s / (ms * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "256 rows x 32000 fp32 logits, N(0, 1.5) plus 8 strong "
                               "candidates per row; (temperature, top_k, top_p) cycling through "
                               "the pages' (0.7, 50, 0.9) and 7 other settings", "seed": 453,
                   "logits_batches": SAMPLER_BUFFERS},
        "us_per_launch": round(ms * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "sample_kernel<float, 32>", "algorithmic_bytes_per_launch": int(algo)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=WORKLOADS, default="llama13b")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-K partition length in tokens (default: 512 for gqa as its "
                         "configuration states, 2048 for the others)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="default workload only: skip the Llama-2-7B, GQA and mixed "
                         "sub-results the default line carries")
    ap.add_argument("--prefill-split", type=int, default=None,
                    help="keys per run of the split prefill (pa_prefill_chunk_split): "
                         "mixed_gqa defaults to 2048, the other mixed workloads to 0 = "
                         "pa_prefill_chunk, one workgroup per query tile; prefill_long "
                         "defaults to 5504")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode call and its merge (for counter runs); prints "
                         "a short JSON line")
    ap.add_argument("--no-prefix-groups", action="store_true",
                    help="mixed workloads: decode with pa_decode (each sample streams the "
                         "shared prefix itself) instead of pa_decode_shared_prefix")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--digest-counters", nargs=5, metavar=("KIND", "CSV", "CSV", "CSV", "CSV"),
                    help="write the committed HBM-traffic summary of KIND (decode or copy) "
                         "from four rocprofv3 counter_collection.csv files: the kernel's "
                         "FETCH_SIZE and WRITE_SIZE runs, then the plain copy's FETCH_SIZE "
                         "and WRITE_SIZE runs (no GPU needed)")
    args = ap.parse_args(argv)
    if args.digest_counters:
        return digest_counters(*args.digest_counters)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-attention step runs on a single "
              "device; run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_453_amd import lib
    from workloads import accounting
    from workloads.device import to_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        return copy_calibration(torch, dev)
    lib.load()
    ps = args.partition_size
    if args.workload == "block_moves":
        return bench_block_moves(args, torch, dev, lib, StepTimer(torch))
    if args.workload == "prefix_cache":
        return bench_prefix_cache(args, torch, dev, lib, StepTimer(torch))
    if args.workload == "prefill_long":
        return bench_prefill_long(args, torch, dev, lib, StepTimer(torch))
    if args.workload == "sampler":
        return bench_sampler(args, torch, dev, lib, StepTimer(torch))
    if args.workload == "stream_read":
        return bench_stream_read(args, torch, dev, lib, StepTimer(torch))
    result = bench_attention(args, torch, dev, lib, args.workload)
    if result is None:
        return 0
    if args.workload == "llama13b" and not args.no_other_configs:
        # the other decode configurations of the hot path, each in its own
        # allocation after the headline one is freed, timed the same way
        torch.cuda.empty_cache()
        result["other_configs"] = other_configs(args, torch, dev, lib)
    print(json.dumps(result), flush=True)
    return 0


def bench_attention(args, torch, dev, lib, name: str, partition_size=None, steps=None,
                    with_cpu: bool = True):
    """One attention workload (decode, scatter, prefill as the workload has them):
    returns the result dict of its JSON line (None for --decode-only, which
    prints its own short line)."""
    import numpy as np

    from workloads import accounting
    from workloads.device import to_device

    ps = args.partition_size if partition_size is None else partition_size
    steps = args.steps if steps is None else steps
    fp8 = name.endswith("_fp8")
    base = name[:-len("_fp8")] if fp8 else name
    if ps is None:
        ps = 512 if base == "gqa" else 2048

    log(f"bench: generating the {name} workload")
    t0 = time.time()
    w, cfg = build_workload(base, ps)
    g = w.decode
    codes = None
    if fp8:
        from workloads import fp8_pools
        from workloads.device import upload_fp8_pools
        codes = fp8_pools(w, 453)
        cfg["workload"] = cfg["workload"].replace("paged decode", "paged decode over an FP8 "
                                                  "(E4M3) cache")
        if base.startswith("mixed"):
            cfg["workload"] = cfg["workload"].replace("chunked prefill", "FP8 chunked prefill")
        cfg["kv_cache"] = (f"fp8 e4m3 codes, random sign / exponent field 0..9 / mantissa; "
                           f"k_scale {FP8_K_SCALE}, v_scale {FP8_V_SCALE}")
    log(f"bench: generated in {time.time() - t0:.1f} s; uploading")
    dw = to_device(w, device=dev, pools=not fp8)
    if fp8:
        dw.k_cache, dw.v_cache = upload_fp8_pools(w, codes[0], codes[1], device=dev)
    dg = dw.decode
    ws_bytes = lib.pa_decode_workspace_bytes(g.num_seqs, w.num_heads, w.head_dim,
                                             g.max_context_len, ps)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    timer = StepTimer(torch)

    def scatter():
        if fp8:
            lib.pa_reshape_and_cache_fp8(dw.new_k, dw.new_v, dw.k_cache, dw.v_cache,
                                         dw.slot_mapping, FP8_K_SCALE, FP8_V_SCALE, stream=stream)
        else:
            lib.pa_reshape_and_cache(dw.new_k, dw.new_v, dw.k_cache, dw.v_cache,
                                     dw.slot_mapping, stream=stream)

    # samples of one prompt: their common partitions are streamed once per group
    grouped = dg.prefix_group is not None and ps > 0 and not args.no_prefix_groups
    max_group = int(np.bincount(g.prefix_group).max()) if g.prefix_group is not None else 1

    def plain_decode(s=stream):
        if fp8:
            lib.pa_decode_fp8(dg.out, dg.query, dw.k_cache, dw.v_cache, dg.block_tables,
                              dg.context_lens, w.scale, FP8_K_SCALE, FP8_V_SCALE,
                              g.max_context_len, ps, ws if ps else None, stream=s,
                              shared_prefix_blocks=dg.shared_prefix_blocks)
        else:
            lib.pa_decode(dg.out, dg.query, dw.k_cache, dw.v_cache, dg.block_tables,
                          dg.context_lens, w.scale, g.max_context_len, ps, ws if ps else None,
                          stream=s, shared_prefix_blocks=dg.shared_prefix_blocks)

    def grouped_decode(s=stream):
        if fp8:
            lib.pa_decode_fp8_shared_prefix(
                dg.out, dg.query, dw.k_cache, dw.v_cache, dg.block_tables, dg.context_lens,
                w.scale, FP8_K_SCALE, FP8_V_SCALE, g.max_context_len, ps, ws,
                dg.shared_prefix_blocks, dg.prefix_group, max_group, stream=s)
        else:
            lib.pa_decode_shared_prefix(
                dg.out, dg.query, dw.k_cache, dw.v_cache, dg.block_tables, dg.context_lens,
                w.scale, g.max_context_len, ps, ws, dg.shared_prefix_blocks, dg.prefix_group,
                max_group, stream=s)

    decode = grouped_decode if grouped else plain_decode

    def reduce(s=stream):
        if ps:
            lib.pa_decode_splitk_reduce(dg.out, ws, dg.context_lens, g.max_context_len, ps,
                                        stream=s)

    # long causal key ranges of the prefill chunks split over workgroups
    pf_split = 0
    if w.prefill is not None:
        # grouped-query heads: the split pays (2048-key runs); 40 heads: one run per tile
        default_split = 2048 if base == "mixed_gqa" and not fp8 else 0
        pf_split = default_split if args.prefill_split is None else args.prefill_split
    pf_maxc = int(w.prefill.context_lens.max()) if w.prefill is not None else 0
    pws = None
    if pf_split:
        pq = dw.prefill.query
        pws = torch.empty(max(lib.pa_prefill_workspace_bytes(pq.shape[0], pq.shape[1], pq.shape[2],
                                                             pf_maxc, pf_split), 16),
                          dtype=torch.uint8, device=dev)

    def split_prefill(s=stream):
        p = dw.prefill
        if fp8:
            lib.pa_prefill_chunk_fp8_split(p.out, p.query, dw.k_cache, dw.v_cache, p.block_tables,
                                           p.query_start_loc, p.context_lens, w.scale,
                                           FP8_K_SCALE, FP8_V_SCALE, p.max_query_len, pf_maxc,
                                           pf_split, pws, stream=s)
        else:
            lib.pa_prefill_chunk_split(p.out, p.query, dw.k_cache, dw.v_cache, p.block_tables,
                                       p.query_start_loc, p.context_lens, w.scale,
                                       p.max_query_len, pf_maxc, pf_split, pws, stream=s)

    def plain_prefill(s=stream):
        p = dw.prefill
        if fp8:
            lib.pa_prefill_chunk_fp8(p.out, p.query, dw.k_cache, dw.v_cache, p.block_tables,
                                     p.query_start_loc, p.context_lens, w.scale, FP8_K_SCALE,
                                     FP8_V_SCALE, p.max_query_len, stream=s)
        else:
            lib.pa_prefill_chunk(p.out, p.query, dw.k_cache, dw.v_cache, p.block_tables,
                                 p.query_start_loc, p.context_lens, w.scale, p.max_query_len,
                                 stream=s)

    prefill = split_prefill if pf_split else plain_prefill
    launches = []
    if w.slot_mapping is not None:
        launches.append(("reshape_and_cache", scatter))
    if w.prefill is not None:
        launches.append(("prefill", prefill))
    launches.append(("decode", decode))
    if ps:
        launches.append(("splitk_reduce", reduce))

    if args.decode_only:
        launches = [(n, f) for n, f in launches if n in ("decode", "splitk_reduce")]

    def step():
        for _, fn in launches:
            fn()

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {steps} steps")
    ms_per_step = timer.per_step(step, steps, [stream])
    kernel_ms = timer.per_launch(launches, steps, stream)
    log("bench: step %.1f us (%s)" % (ms_per_step * 1e3, ", ".join(
        f"{k} {v * 1e3:.1f}" for k, v in kernel_ms.items())))

    if args.decode_only:
        kv = accounting.decode_kv_bytes(g.context_lens, w.num_kv_heads, w.head_dim,
                                        1 if fp8 else w.elem_bytes)
        unique = accounting.unique_kv_bytes(g.block_tables, g.context_lens, w.num_kv_heads,
                                            w.head_dim, 1 if fp8 else w.elem_bytes)
        print(json.dumps({
            "mode": "decode_only", "workload": name, "partition_size": ps,
            "entry_point": ("pa_decode_shared_prefix" if grouped else "pa_decode"),
            "decode_us": round(kernel_ms["decode"] * 1e3, 2),
            "kv_bytes_logical": int(kv), "kv_bytes_unique": int(unique)}), flush=True)
        return None

    if pf_split:
        # the same prefill without splitting, for comparison
        pf_ms = timer.per_launch([("prefill_unsplit", plain_prefill)], steps, stream)
        log("bench: prefill without splitting %.1f us" % (pf_ms["prefill_unsplit"] * 1e3))

    if grouped:
        # the same decode without the grouped pass, for comparison
        extra_ms = timer.per_launch([("decode_ungrouped", plain_decode)], steps, stream)
        log("bench: decode without prefix groups %.1f us" % (extra_ms["decode_ungrouped"] * 1e3))

    kv_elem = 1 if fp8 else w.elem_bytes
    kv = accounting.decode_kv_bytes(g.context_lens, w.num_kv_heads, w.head_dim, kv_elem)
    gbs = kv / (ms_per_step * 1e-3) / 1e9
    decode_gbs = kv / (kernel_ms["decode"] * 1e-3) / 1e9
    tokens = g.num_seqs
    extra = {}
    group = w.num_heads // w.num_kv_heads
    kv_name = "fp8" if fp8 else "bf16"
    dec_kernel = (f"decode_gqa_mfma_kernel<{kv_name}>" if group >= 4 else
                  f"decode_valu_kernel<bf16,{kv_name},{w.head_dim},{group}>")
    if group <= 4 and ps > 0 and base in ("llama13b", "llama7b"):
        # a plain split-K decode: the schedule launch, then the dealt kernel
        dec_kernel = (f"decode_valu_dealt_kernel<bf16,{kv_name},{w.head_dim},{group}> "
                      "(after decode_schedule_kernel, one pa_decode call)")
    if grouped and group >= 4:
        dec_kernel = (f"decode_gqa_mfma_kernel<{kv_name},grouped> + "
                      f"decode_gqa_mfma_kernel<{kv_name}> (one pa_decode_shared_prefix call)")
    elif grouped:
        dec_kernel = (f"decode_valu_kernel<bf16,{kv_name},{w.head_dim},3,grouped> + "
                      f"decode_valu_kernel<bf16,{kv_name},{w.head_dim},{group}> "
                      "(one pa_decode_shared_prefix call)")
    roofline = {"bound": "hbm", "achieved": round(decode_gbs, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(decode_gbs / HBM_PEAK_GBS, 4),
                "traffic": {"llama13b": measured_traffic("decode"),
                            "llama7b": measured_traffic("decode_7b"),
                            "gqa": measured_traffic("decode_gqa")}.get(name),
                "kernel": dec_kernel, "algorithmic_bytes_per_launch": int(kv)}

    if w.prefill is not None:
        p = w.prefill
        flops = accounting.prefill_flops(p.query_start_loc, p.context_lens, w.num_heads,
                                         w.head_dim)
        unique = accounting.unique_kv_bytes(g.block_tables, g.context_lens, w.num_kv_heads,
                                            w.head_dim, kv_elem)
        tokens += int(p.query_start_loc[-1])
        pf_tflops = flops / (kernel_ms["prefill"] * 1e-3) / 1e12
        unique_gbs = unique / (kernel_ms["decode"] * 1e-3) / 1e9
        # the decode of shared prefixes must read each physical row once at least
        if name == "mixed":
            roofline["traffic"] = measured_traffic("mixed_decode" if grouped
                                                   else "mixed_decode_plain")
        roofline.update({"achieved": round(unique_gbs, 2),
                         "frac": round(unique_gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": int(unique),
                         "logical_bytes_per_launch": int(kv),
                         "logical_gbs": round(decode_gbs, 2),
                         "note": "achieved = unique (physical) KV bytes / decode time; "
                                 "logical bytes count shared prefix rows once per sequence"})
        extra["roofline_prefill"] = {
            "bound": "mfma", "achieved": round(pf_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None, "kernel": ("prefill_mfma_kernel<fp8,128,32,4>" if fp8 else
                                        "prefill_x32_kernel<128,4>") + (
                f" in runs of {pf_split} keys + prefill_merge_kernel (one "
                "pa_prefill_chunk_split call)" if pf_split else ""),
            "algorithmic_flops_per_launch": int(flops)}
        if pf_split:
            extra["roofline_prefill"]["prefill_us_without_splitting"] = round(
                pf_ms["prefill_unsplit"] * 1e3, 2)
        extra["prefill_tokens_per_step"] = int(p.query_start_loc[-1])
        # a rate against the HBM peak must count each physical row once
        extra["kv_gbs_logical"] = round(gbs, 2)
        extra["kv_bytes_unique_per_step"] = int(unique)
        gbs = unique / (ms_per_step * 1e-3) / 1e9
        extra["prefixes"] = w.meta.get("prefixes")
        extra["decode_prefix_groups"] = {
            "entry_point": "pa_decode_shared_prefix" if grouped else "pa_decode",
            "groups": int(np.unique(g.prefix_group).size) if g.prefix_group is not None else 0,
            "max_group_size": max_group}
        if grouped:
            extra["decode_prefix_groups"]["decode_us_without_grouping"] = round(
                extra_ms["decode_ungrouped"] * 1e3, 2)

        # the same step with prefill (matrix cores) and decode (HBM) on two streams
        side = torch.cuda.Stream(device=dev)

        def step_overlap():
            fork = torch.cuda.Event()
            fork.record(stream)
            side.wait_event(fork)
            prefill(side)
            decode(stream)
            join = torch.cuda.Event()
            join.record(side)
            stream.wait_event(join)
            reduce(stream)

        for _ in range(args.warmup):
            step_overlap()
        ms_overlap = timer.per_step(step_overlap, steps, [stream, side])
        extra["overlapped_two_streams"] = {
            "ms_per_step": round(ms_overlap, 5),
            "kv_gbs_logical": round(kv / (ms_overlap * 1e-3) / 1e9, 2),
            "tokens_per_s": round(tokens / (ms_overlap * 1e-3), 1)}
        log(f"bench: overlapped step {ms_overlap * 1e3:.1f} us")

    cpu = None
    if with_cpu and not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        cpu = cpu_baseline_report(w, fp8_pools=codes)

    config = {"workload": cfg.pop("workload"), "num_seqs": g.num_seqs,
              "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
              "head_dim": w.head_dim, "block_size": 16,
              "total_context_tokens": int(g.context_lens.sum()),
              "num_blocks": w.num_blocks, "partition_size": ps}
    config.update(cfg)
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_p10_p50_p90": timer.spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 kv / bf16 q" if fp8 else "bf16",
        "data": "synthetic",
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "tokens_per_s_note": "one decode token per sequence (plus the prefill chunk tokens "
                             "where present) per step, one attention layer",
        "kv_bytes_per_step": int(kv),
        "value_note": "KV bytes of the step / step time" + (
            "; FP8 cache: one byte per K/V element" if fp8 else "") + (
            "; unique (physical) bytes: shared prefix rows count once"
            if w.prefill is not None else ""),
        "kernel_us": {k: round(v * 1e3, 2) for k, v in kernel_ms.items()},
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    result.update(extra)
    if name == "llama13b":
        # the part's achievable read rate, beside the 8 TB/s peak the roofline uses
        read = stream_read_gbs(torch, dev, lib, timer)
        result["achievable_read_gbs"] = round(read, 2)
        result["decode_pct_of_achievable_read"] = round(100.0 * decode_gbs / read, 2)
    return result



if __name__ == "__main__":
    sys.exit(main())
