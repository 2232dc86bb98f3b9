#!/usr/bin/env python3
"""Paged attention throughput on one MI355X, against the HBM and MFMA rooflines.

Default workload (seeded, synthetic): one decode iteration of one LLaMA-7B
attention layer -- 64 sequences x 32 heads x head_dim 128, f16, block_size
16, context lengths ~ U[128, 2048], block tables = slices of one random
permutation of a pool sized to fit exactly, q/K/V ~ N(0,1).

Other workloads (``--workload``), same machinery:
  mixed256    256 sequences x 32 x 128, bf16, block_size 32, lognormal
              context lengths (mean ~600, clipped to [1, 4096]), 1.25x pool
  prefix13b   32 prompts x 8 samples, 40 x 128, f16, block_size 16, a
              1024-token prompt whose blocks all 8 samples share, tails U[0,256];
              decoded by the shared-prefix call (each shared tile read once
              per prompt; --plain: the ordinary decode), so its algorithmic
              bytes count each aliased K/V byte once
  mixed_step  40 x 128, f16, block_size 16: cache write of 2048 rows, causal
              prefill of 4 chunks (L ~ U[256,512] after U[0,1024] cached
              tokens) and decode of 96 sequences (ctx ~ U[256,4096])
  prefill_long  40 x 128, f16, block_size 16: cache write of the chunks'
              4096 rows, then causal prefill of 8 chunks of 512 queries after
              1536 cached tokens (150 GFLOP): the compute-bound path, reported
              in TFLOP/s against the dense MFMA peak
  prefill_f32 the mixed step's cache write and its 4 prefill chunks with f32
              caches and queries: the f32 prefill kernel, in TFLOP/s against
              the dense fp32 MFMA peak

One step = the workload's whole path, all inputs resident in HBM:
reshape_and_cache of the step's new tokens, [prefill,] then split-K decode
(partition kernel + reduction kernel) with an output in the input dtype.
The pure decode steps (llama7b, mixed256: one new token per sequence) write
their new tokens from inside the partition kernel
(paged_attention_decode_with_cache_write, bit-identical to the separate
write); --separate-cache-write launches reshape_and_cache first instead.
The timed steps replay the step captured as a HIP graph (checked
bit-identical to the eager step); --eager times plain launches instead. The
mixed step is timed as one pa_attention_step call with the prefill on a
side stream next to the decode (the in-order graph is timed too).

Prints ONE JSON line: value = algorithmic bytes of the step / step time
(GB/s, 1e9 B/s); roofline = the decode partition kernel's algorithmic bytes
over its average launch time against the 8 TB/s HBM peak, timed with HIP
events on the launch stream in a cold-cache pass (a 1 GiB read before every
step evicts L2 and the memory-side cache; the warm back-to-back average is
reported next to it); cpu_baseline = the fp64 oracle on the host cores over
the same work, and on one thread over a sample of it.
"""
import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention achieved HBM GB/s (% of peak) at LLaMA-7B layer shape"
METRIC_OTHER = "paged attention step achieved HBM GB/s (% of peak)"
HBM_PEAK_GBPS = 8000.0
# dense matrix-core peaks of MI355X (fp32 equals the fp32 vector rate)
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
PREFILL_WORKLOADS = ("prefill_long", "prefill_f32")
KERNEL_SOURCES = ["pa_decode.hip", "pa_decode_device.h", "pa_device.h", "pa_bounds.h", "pa_internal.h"]
SHARED_KERNEL_SOURCES = KERNEL_SOURCES + ["pa_shared.hip"]
PREFILL_KERNEL_SOURCES = ["pa_prefill.hip", "pa_grid.h", "pa_device.h", "pa_bounds.h", "pa_internal.h"]
LEAD_CYCLES = 4_000_000  # GPU spin before each cold step (gpu_lead), ~2 ms
WARM_LEAD_CYCLES_PER_STEP = 1_000_000  # spin before the back-to-back eager pass, per step queued behind it
CPU_SECONDS = 10.0  # the oracle repeats its pass until about this much CPU time has elapsed

WORKLOADS = {
    "llama7b": "llama7b_decode_step: cache write of 64 new tokens + split-K paged decode, 64 seqs x 32 heads "
               "x 128, f16, block_size 16, ctx U[128,2048], seed 393",
    "mixed256": "mixed256_decode_step: cache write of 256 new tokens + split-K paged decode, 256 seqs x 32 "
                "heads x 128, bf16, block_size 32, ctx lognormal(mean 600) clipped to [1,4096], 1.25x pool, seed 394",
    "prefix13b": "prefix13b_decode_step: 32 prompts x 8 samples sharing a 1024-token prompt's blocks, tails "
                 "U[0,256], 40 heads x 128, f16, block_size 16, seed 395",
    "mixed_step": "mixed_step: reshape_and_cache of 2048 rows + causal prefill of 4 chunks (L U[256,512], prior "
                  "U[0,1024]) + split-K decode of 96 seqs (ctx U[256,4096]), 40 heads x 128, f16, block_size 16, "
                  "seed 396",
    "prefill_long": "prefill_long: reshape_and_cache of the chunks' 4096 rows + causal prefill of 8 chunks of 512 "
                    "queries after 1536 cached tokens, 40 heads x 128, f16, block_size 16, seed 397",
    "prefill_f32": "prefill_f32: reshape_and_cache of the mixed step's 2048 rows + causal prefill of its 4 chunks "
                   "(L U[256,512], prior U[0,1024]), 40 heads x 128, f32, block_size 16, seed 396",
}
PREFILL_METRIC = "causal paged prefill achieved TFLOP/s (% of the dense MFMA peak)"
PREFILL_F32_METRIC = "causal paged prefill achieved TFLOP/s (% of the dense fp32 MFMA peak)"


def traffic_file(workload, shared=False, separate_write=False):
    if workload in PREFILL_WORKLOADS:
        return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    tag = workload + ("_shared" if shared else "_plain" if workload == "prefix13b" else "")
    tag += "_separate_write" if separate_write else ""
    return os.path.join(ROOT, "profiles", f"decode_{tag}_traffic.json")


def traffic_kernel(shared, workload=None):
    """The kernel whose HBM traffic is recorded: the partition kernel, the
    shared-prefix step kernel for the shared-prefix call, or the prefill
    kernel for the compute-bound workload."""
    if workload == "prefill_long":
        return "prefill_mfma_kernel"
    if workload == "prefill_f32":
        return "prefill_f32_kernel"
    return "shared_prefix_step_kernel" if shared else "decode_partition_kernel"


def kernel_source_hash(shared=False, workload=None):
    h = hashlib.sha256()
    names = PREFILL_KERNEL_SOURCES if workload in PREFILL_WORKLOADS else (
        SHARED_KERNEL_SOURCES if shared else KERNEL_SOURCES)
    for name in names:
        with open(os.path.join(ROOT, "paged_kv_cache_391_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gpu_lead(cycles=None):
    """Queue a GPU spin (LEAD_CYCLES, ~1 ms, by default) ahead of timed
    launches: the host queues them while the GPU is still busy, so no event
    pair around a kernel can include GPU idle time spent waiting for the
    host."""
    import torch
    if hasattr(torch.cuda, "_sleep"):  # a private helper of torch: without it, no lead
        torch.cuda._sleep(LEAD_CYCLES if cycles is None else cycles)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _counter_rows(path):
    """(kernel name, counter value) per dispatch from a rocprofv3 counter
    collection CSV (one counter per run)."""
    import csv
    import glob
    files = [path] if path.endswith(".csv") else glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                                              recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def record_traffic(workload, shared, fetch_dir, write_dir, copy_bytes, separate_write=False):
    """Turn two counter runs of this benchmark (FETCH_SIZE, then WRITE_SIZE;
    both in KiB per dispatch) into HBM bytes per launch of the dominant
    kernel, each scaled by what the same counter reads for the plain device
    copy of known size in the same run, and store them with the hash of the
    kernel source they describe."""
    kname = traffic_kernel(shared, workload)
    out = {}
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _counter_rows(d)
        part = [v for k, v in rows if kname in k]
        copy = [v for k, v in rows if "copyBuffer" in k or "copy" in k.lower()]
        copy = max(copy)  # the probe copy is the largest copy dispatch
        scale = (copy_bytes / 1024.0) / copy
        out[name] = {"partition_kernel_kib_avg": sum(part) / len(part), "copy_kib": copy, "scale": scale,
                     "dispatches": len(part)}
    fetch = out["fetch"]["partition_kernel_kib_avg"] * 1024 * out["fetch"]["scale"]
    write = out["write"]["partition_kernel_kib_avg"] * 1024 * out["write"]["scale"]
    flags = f"--workload {workload}" + (" --plain" if workload == "prefix13b" and not shared else "") + (
        " --separate-cache-write" if separate_write else "")
    rec = {"kernel": kname, "workload": f"{workload} (bench.py {flags})",
           "kernel_source_sha256": kernel_source_hash(shared, workload), "hbm_bytes_per_launch": round(fetch + write),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write), "counters": out}
    import paged_kv_cache_391_amd as pa
    rec["partition_tokens"] = pa.decode_partition_tokens()
    with open(traffic_file(workload, shared, separate_write), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def decode_bytes(ctx, H, D, elt, bs):
    """Algorithmic bytes of decode over valid tokens: K and V of every valid
    token, one table entry per used block, the context length, q and out."""
    import numpy as np
    ctx = ctx.astype(np.int64)
    S = ctx.shape[0]
    kv = int(ctx.sum()) * H * D * elt * 2
    table = int(np.ceil(ctx / bs).sum()) * 4 + 4 * S
    return kv, table, 2 * S * H * D * elt


def partition_kernel_bytes(ctx, H, D, elt, bs, P):
    """Bytes the partition kernel must move: K/V, table entries and q, plus
    either the final output row or (m, l, acc) per partition."""
    import numpy as np
    ctx = ctx.astype(np.int64)
    kv, table, _ = decode_bytes(ctx, H, D, elt, bs)
    S = ctx.shape[0]
    nparts = np.ceil(np.ceil(ctx / 16) / (P // 16)).astype(np.int64)
    writes = int(np.where(nparts > 1, nparts * H * (D + 2) * 4, H * D * elt).sum())
    return kv + table + S * H * D * elt + writes


def unique_kv_bytes(block_tables, ctx, H, D, elt, bs):
    """K/V bytes of the distinct cache slots the step reads (aliased blocks
    counted once)."""
    import numpy as np
    slots = []
    for s in range(ctx.shape[0]):
        t = np.arange(int(ctx[s]))
        slots.append(block_tables[s, t // bs].astype(np.int64) * bs + t % bs)
    n = np.unique(np.concatenate(slots)).size if slots else 0
    return int(n) * H * D * elt * 2


def prefill_work(p, H, D, elt):
    """(flops, bytes) of causal prefill: unmasked query-key pairs only; each
    chunk reads its context's K/V once and its q, writes its out."""
    import numpy as np
    L = np.diff(p.query_start_loc).astype(np.int64)
    ctx = p.context_lens.astype(np.int64)
    c = ctx - L
    flops = int((4 * D * H * (L * c + L * (L + 1) // 2)).sum())
    byts = int((ctx * H * D * elt * 2 + 2 * L * H * D * elt).sum())
    return flops, byts


def _host_cpu():
    """Model name of the host CPU (first entry of /proc/cpuinfo) and the
    cores this process may run on."""
    name = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return name, avail


def _oracle_rate(wl, kc, vc, rows, threads, seconds, byts):
    """GB/s of the oracle's decode (and, with every row, its prefill) over
    the first `rows` decode sequences, whose algorithmic bytes are `byts`,
    repeated until `seconds` have elapsed."""
    import numpy as np
    import oracle
    d, p = wl.decode, wl.prefill
    whole = rows >= d.num_seqs
    q, bt, ctx = d.q[:rows], d.block_tables[:rows], d.context_lens[:rows]

    def one_pass():
        if whole and p is not None:
            oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, wl.dtype,
                           threads=threads)
        oracle.decode(q, kc, vc, bt, ctx, wl.scale, wl.dtype, threads=threads)

    reps, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    per = el / reps
    return byts / per / 1e9, reps, el, per, int(np.asarray(ctx, dtype=np.int64).sum())


def cpu_baseline(wl, threads, alg_bytes, sample_bytes):
    """The fp64 oracle, as it stands, on the host: all usable cores (up to
    16) over the step's whole decode (and prefill), then one thread over a
    bounded sample (the first eighth of the decode sequences); each repeated
    until about CPU_SECONDS have elapsed. Rates use the same algorithmic-byte
    definition as the GPU step's value: `alg_bytes` for the whole work,
    `sample_bytes(rows)` for the decode of the first `rows` sequences."""
    import oracle
    kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                      wl.block_size, wl.dtype)
    S = wl.decode.num_seqs
    rate, reps, el, per, _ = _oracle_rate(wl, kc, vc, S, threads, CPU_SECONDS, alg_bytes)
    rows1 = max(1, S // 8)
    rate1, reps1, el1, per1, tok1 = _oracle_rate(wl, kc, vc, rows1, 1, CPU_SECONDS, sample_bytes(rows1))
    model, avail = _host_cpu()
    what = "prefill of the 4 chunks + decode" if wl.prefill is not None else "the whole decode"
    return {"value": round(rate, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of this workload, {reps} pass(es) in {el:.1f} s ({per:.3f} s each); fp64, gather + "
                      "softmax attention per (row, head), OpenMP over pairs; same algorithmic-byte definition as "
                      "value",
            "one_thread": {"value": round(rate1, 3), "unit": "GB/s", "cores": 1,
                           "sample": f"decode of the first {rows1} of {S} sequences ({tok1} context tokens), "
                                     f"{reps1} pass(es) in {el1:.1f} s ({per1:.3f} s each)"},
            "host": {"cpu_model": model, "usable_cores": avail}}


def prefill_config(workload="prefill_long"):
    from workloads import config5, prefill_workload
    if workload == "prefill_f32":
        return config5(dtype="f32")
    return prefill_workload("prefill_long", 397, "f16", 40, 128, 16, [1536] * 8, [512] * 8, maxb=128)


def _oracle_prefill_rate(wl, kc, vc, pairs, threads, seconds):
    """TFLOP/s of the oracle's causal prefill over the given (query row,
    head) pairs (4 d flops per visible key), repeated until `seconds`."""
    import numpy as np
    import oracle
    p = wl.prefill
    L = np.diff(p.query_start_loc)
    seq = np.searchsorted(p.query_start_loc, pairs[:, 0], side="right") - 1
    visible = p.context_lens[seq] - L[seq] + (pairs[:, 0] - p.query_start_loc[seq]) + 1
    flops = float(4 * wl.head_dim * visible.astype(np.int64).sum())
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start_loc, wl.scale, wl.dtype,
                       rows=pairs, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return flops * reps / el / 1e12, reps, el


def plain_copy_GBps(gib):
    """Bandwidth of a plain device copy of `gib` GiB (torch), 10 copies after
    3 warm-ups; in a counter run its dispatches calibrate FETCH_SIZE and
    WRITE_SIZE."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    return gbps


def prefill_main(args):
    """The compute-bound path: one step = the chunks' cache write + the
    causal prefill; value = prefill flops per step time (TFLOP/s); roofline =
    the prefill kernel, cold, against the dense f16 MFMA peak."""
    import numpy as np
    import torch

    import oracle
    import paged_kv_cache_391_amd as pa
    from tests._gpu import OnDevice

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t = time.time()
    wl = prefill_config(args.workload)
    p = wl.prefill
    log(f"[bench] {args.workload}: generated in {time.time() - t:.1f}s: {wl.num_blocks} blocks, {p.total_q} queries")
    od = OnDevice(wl)
    H, D, elt = wl.num_heads, wl.head_dim, wl.elt_bytes
    out = torch.empty_like(od.pf_q)  # output in the input dtype
    flops, pf_bytes = prefill_work(p, H, D, elt)
    T = int(wl.new.slot_mapping.shape[0])
    cache_write_bytes = 4 * T * H * D * elt + 4 * T

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pa.reshape_and_cache(od.new_k, od.new_v, od.k_cache, od.v_cache, od.slot_mapping)
        if ev is not None:
            ev[1].record()
        pa.paged_attention_prefill(out, od.pf_q, od.k_cache, od.v_cache, od.pf_block_tables, od.pf_context_lens,
                                   od.pf_qsl, wl.scale, max_q_len=p.max_q_len, max_context_len=p.max_context_len)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    gpu_lead(WARM_LEAD_CYCLES_PER_STEP * args.steps)  # the host queues the whole pass before the GPU starts it
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    eager_ms = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps  # GPU span of the back-to-back steps
    cw_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    pf_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    eager_out = out.clone()

    # cold pass: a 1 GiB read before every step evicts L2 and the MALL
    scratch = torch.zeros((args.evict_mib << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        gpu_lead()
        if args.evict_mode == "read":
            torch.sum(scratch, dim=0, out=sink)
        else:
            scratch.fill_(float(i))
        step(cold[i])
    torch.cuda.synchronize()
    del scratch, sink
    cold_pf = np.array([e[1].elapsed_time(e[2]) for e in cold])
    if not torch.equal(out, eager_out):
        raise SystemExit("cold-cache step output differs from the warm one")

    ms_per_step, graph_ok = eager_ms, None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph_ok = True
        for _ in range(max(1, args.warmup)):
            out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            graph_ok = graph_ok and bool(torch.equal(out, eager_out))
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        if not graph_ok:
            raise SystemExit("graph replay disagrees with the eager step")

    f32 = wl.dtype == "f32"
    peak = MFMA_PEAK_TFLOPS[wl.dtype]
    cold_ms = float(cold_pf.mean())
    pf_tflops = flops / (cold_ms * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step ({'graph' if not args.eager else 'eager'}; eager "
        f"{eager_ms * 1e3:.1f} us): cache write {cw_ms * 1e3:.1f} us, prefill {pf_ms * 1e3:.1f} us warm "
        f"({flops / (pf_ms * 1e-3) / 1e12:.0f} TFLOP/s), {cold_ms * 1e3:.1f} us cold ({pf_tflops:.0f} TFLOP/s), "
        f"graph output == eager: {graph_ok}")

    def pct(x):
        return {"mean": round(float(x.mean()) * 1e3, 2), "median": round(float(np.median(x)) * 1e3, 2),
                "p10": round(float(np.percentile(x, 10)) * 1e3, 2), "p90": round(float(np.percentile(x, 90)) * 1e3, 2)}

    copy_gbps = plain_copy_GBps(args.copy_probe_gib)
    traffic = None
    tf = traffic_file(args.workload)
    if os.path.exists(tf):
        trec = json.load(open(tf))
        if trec.get("kernel_source_sha256") == kernel_source_hash(workload=args.workload):
            traffic = trec.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping,
                                          wl.block_size, wl.dtype)
        threads = max(1, min(16, _host_cpu()[1]))
        last = int(p.query_start_loc[-2])
        many = np.stack(np.meshgrid(np.arange(last, last + 128), np.arange(H), indexing="ij"), -1).reshape(-1, 2)
        few = many[:256]
        rate, reps, el = _oracle_prefill_rate(wl, kc, vc, many.astype(np.int32), threads, CPU_SECONDS)
        rate1, reps1, el1 = _oracle_prefill_rate(wl, kc, vc, few.astype(np.int32), 1, CPU_SECONDS)
        model, avail = _host_cpu()
        cpu = {"value": round(rate, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"fp64 causal prefill of the first 128 queries of the last chunk x {H} heads "
                         f"({many.shape[0]} (query, head) rows), {reps} pass(es) in {el:.1f} s; 4 d flops per "
                         "visible key, the definition of value",
               "one_thread": {"value": round(rate1, 6), "unit": "TFLOP/s", "cores": 1,
                              "sample": f"the first {few.shape[0]} of those rows, {reps1} pass(es) in {el1:.1f} s"},
               "host": {"cpu_model": model, "usable_cores": avail}}

    rec = {
        "metric": PREFILL_F32_METRIC if f32 else PREFILL_METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "global_batch": int(p.num_seqs),
                   "seq_len": int(p.max_context_len), "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(pf_tflops, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(pf_tflops / peak, 4), "traffic": traffic,
                     "kernel": (f"prefill_f32_kernel<{D},{wl.block_size}>" if f32 else
                                f"prefill_mfma_kernel<{wl.dtype},{D},{wl.block_size}>"),
                     "flops_per_launch": flops, "bytes_per_launch": pf_bytes,
                     "avg_launch_us": round(cold_ms * 1e3, 2),
                     "timing": f"HIP events on the launch stream around each of {args.steps} eager launches, "
                               f"each after a GPU spin (the launches queued ahead) and a {args.evict_mib} MiB "
                               f"{args.evict_mode} that evicts L2 and MALL",
                     "launch_us": pct(cold_pf), "warm_avg_launch_us": round(pf_ms * 1e3, 2),
                     "hbm_frac": round(pf_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "roofline_us": round(max(flops / (peak * 1e12), pf_bytes / (HBM_PEAK_GBPS * 1e9)) * 1e6, 2)},
        "timing": "hip_graph_replay" if not args.eager else "eager",
        "eager_ms_per_step": round(eager_ms, 5),
        "hbm_copy_probe_GBps": round(copy_gbps, 1),
        "step_bytes": cache_write_bytes + pf_bytes,
        "phases_us": {"reshape_and_cache": round(cw_ms * 1e3, 2), "prefill": round(pf_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=list(WORKLOADS), default="llama7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--plain", action="store_true", help="prefix13b: ordinary decode instead of the shared-prefix call")
    ap.add_argument("--separate-cache-write", action="store_true",
                    help="llama7b/mixed256: reshape_and_cache as its own launch before the decode")
    ap.add_argument("--block-size", type=int, default=None,
                    help="llama7b: block size (8/16/32/64) for the block-size trade-off; default 16")
    ap.add_argument("--copy-probe-gib", type=float, default=1.0, help="size of the plain-copy bandwidth probe")
    ap.add_argument("--evict-mib", type=int, default=1024,
                    help="MiB read (or written) before every step of the cold-cache pass (evicts L2 and MALL)")
    ap.add_argument("--evict-mode", choices=["read", "write"], default="read",
                    help="how the cold-cache pass evicts: read the scratch buffer (caches left clean) or write it")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="store HBM bytes per launch from two rocprofv3 --pmc runs of this script and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, args.workload == "prefix13b" and not args.plain, args.record_traffic[0],
                       args.record_traffic[1], int(args.copy_probe_gib * (1 << 30)), args.separate_cache_write)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: each GPU would run this path on its own share of sequences or "
            "heads with no collective in the timed region, so only --gpus 1 is measured.")
        sys.exit(2)

    # no garbage-collection pause of the host inside the timed launches
    gc.collect()
    gc.disable()
    if args.workload in PREFILL_WORKLOADS:
        if args.block_size is not None or args.plain:
            raise SystemExit(f"--block-size and --plain do not apply to {args.workload}")
        prefill_main(args)
        return

    import numpy as np
    import torch

    import paged_kv_cache_391_amd as pa
    from tests._gpu import OnDevice
    from workloads import config2, config3, config4, config5

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t = time.time()
    if args.block_size is not None and args.workload != "llama7b":
        raise SystemExit("--block-size applies to the llama7b workload only")
    if args.separate_cache_write and args.workload not in ("llama7b", "mixed256"):
        raise SystemExit("--separate-cache-write applies to the pure decode workloads (llama7b, mixed256)")
    if args.block_size is not None:
        wl = config2(block_size=args.block_size)
    else:
        wl = {"llama7b": config2, "mixed256": config3, "prefix13b": config4, "mixed_step": config5}[args.workload]()
    log(f"[bench] {args.workload}: generated in {time.time() - t:.1f}s: {wl.num_blocks} blocks, "
        f"sum ctx {int(wl.decode.context_lens.sum())}")
    od = OnDevice(wl)
    d, p = wl.decode, wl.prefill
    S, H, D, bs, elt = d.num_seqs, wl.num_heads, wl.head_dim, wl.block_size, wl.elt_bytes
    maxctx = d.max_context_len
    shared = args.workload == "prefix13b" and not args.plain
    if shared:
        # samples of one prompt are consecutive rows sharing the prompt's whole blocks
        nsamp = len(wl.notes["tails"][0])
        gs = torch.arange(0, S + 1, nsamp, dtype=torch.int32, device="cuda")
        pl = torch.tensor([(p // bs) * bs for p in wl.notes["prompt_lens"]], dtype=torch.int32, device="cuda")
        max_prefix = int(pl.max().item())
        ws = pa.make_decode_shared_workspace(S, H, D, maxctx)
    else:
        ws = pa.make_decode_workspace(S, H, D, maxctx)
    out = torch.empty_like(od.q)  # output in the input dtype: the production path
    pf_out = torch.empty_like(od.pf_q) if p is not None else None
    P = pa.decode_partition_tokens()
    # one new token per sequence, at its last position: the partition kernel writes it
    fused = args.workload in ("llama7b", "mixed256") and not args.separate_cache_write
    if fused:
        assert tuple(od.new_k.shape) == tuple(od.q.shape) and int(od.slot_mapping.shape[0]) == S

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if not fused:
            pa.reshape_and_cache(od.new_k, od.new_v, od.k_cache, od.v_cache, od.slot_mapping)
        if ev is not None:
            ev[1].record()
        if p is not None:
            pa.paged_attention_prefill(pf_out, od.pf_q, od.k_cache, od.v_cache, od.pf_block_tables,
                                       od.pf_context_lens, od.pf_qsl, wl.scale, max_q_len=p.max_q_len,
                                       max_context_len=p.max_context_len)
        if ev is not None:
            ev[2].record()
        if shared:
            pa.paged_attention_decode_shared_prefix(out, od.q, od.k_cache, od.v_cache, od.block_tables,
                                                    od.context_lens, gs, pl, wl.scale, maxctx, nsamp, max_prefix, ws)
            if ev is not None:
                ev[3].record()
                ev[4].record()
        elif fused:
            pa.paged_attention_decode_with_cache_write_partitions(out, od.q, od.k_cache, od.v_cache, od.new_k,
                                                                  od.new_v, od.slot_mapping, od.block_tables,
                                                                  od.context_lens, wl.scale, maxctx, ws)
            if ev is not None:
                ev[3].record()
            pa.paged_attention_decode_with_cache_write_reduce(out, od.q, od.k_cache, od.v_cache, od.new_k, od.new_v,
                                                              od.slot_mapping, od.block_tables, od.context_lens,
                                                              wl.scale, maxctx, ws)
            if ev is not None:
                ev[4].record()
        else:
            pa.paged_attention_decode_partitions(out, od.q, od.k_cache, od.v_cache, od.block_tables,
                                                 od.context_lens, wl.scale, maxctx, ws)
            if ev is not None:
                ev[3].record()
            pa.paged_attention_decode_reduce(out, od.context_lens, D, maxctx, od.q.dtype, ws)
            if ev is not None:
                ev[4].record()

    # ---- algorithmic work (valid tokens only)
    kv, table, qo = decode_bytes(d.context_lens, H, D, elt, bs)
    T = int(wl.new.slot_mapping.shape[0])
    t_valid = int((wl.new.slot_mapping >= 0).sum())
    cache_write_bytes = 4 * t_valid * H * D * elt + 4 * T
    k2_bytes = partition_kernel_bytes(d.context_lens, H, D, elt, bs, P)
    if fused:
        # the partition kernel reads the new tokens and their slots; it writes them too only when no
        # reduction follows (a split call leaves the writes to the reduction kernel)
        k2_bytes += cache_write_bytes if ws is None else 2 * t_valid * H * D * elt + 4 * T
    pf_flops, pf_bytes = prefill_work(p, H, D, elt) if p is not None else (0, 0)
    logical_kv = kv
    if args.workload == "prefix13b":
        kv = unique_kv_bytes(d.block_tables, d.context_lens, H, D, elt, bs)  # each aliased byte once
        if shared:
            k2_bytes = kv + table + qo  # the whole shared-prefix call: distinct K/V, table, q and out
        else:
            k2_bytes -= logical_kv - kv  # the plain decode too is held to the distinct bytes
    step_bytes = kv + table + qo + cache_write_bytes + pf_bytes

    # eager pass: HIP events on the launch stream around every kernel launch
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    gpu_lead(WARM_LEAD_CYCLES_PER_STEP * args.steps)  # the host queues the whole pass before the GPU starts it
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    eager_ms = evs[0][0].elapsed_time(evs[-1][-1]) / args.steps  # GPU span of the back-to-back steps

    def phase_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / args.steps

    cw_ms, pf_ms, k2_ms, k3_ms = phase_ms(0, 1), phase_ms(1, 2), phase_ms(2, 3), phase_ms(3, 4)
    eager_out = out.clone()
    eager_pf = pf_out.clone() if pf_out is not None else None

    # cold pass: before every step 1 GiB of scratch is read (or written),
    # outside the events, which evicts L2 and the memory-side cache, so each
    # step reads its K/V from HBM. Reading leaves the caches clean; writing
    # also leaves them full of dirty lines whose write-back the step pays for.
    scratch = torch.zeros((args.evict_mib << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        gpu_lead()
        if args.evict_mode == "read":
            torch.sum(scratch, dim=0, out=sink)  # one reduction kernel that reads the buffer once
        else:
            scratch.fill_(float(i))
        step(cold[i])
    torch.cuda.synchronize()
    del scratch, sink
    cold_k2 = np.array([e[2].elapsed_time(e[3]) for e in cold])
    cold_step = np.array([e[0].elapsed_time(e[4]) for e in cold])
    if not torch.equal(out, eager_out):
        raise SystemExit("cold-cache step output differs from the warm one")

    def pct(x):
        return {"mean": round(float(x.mean()) * 1e3, 2), "median": round(float(np.median(x)) * 1e3, 2),
                "p10": round(float(np.percentile(x, 10)) * 1e3, 2), "p90": round(float(np.percentile(x, 90)) * 1e3, 2)}

    # the mixed step as one scheduler iteration: pa_attention_step with the
    # prefill on a side stream, concurrent with the decode
    step_side = torch.cuda.Stream() if p is not None else None
    step_events = pa.make_step_events() if p is not None else None

    def concurrent_step():
        pa.attention_step(od.k_cache, od.v_cache, wl.scale, od.new_k, od.new_v, od.slot_mapping,
                          prefill_out=pf_out, prefill_q=od.pf_q, prefill_block_tables=od.pf_block_tables,
                          prefill_context_lens=od.pf_context_lens, prefill_query_start_loc=od.pf_qsl,
                          prefill_max_q_len=p.max_q_len, prefill_max_context_len=p.max_context_len,
                          decode_out=out, decode_q=od.q, decode_block_tables=od.block_tables,
                          decode_context_lens=od.context_lens, decode_max_context_len=maxctx, workspace=ws,
                          side_stream=step_side, fork_event=step_events[0], join_event=step_events[1])

    def same():
        ok = bool(torch.equal(out, eager_out))
        return ok and (pf_out is None or bool(torch.equal(pf_out, eager_pf)))

    def time_graph(fn):
        """Capture fn once as a HIP graph; check replays against the eager
        outputs; mean wall time per replay over args.steps back-to-back."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        ok = True
        for _ in range(max(1, args.warmup)):
            out.zero_()
            if pf_out is not None:
                pf_out.zero_()
            graph.replay()
            torch.cuda.synchronize()
            ok = ok and same()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        return ms, ok and same()

    # timed pass: the step captured once as a HIP graph and replayed, as a
    # serving loop runs it (no host launch gaps between the kernels)
    ms_per_step = eager_ms
    graph_ok = None
    sequential_ms = None
    if not args.eager:
        if p is not None:
            sequential_ms, seq_ok = time_graph(step)
            ms_per_step, graph_ok = time_graph(concurrent_step)
            graph_ok = graph_ok and seq_ok
        else:
            ms_per_step, graph_ok = time_graph(step)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    k2_cold_ms = float(cold_k2.mean())
    k2_gbps = k2_bytes / (k2_cold_ms * 1e-3) / 1e9
    k2_warm_gbps = k2_bytes / (k2_ms * 1e-3) / 1e9
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step ({'graph' if not args.eager else 'eager'}; eager "
        f"{eager_ms * 1e3:.1f} us): cache write " + ("in the partition kernel" if fused else f"{cw_ms * 1e3:.1f} us")
        + (f", prefill {pf_ms * 1e3:.1f} us ({pf_flops / (pf_ms * 1e-3) / 1e12:.0f} TFLOP/s)" if p else "")
        + f", partition kernel {k2_ms * 1e3:.1f} us warm ({k2_warm_gbps:.0f} GB/s), {k2_cold_ms * 1e3:.1f} us "
          f"cold ({k2_gbps:.0f} GB/s), reduction {k3_ms * 1e3:.1f} us, "
          f"graph output == eager: {graph_ok}")
    if graph_ok is False:
        raise SystemExit("graph replay disagrees with the eager step")

    # ---- plain device copy: measured bandwidth next to the spec peak
    copy_gbps = plain_copy_GBps(args.copy_probe_gib)

    traffic = None
    tf = traffic_file(args.workload, shared, args.separate_cache_write)
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("kernel_source_sha256") == kernel_source_hash(shared) and rec.get("partition_tokens") == P:
            traffic = rec.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        def sample_bytes(rows):
            kv_r, table_r, qo_r = decode_bytes(d.context_lens[:rows], H, D, elt, bs)
            if args.workload == "prefix13b":
                kv_r = unique_kv_bytes(d.block_tables[:rows], d.context_lens[:rows], H, D, elt, bs)
            return kv_r + table_r + qo_r

        cpu = cpu_baseline(wl, max(1, min(16, _host_cpu()[1])), kv + table + qo + pf_bytes, sample_bytes)

    rec = {
        "metric": METRIC if args.workload == "llama7b" else METRIC_OTHER,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "global_batch": S, "seq_len": int(maxctx),
                   "partition_tokens": P, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(k2_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k2_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": ("shared-prefix decode call (shared, tail and reduction kernels)" if shared
                                else f"decode_partition_kernel<{wl.dtype},{D},{bs}>"
                                + (" with the cache write" if fused else "")),
                     "bytes_per_launch": k2_bytes, "avg_launch_us": round(k2_cold_ms * 1e3, 2),
                     "timing": f"HIP events on the launch stream around each of {args.steps} eager launches, "
                               f"each after a GPU spin (the launches queued ahead) and a {args.evict_mib} MiB "
                               f"{args.evict_mode} that evicts L2 and MALL",
                     "launch_us": pct(cold_k2), "warm_avg_launch_us": round(k2_ms * 1e3, 2),
                     "warm_GBps": round(k2_warm_gbps, 1)},
        "timing": ("hip_graph_replay" + (" of pa_attention_step (prefill on a side stream, concurrent with the "
                                          "decode)" if p is not None else "")) if not args.eager else "eager",
        "eager_ms_per_step": round(eager_ms, 5),
        "cold_step_us": pct(cold_step),
        "hbm_copy_probe_GBps": round(copy_gbps, 1),
        "step_bytes": step_bytes,
        "phases_us": ({"decode_partitions_with_cache_write": round(k2_ms * 1e3, 2)} if fused else
                      {"reshape_and_cache": round(cw_ms * 1e3, 2), "decode_partitions": round(k2_ms * 1e3, 2)})
                     | {"decode_reduce": round(k3_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    if args.block_size is not None:
        used_slots = int((-(-d.context_lens.astype(np.int64) // bs)).sum()) * bs
        rec["config"]["workload"] = rec["config"]["workload"].replace("block_size 16", f"block_size {bs}")
        rec["block_size_tradeoff"] = {"block_size": bs, "slot_utilisation": round(int(d.context_lens.sum()) / used_slots, 5),
                                      "table_bytes": table, "tile_bytes": bs * D * elt}
    if args.workload == "prefix13b":
        rec["aliasing"] = {"path": "shared-prefix decode" if shared else "plain decode",
                           "logical_kv_bytes": logical_kv, "unique_kv_bytes": kv,
                           "logical_GBps": round(logical_kv / (k2_cold_ms * 1e-3) / 1e9, 1),
                           "unique_GBps": round(kv / (k2_cold_ms * 1e-3) / 1e9, 1),
                           # counter-measured HBM bytes of the dominant kernel (the partition kernel, or
                           # the shared-prefix step kernel) over the same time, when recorded for this build
                           "hbm_GBps": None if traffic is None else round(traffic / (k2_cold_ms * 1e-3) / 1e9, 1)}
    if p is not None:
        pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12
        rec["phases_us"]["prefill"] = round(pf_ms * 1e3, 2)
        if sequential_ms is not None:
            rec["sequential_ms_per_step"] = round(sequential_ms, 5)
        rec["prefill"] = {"bound": "mfma", "flops": pf_flops, "achieved_TFLOPs": round(pf_tflops, 1),
                          "peak_TFLOPs": MFMA_PEAK_TFLOPS[wl.dtype],
                          "mfma_frac": round(pf_tflops / MFMA_PEAK_TFLOPS[wl.dtype], 4), "bytes": pf_bytes,
                          "hbm_frac": round(pf_bytes / (pf_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "roofline_us": round(max(pf_flops / (MFMA_PEAK_TFLOPS[wl.dtype] * 1e12),
                                                   pf_bytes / (HBM_PEAK_GBPS * 1e9)) * 1e6, 2)}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
