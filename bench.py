#!/usr/bin/env python3
"""Paged decode attention throughput at the LLaMA-7B layer shape on one MI355X.

Workload (seeded, synthetic): 64 sequences x 32 heads x head_dim 128, f16,
block_size 16, context lengths ~ U[128, 2048], block tables = slices of one
random permutation of a pool sized to fit exactly, q/K/V ~ N(0,1).

One step = one decode iteration of one attention layer, all inputs resident
in HBM: reshape_and_cache of the 64 new tokens, then split-K decode
(partition kernel + reduction kernel) with an f16 output. The timed steps
replay the step captured as a HIP graph (checked bit-identical to the eager
step); --eager times plain launches instead.

Prints ONE JSON line: value = algorithmic bytes of the step / step time
(GB/s, 1e9 B/s); roofline = the partition kernel's algorithmic bytes over its
average launch time (HIP events on the launch stream) against the 8 TB/s HBM
peak; cpu_baseline = the fp64 oracle on the host cores over the same decode.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention achieved HBM GB/s (% of peak) at LLaMA-7B layer shape"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama7b_traffic.json")
KERNEL_SOURCES = ["pa_decode.hip", "pa_device.h", "pa_internal.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_391_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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


def record_traffic(fetch_dir, write_dir, copy_bytes):
    """Turn two counter runs of this benchmark (FETCH_SIZE, then WRITE_SIZE;
    both in KiB per dispatch) into HBM bytes per launch of the partition
    kernel, each scaled by what the same counter reads for the plain device
    copy of known size in the same run, and store them with the hash of the
    kernel source they describe."""
    out = {}
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _counter_rows(d)
        part = [v for k, v in rows if "decode_partition_kernel" in k]
        copy = [v for k, v in rows if "copyBuffer" in k or "copy" in k.lower()]
        copy = max(copy)  # the 1 GiB probe copy is the largest copy dispatch
        scale = (copy_bytes / 1024.0) / copy
        out[name] = {"partition_kernel_kib_avg": sum(part) / len(part), "copy_kib": copy, "scale": scale,
                     "dispatches": len(part)}
    fetch = out["fetch"]["partition_kernel_kib_avg"] * 1024 * out["fetch"]["scale"]
    write = out["write"]["partition_kernel_kib_avg"] * 1024 * out["write"]["scale"]
    rec = {"kernel": "decode_partition_kernel<f16,128,16>", "workload": "llama7b decode (bench.py)",
           "kernel_source_sha256": kernel_source_hash(), "hbm_bytes_per_launch": round(fetch + write),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write), "counters": out}
    import paged_kv_cache_391_amd as pa
    rec["partition_tokens"] = pa.decode_partition_tokens()
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--copy-probe-gib", type=float, default=1.0, help="size of the plain-copy bandwidth probe")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="store HBM bytes per launch from two rocprofv3 --pmc runs of this script and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic[0], args.record_traffic[1], int(args.copy_probe_gib * (1 << 30)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: each GPU would run this path on its own share of sequences or "
            "heads with no collective in the timed region, so only --gpus 1 is measured.")
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_391_amd as pa
    from tests._gpu import OnDevice
    from workloads import config2

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    t = time.time()
    wl = config2()
    log(f"[bench] generated workload in {time.time() - t:.1f}s: {wl.num_blocks} blocks, "
        f"sum ctx {int(wl.decode.context_lens.sum())}")
    od = OnDevice(wl)
    d = wl.decode
    S, H, D, bs, elt = d.num_seqs, wl.num_heads, wl.head_dim, wl.block_size, wl.elt_bytes
    maxctx = d.max_context_len
    ws = pa.make_decode_workspace(S, H, D, maxctx)
    out = torch.empty_like(od.q)  # f16 output: the production path
    P = pa.decode_partition_tokens()

    def step(ev=None):
        pa.reshape_and_cache(od.new_k, od.new_v, od.k_cache, od.v_cache, od.slot_mapping)
        if ev is not None:
            ev[0].record()
        pa.paged_attention_decode_partitions(out, od.q, od.k_cache, od.v_cache, od.block_tables, od.context_lens,
                                             wl.scale, maxctx, ws)
        if ev is not None:
            ev[1].record()
        pa.paged_attention_decode_reduce(out, od.context_lens, D, maxctx, od.q.dtype, ws)
        if ev is not None:
            ev[2].record()

    # ---- algorithmic bytes (valid tokens only)
    ctx = d.context_lens.astype(np.int64)
    kv_bytes = int(ctx.sum()) * H * D * elt * 2
    table_bytes = int(np.ceil(ctx / bs).sum()) * 4 + 4 * S
    qo_bytes = 2 * S * H * D * elt
    T = int(wl.new.slot_mapping.shape[0])
    cache_write_bytes = 4 * T * H * D * elt + 4 * T
    nparts = np.ceil(np.ceil(ctx / 16) / (P // 16)).astype(np.int64)
    k2_writes = int(np.where(nparts > 1, nparts * H * (D + 2) * 4, H * D * elt).sum())
    k2_bytes = kv_bytes + table_bytes + S * H * D * elt + k2_writes
    decode_bytes = kv_bytes + table_bytes + qo_bytes
    step_bytes = decode_bytes + cache_write_bytes

    # eager pass: HIP events on the launch stream around every partition-kernel launch
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    k2_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    k3_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    eager_out = out.clone()

    # timed pass: the step captured once as a HIP graph and replayed, as a
    # serving loop runs decode (no host launch gaps between the 3 kernels)
    ms_per_step = eager_ms
    graph_ok = None
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
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        graph_ok = graph_ok and bool(torch.equal(out, eager_out))
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    k2_gbps = k2_bytes / (k2_ms * 1e-3) / 1e9
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step ({'graph' if not args.eager else 'eager'}; eager "
        f"{eager_ms * 1e3:.1f} us), partition kernel {k2_ms * 1e3:.1f} us ({k2_gbps:.0f} GB/s), "
        f"reduction {k3_ms * 1e3:.1f} us, graph output == eager: {graph_ok}")
    if graph_ok is False:
        raise SystemExit("graph replay disagrees with the eager step")

    # ---- plain device copy: measured bandwidth next to the spec peak
    n = int(args.copy_probe_gib * (1 << 30)) // 4
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
    copy_gbps = 2 * n * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("kernel_source_sha256") == kernel_source_hash() and rec.get("partition_tokens") == P:
            traffic = rec.get("hbm_bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        kc, vc = oracle.reshape_and_cache(wl.new.k, wl.new.v, wl.k_cache, wl.v_cache, wl.new.slot_mapping, bs,
                                          wl.dtype)
        threads = max(1, min(16, os.cpu_count() or 1))
        t = time.perf_counter()
        oracle.decode(d.q, kc, vc, d.block_tables, d.context_lens, wl.scale, wl.dtype, threads=threads)
        cpu_s = time.perf_counter() - t
        cpu = {"value": round(decode_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole decode of this workload ({S} seqs x {H} heads, one pass, {cpu_s:.2f} s); "
                         "fp64, gather + softmax attention per (seq, head), OpenMP over pairs"}

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama7b_decode_step: reshape_and_cache of 64 new tokens + split-K paged decode, "
                               "64 seqs x 32 heads x 128, f16, block_size 16, ctx U[128,2048], seed 393",
                   "global_batch": S, "seq_len": int(maxctx), "partition_tokens": P, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "achieved": round(k2_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(k2_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "decode_partition_kernel<f16,128,16>", "bytes_per_launch": k2_bytes,
                     "avg_launch_us": round(k2_ms * 1e3, 2)},
        "timing": "hip_graph_replay" if not args.eager else "eager",
        "eager_ms_per_step": round(eager_ms, 5),
        "hbm_copy_probe_GBps": round(copy_gbps, 1),
        "step_bytes": step_bytes,
        "reduce_kernel_avg_us": round(k3_ms * 1e3, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
