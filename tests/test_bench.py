"""bench.py's contract: one GPU only, the algorithmic byte counts behind its
rates, and the JSON line it prints."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_decode_bytes_by_hand():
    # two sequences of 1 and 17 tokens, 2 heads x 4 dims, 2-byte elements, blocks of 16
    kv, table, qo = bench.decode_bytes(np.array([1, 17]), 2, 4, 2, 16)
    assert kv == (1 + 17) * 2 * 4 * 2 * 2          # K and V of every valid token
    assert table == (1 + 2) * 4 + 2 * 4             # one entry per used block, one length per sequence
    assert qo == 2 * 2 * 2 * 4 * 2                  # q and out rows


def test_partition_kernel_bytes_by_hand():
    # 600 tokens split into two 512-token partitions: (m, l, acc) per partition in fp32;
    # 100 tokens in one partition: the output row in the input type
    ctx = np.array([600, 100])
    kv, table, _ = bench.decode_bytes(ctx, 2, 4, 2, 16)
    q = 2 * 2 * 4 * 2
    writes = 2 * 2 * (4 + 2) * 4 + 2 * 4 * 2
    assert bench.partition_kernel_bytes(ctx, 2, 4, 2, 16, 512) == kv + table + q + writes


def test_unique_kv_bytes_counts_aliased_slots_once():
    bt = np.array([[3, 5], [3, 6]], dtype=np.int32)  # both rows alias block 3
    ctx = np.array([20, 18])
    got = bench.unique_kv_bytes(bt, ctx, 2, 4, 2, 16)
    slots = 16 + 4 + 2  # block 3 once, 4 tokens of block 5, 2 of block 6
    assert got == slots * 2 * 4 * 2 * 2


def test_prefill_work_by_hand():
    class P:
        query_start_loc = np.array([0, 3])
        context_lens = np.array([5])
    flops, byts = bench.prefill_work(P, 1, 4, 2)
    # 3 queries after 2 cached tokens: 2*3 + (1+2+3) = 12 unmasked pairs, 4 flops per pair per dim
    assert flops == 4 * 4 * 1 * (3 * 2 + 6)
    assert byts == 5 * 1 * 4 * 2 * 2 + 2 * 3 * 1 * 4 * 2


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "bench_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f'"{name}",X,{value}\n')
    return path


@pytest.mark.parametrize("workload,shared,kernel", [
    ("llama7b", False, "void pa::decode_partition_kernel<(pa::Dt)1, 128, 16, 1, (pa::RowMode)0>(pa::DecodeArgs)"),
    ("prefix13b", True, "void pa::shared_prefix_step_kernel<(pa::Dt)1, 128, 16>(pa::DecodeArgs, int)"),
    ("prefill_long", False, "void pa::prefill_mfma_kernel<(pa::Dt)1, 128, 16>(pa::PrefillArgs)")])
def test_traffic_record_scales_counters_by_the_plain_copy(tmp_path, monkeypatch, workload, shared, kernel):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the recorded kernel,
    each scaled by what the same counter reads for the plain copy of known
    size, averaged over its dispatches; stamped with the hash of the sources
    the kernel is built from. Other kernels in the run are ignored."""
    copy_bytes = 1 << 30
    other = "pa::reshape_and_cache_kernel(int)"
    fetch = _counter_csv(str(tmp_path / "f"), [(kernel, 1000.0), (kernel, 3000.0), (other, 9e9),
                                               ("__amd_rocclr_copyBuffer", 524288.0), ("__amd_rocclr_copyBuffer", 10.0)])
    write = _counter_csv(str(tmp_path / "w"), [(kernel, 40.0), (kernel, 60.0), (other, 9e9),
                                               ("__amd_rocclr_copyBuffer", 1048576.0)])
    out = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_file", lambda w, s=False, sep=False: str(out))
    bench.record_traffic(workload, shared, fetch, write, copy_bytes)
    rec = json.load(open(out))
    assert rec["fetch_bytes_per_launch"] == round(2000.0 * 1024 * 2.0)  # the copy's FETCH reads half its bytes
    assert rec["write_bytes_per_launch"] == round(50.0 * 1024 * 1.0)
    assert rec["hbm_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash(shared, workload)
    assert rec["kernel"] == bench.traffic_kernel(shared, workload)


def test_traffic_records_name_the_roofline_kernels():
    assert bench.traffic_kernel(False) == "decode_partition_kernel"
    assert bench.traffic_kernel(True) == "shared_prefix_step_kernel"
    assert bench.traffic_kernel(False, "prefill_long") == "prefill_mfma_kernel"
    assert bench.kernel_source_hash(False, "prefill_long") != bench.kernel_source_hash(False)
    assert bench.traffic_file("prefill_long").endswith("prefill_long_traffic.json")
    assert bench.traffic_file("prefix13b", True).endswith("decode_prefix13b_shared_traffic.json")
    assert bench.traffic_file("prefix13b", False).endswith("decode_prefix13b_plain_traffic.json")
    assert bench.traffic_file("llama7b", False, True).endswith("decode_llama7b_separate_write_traffic.json")


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline", "--copy-probe-gib", "0.25"], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in rec
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["unit"] == "GB/s" and rec["higher_is_better"] is True and rec["data"] == "synthetic"
    assert "workload" in rec["config"]
    rf = rec["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.2 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0 < rec["value"] < 8000.0


def test_prefill_long_workload_and_its_flops():
    """8 chunks of 512 queries after 1536 cached tokens, 40 heads x 128:
    4 d H (L c + L(L+1)/2) per chunk = 150.37 GFLOP per step."""
    wl = bench.prefill_config()
    p = wl.prefill
    assert p.num_seqs == 8 and p.total_q == 8 * 512
    assert (np.asarray(p.context_lens) == 2048).all()
    flops, byts = bench.prefill_work(p, wl.num_heads, wl.head_dim, wl.elt_bytes)
    assert flops == 8 * 4 * 128 * 40 * (512 * 1536 + 512 * 513 // 2) == 150_365_798_400
    assert byts == 8 * (2048 * 40 * 128 * 2 * 2 + 2 * 512 * 40 * 128 * 2)


@pytest.mark.gpu
def test_bench_prefill_long_prints_the_mfma_roofline():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "prefill_long", "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline"], capture_output=True, text=True, timeout=240,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    assert rec["unit"] == "TFLOP/s" and rec["n_gpus"] == 1
    rf = rec["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0.05 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def _local_includes(name, seen=None):
    """The csrc files a source pulls in through quoted includes, itself included."""
    import re
    seen = set() if seen is None else seen
    if name in seen:
        return seen
    seen.add(name)
    text = open(os.path.join(ROOT, "paged_kv_cache_391_amd", "csrc", name)).read()
    for inc in re.findall(r'^#include "([^"/]+)"', text, flags=re.M):
        _local_includes(inc, seen)
    return seen


def test_traffic_hashes_cover_every_file_the_kernels_are_built_from():
    """A traffic record stays in use only while the hash of the listed kernel
    sources matches; a header the kernel includes but the list misses could
    change the kernel without retiring the record."""
    assert _local_includes("pa_decode.hip") <= set(bench.KERNEL_SOURCES)
    assert _local_includes("pa_shared.hip") <= set(bench.SHARED_KERNEL_SOURCES)
    assert _local_includes("pa_prefill.hip") <= set(bench.PREFILL_KERNEL_SOURCES)
