"""Host-side parts of bench.py: the CPU-oracle baselines and the one-GPU guard (no GPU needed)."""
import subprocess
import sys

import numpy as np

import bench
from nvfp4_w4a4_block_amd import workloads as WL


def test_cpu_baseline_record_shape_and_row_count():
    """The oracle baseline of a GEMM workload: both thread settings reported, and the sample never
    claims more weight rows than the matrix has (tiny: 256 rows)."""
    wl = WL.get("tiny")
    rec = bench.cpu_baseline(wl, 0.02)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0
    assert rec["single_thread"]["cores"] == 1 and rec["single_thread"]["value"] > 0
    assert f"first {wl.N} of {wl.N} weight rows" in rec["sample"]


def test_kv_cpu_baseline_record_shape():
    bits = WL.make_kv(tokens=32)
    rec = bench.kv_cpu_baseline(bits, 0.02)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["value"] > 0 and rec["cores"] == 1
    assert f"first {bits.size} elements" in rec["sample"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU only" in r.stderr
