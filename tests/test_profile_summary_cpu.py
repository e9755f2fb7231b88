"""The rocprofv3 summary tool behind profiles/ (host only): the traffic record's arithmetic and its
source hash, which bench.py compares before it reports a record's bytes."""
import csv
import json
import os
import subprocess
import sys

import bench
from nvfp4_w4a4_block_amd import profile_summary as PS

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counter_csv(path, counter, kernel_kib, copy_kib):
    """Three dispatches of a kernel, then three reference copies (what bench.py --copy-reference-mib runs)."""
    rows, d = [], 0
    for v in kernel_kib:
        d += 1
        rows.append({"Dispatch_Id": d, "Kernel_Name": "void ns::my_kernel<1>(int)", "Counter_Name": counter,
                     "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 1})
    for _ in range(3):
        d += 1
        rows.append({"Dispatch_Id": d, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                     "Counter_Value": copy_kib, "Start_Timestamp": 0, "End_Timestamp": 1})
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows)


def test_traffic_record_scales_each_counter_by_the_reference_copy(tmp_path):
    # a 128 MiB copy reads 128 MiB and writes 128 MiB; suppose the counters report half the reads
    # (FETCH_SIZE) and all the writes (WRITE_SIZE): the kernel's bytes are rescaled by the same factors
    fetch, write, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "rec.json"
    _counter_csv(fetch, "FETCH_SIZE", [1000.0, 1000.0, 1000.0], 65536.0)
    _counter_csv(write, "WRITE_SIZE", [10.0, 30.0, 20.0], 131072.0)
    src = os.path.relpath(bench.__file__, PS.ROOT)
    subprocess.run([sys.executable, "-m", "nvfp4_w4a4_block_amd.profile_summary", "traffic", str(fetch), str(write),
                    str(out), "--kernel", "my_kernel", "--sources", src, "--command", "fetch pass",
                    "--command", "write pass"], check=True, cwd=PS.ROOT)
    rec = json.loads(out.read_text())
    assert rec["dispatches"] == 3
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["traffic_bytes_per_launch"] == (1000 * 2 + 20) * 1024
    assert rec["sources_sha256"] == PS.sources_sha256([src])


def test_every_committed_traffic_record_names_existing_sources_and_a_positive_count():
    d = os.path.join(PS.ROOT, "profiles")
    recs = [f for f in os.listdir(d) if f.startswith("traffic_") and f.endswith(".json")]
    assert recs
    for f in recs:
        rec = json.load(open(os.path.join(d, f)))
        assert rec["traffic_bytes_per_launch"] > 0 and rec["dispatches"] > 0, f
        for src in rec["sources"]:
            assert os.path.exists(os.path.join(PS.ROOT, src)), (f, src)
        assert len(rec["commands"]) == 2 and "FETCH_SIZE" in rec["commands"][0] and "WRITE_SIZE" in rec["commands"][1], f
