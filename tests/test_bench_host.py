"""Host-side logic of bench.py that turns rocprofv3 counter files into the
HBM traffic record: dispatch order, the step loop's own partition kernel
(side measurements launch other instances later), warm-up dispatches
skipped, and the calibration by a copy of known size. No GPU."""
import argparse
import csv
import json
import os

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
MAIN = "void pa::decode_partition_mfma<16, 4, 2, false, false, 2>(pa::DecodeArgs)"
SIDE = "void pa::decode_partition_valu<unsigned short, 128, 16, 8, 4>(pa::DecodeArgs)"
COPY = "pa::copy_blocks_kernel(pa::CopyArgs)"


def _write(dirname, counter, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for did, name, val in rows:
            w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": val})


def test_traffic_record_from_counter_files(tmp_path):
    warm, steps = 2, 3
    # step loop: 2 warm-up + 3 timed partition launches, then side launches of
    # another instance, then the calibration copies; rows deliberately shuffled
    fetch = [(1, MAIN, 900.0), (2, MAIN, 900.0), (3, MAIN, 100.0), (4, MAIN, 110.0),
             (5, MAIN, 120.0), (6, SIDE, 5000.0), (7, COPY, 10.0), (8, COPY, 64.0),
             (9, COPY, 64.0), (10, COPY, 64.0)]
    write = [(d, n, v / 2) for d, n, v in fetch]
    _write(tmp_path / "f", "FETCH_SIZE", reversed(fetch))
    _write(tmp_path / "w", "WRITE_SIZE", write[::2] + write[1::2])
    out = tmp_path / "rec.json"
    args = argparse.Namespace(traffic_from=[str(tmp_path / "f"), str(tmp_path / "w")],
                              copy_calibration_mib=1, steps=steps, warmup=warm,
                              workload="llama3_8b", traffic_out=str(out))
    assert bench.summarise_traffic(args) == 0
    rec = json.loads(out.read_text())
    # llama3_8b block: 8 heads x 16 x 128 x 2 B = 32 KiB; 1 MiB -> 32 blocks, x2 pools
    known_kib = 2 * 32 * 32768 / 1024
    f, w = rec["FETCH_SIZE"], rec["WRITE_SIZE"]
    assert f["dispatches"] == 3 and f["partition_kib_mean"] == 110.0
    assert w["partition_kib_mean"] == 55.0
    assert f["copy_kib_median"] == 64.0 and f["scale"] == known_kib / 64.0
    assert rec["bytes_per_launch"] == round((110.0 * known_kib / 64.0 + 55.0 * known_kib / 32.0) * 1024)
    assert rec["variant"] == "mfma" and rec["workload"] == "llama3_8b"
    assert rec["source_hash"] == bench.kernel_source_hash()
