"""Host logic of bench.py's profile summaries (CPU only): the calibrated HBM traffic of a pass.

A pass may be several kernels, some dispatched more than once per pass (the T-XL key-side pass:
one storing launch and three adding launches of another kernel).  Its traffic is each kernel's
mean calibrated bytes per dispatch weighted by its dispatches per pass, and each counter is
divided by what it reads for the plain copy of known size."""

import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

STORE = "void relpos::bwd_kernel<unsigned short, 2, 1, 0, 1>(relpos::BwdArgs)"
ADD = "void relpos::bwd_kernel<unsigned short, 2, 1, 0, 0>(relpos::BwdArgs)"
FWD = "void relpos::fwd_kernel<unsigned short, 2>(relpos::FwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pass_traffic_weights_kernels_by_dispatches_per_pass(tmp_path):
    copy_mib = 16
    kib = copy_mib * 1024.0
    # the copy reads FETCH_SIZE = 0.5 x and WRITE_SIZE = 1.0 x its bytes
    fetch = [(COPY, 0.5 * kib)]
    write = [(COPY, 1.0 * kib)]
    passes = 2
    for _ in range(passes):
        fetch += [(STORE, 100.0)] + [(ADD, 40.0)] * 3 + [(FWD, 10.0)]
        write += [(STORE, 1000.0)] + [(ADD, 900.0)] * 3 + [(FWD, 5.0)]
    f_csv, w_csv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(f_csv, "FETCH_SIZE", fetch)
    _write(w_csv, "WRITE_SIZE", write)
    out = tmp_path / "traffic.md"
    bench.summarize_pmc(str(f_csv), str(w_csv), copy_mib, str(out), "cmd")
    recs = {}
    for line in open(out):
        if line.startswith("traffic-record: "):
            r = json.loads(line[len("traffic-record: "):])
            recs[(r["mech"], r["pass"])] = r["bytes_per_pass"]
    per_kib = 1024.0
    want_dkdv = ((100.0 / 0.5 + 1000.0) + 3 * (40.0 / 0.5 + 900.0)) * per_kib
    want_fwd = (10.0 / 0.5 + 5.0) * per_kib
    assert abs(recs[("txl", "bwd_dkdv")] - want_dkdv) < 1e-6 * want_dkdv
    assert abs(recs[("txl", "fwd")] - want_fwd) < 1e-6 * want_fwd


def test_pass_of_kernel_names():
    assert bench.pass_of_kernel(STORE) == ("txl", "bwd_dkdv")
    assert bench.pass_of_kernel("void relpos::bwd_kernel<unsigned short, 0, 0, 0, -1>(relpos::BwdArgs)") == ("t5", "bwd_dq")
    assert bench.pass_of_kernel(FWD) == ("txl", "fwd")
    assert bench.pass_of_kernel(COPY) is None
