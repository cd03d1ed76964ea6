"""Host logic of the counter summary: calibration on the copy, per-call
totals, and the digest gate that keeps stale figures out of the bench line."""
import csv
import os

import traffic


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_scales_by_the_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    dma = "void specv::(anonymous namespace)::k_dma<specv::DmaCfg<1,2> >(int)"
    pk = "void specv::(anonymous namespace)::k_packed<12>(int)"
    acc = "void specv::(anonymous namespace)::k_accept<unsigned short, true, false>(Args)"
    kib = traffic.COPY_BYTES // 1024
    fetch = [
        # the copy's fetch counter reads half the bytes moved, summed over two channels
        {"Dispatch_Id": 1, "Kernel_Name": copy, "Grid_Size": 4096, "Counter_Value": kib / 4},
        {"Dispatch_Id": 1, "Kernel_Name": copy, "Grid_Size": 4096, "Counter_Value": kib / 4},
        {"Dispatch_Id": 2, "Kernel_Name": dma, "Grid_Size": 64, "Counter_Value": 100},
        {"Dispatch_Id": 3, "Kernel_Name": dma, "Grid_Size": 64, "Counter_Value": 300},
        {"Dispatch_Id": 4, "Kernel_Name": acc, "Grid_Size": 32, "Counter_Value": 50},
        {"Dispatch_Id": 5, "Kernel_Name": pk, "Grid_Size": 512, "Counter_Value": 70},
    ]
    write = [
        {"Dispatch_Id": 1, "Kernel_Name": copy, "Grid_Size": 4096, "Counter_Value": kib},
        {"Dispatch_Id": 2, "Kernel_Name": dma, "Grid_Size": 64, "Counter_Value": 10},
        {"Dispatch_Id": 3, "Kernel_Name": dma, "Grid_Size": 64, "Counter_Value": 10},
        {"Dispatch_Id": 4, "Kernel_Name": acc, "Grid_Size": 32, "Counter_Value": 1},
        {"Dispatch_Id": 5, "Kernel_Name": pk, "Grid_Size": 512, "Counter_Value": 3},
    ]
    _csv(tmp_path / "f.csv", fetch)
    _csv(tmp_path / "w.csv", write)
    res = traffic.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert abs(res["fetch_scale"] - 2.0) < 1e-12 and abs(res["write_scale"] - 1.0) < 1e-12
    launch = res["launches"]["k_dma<specv::DmaCfg<1,2> > grid=64"]
    assert launch["dispatches"] == 2
    assert launch["bytes"] == 200 * 1024 * 2 + 10 * 1024
    assert res["calls"]["lmhead_stored_w"]["bytes"] == launch["bytes"]
    # the lm-head call the benchmark times is the packed-weight product
    assert res["calls"]["lmhead"]["bytes"] == 70 * 1024 * 2 + 3 * 1024
    assert res["calls"]["accept"]["bytes"] == 50 * 1024 * 2 + 1024


def test_stale_summary_is_ignored(tmp_path):
    good = tmp_path / "good.md"
    good.write_text('x\ntraffic: {"source_sha256": "%s", "lmhead_bytes": 7, "accept_bytes": 3}\n'
                    % traffic.source_digest())
    assert traffic.read_committed(str(good))["lmhead_bytes"] == 7
    stale = tmp_path / "stale.md"
    stale.write_text('traffic: {"source_sha256": "00", "lmhead_bytes": 7, "accept_bytes": 3}\n')
    assert traffic.read_committed(str(stale)) is None
    assert traffic.read_committed(str(tmp_path / "missing.md")) is None
