"""Host-side parts of bench.py: turning two rocprofv3 counter databases into HBM bytes per attention call.

The databases here are synthetic sqlite files with the one table the summariser reads, so the arithmetic
(calibration against the copy kernel, per-kernel means, which kernels make up the attention call) is checked
without a GPU.
"""

from __future__ import annotations

import json
import os
import sqlite3

import bench

# every kernel an attention call can launch, with a distinct per-dispatch counter value
ATTENTION_KERNELS = {
    "void pa::(anonymous namespace)::decode_valu_kernel<1, 128>(pa::DecodeArgs)": 11,
    "void pa::(anonymous namespace)::decode_valu_balanced_kernel<1, 128, false>(pa::DecodeArgs)": 13,
    "void pa::(anonymous namespace)::decode_gqa_mfma_kernel<1, 128, 8>(pa::DecodeArgs)": 17,
    "void pa::(anonymous namespace)::decode_gqa_mfma_balanced_kernel<1, 128, 8>(pa::DecodeArgs)": 19,
    "void pa::(anonymous namespace)::lse_reduce_kernel<128>(pa::DecodeArgs)": 23,
    "void pa::(anonymous namespace)::balanced_reduce_kernel<128>(pa::DecodeArgs)": 29,
}
COPY = "pa::(anonymous namespace)::stream_copy_kernel(pa::U4*, pa::U4 const*, long)"
OTHER = "pa::(anonymous namespace)::reshape_and_cache_kernel(pa::U4 const*, pa::U4 const*, pa::U4*, pa::U4*, int const*"


def make_db(path, counter, copy_value, scale):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, dispatch_id int, counter_name text, value real)")
    rows, d = [], 0
    for _ in range(3):  # three dispatches of each, with the counter split over two entries (two XCD samples)
        for name, v in [(COPY, copy_value)] + [(k, v * scale) for k, v in ATTENTION_KERNELS.items()] + [(OTHER, 1e9)]:
            d += 1
            rows += [(name, d, counter, v / 2), (name, d, counter, v / 2)]
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_traffic_summary_counts_every_attention_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda label: os.path.join(tmp_path, f"traffic_{label}.md"))
    fetch_db, write_db = os.path.join(tmp_path, "f.db"), os.path.join(tmp_path, "w.db")
    # the copy kernel moves COPY_BYTES each way: FETCH_SIZE reads 2 MiB units of it here, WRITE_SIZE 1 MiB
    make_db(fetch_db, "FETCH_SIZE", bench.COPY_BYTES / 2048.0, 1000.0)
    make_db(write_db, "WRITE_SIZE", bench.COPY_BYTES / 1024.0, 10.0)
    path = bench.write_traffic_summary("tiny_fp32", fetch_db, write_db, "cmd f", "cmd w")
    text = open(path).read()
    for name in ATTENTION_KERNELS:
        assert name[:90] in text, f"{name} missing from the summary"
    assert OTHER[:60] not in text and COPY[:60] not in text
    rec = json.loads(text.split(bench.TRAFFIC_TAG, 1)[1].rsplit("-->", 1)[0])
    total = sum(ATTENTION_KERNELS.values())
    assert rec["fetch_bytes_per_call"] == round(total * 1000.0 * 2048)
    assert rec["write_bytes_per_call"] == round(total * 10.0 * 1024)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()


def test_stored_traffic_is_ignored_once_the_kernels_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda label: os.path.join(tmp_path, f"traffic_{label}.md"))
    rec = {"kernel_source_hash": bench.kernel_source_hash(), "bytes_per_call": 123}
    with open(bench.traffic_path("w"), "w") as f:
        f.write("# x\n" + bench.TRAFFIC_TAG + json.dumps(rec) + " -->\n")
    assert bench.load_traffic("w") == 123
    rec["kernel_source_hash"] = "0" * 16
    with open(bench.traffic_path("w"), "w") as f:
        f.write("# x\n" + bench.TRAFFIC_TAG + json.dumps(rec) + " -->\n")
    assert bench.load_traffic("w") is None
