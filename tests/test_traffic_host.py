"""Host logic of the traffic harness (exact_attention_89_amd/traffic.py) on synthetic
counter files: calibration against the copy kernel, per-call and per-kernel
accounting, the guard on the calibration dispatches.  No GPU involved."""

from __future__ import annotations

import argparse
import csv
import json
import os

import pytest

from exact_attention_89_amd import traffic

MUL = "void at::native::vectorized_elementwise_kernel<4, MulFunctor<float> >(int)"
FUSED = "void attn89::(anonymous namespace)::attn_fwd_bf16_pp_kernel<128, false>(attn89::FwdArgs)"
SPLIT = "void attn89::(anonymous namespace)::attn_fwd_bf16_4w_kernel<128, false, true>(attn89::FwdArgs)"
MERGE = "void attn89::(anonymous namespace)::splitkv_merge_kernel<128>(attn89::FwdArgs)"


def _write_counters(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name",
                    "Counter_Value"])
        for did, (name, kib) in enumerate(rows, start=1):
            w.writerow([did, did, name, counter, kib])


def _make_run(root, impl, manifest, fetch_rows, write_rows):
    d = os.path.join(root, impl)
    os.makedirs(d, exist_ok=True)
    json.dump(manifest, open(os.path.join(d, "manifest.json"), "w"))
    _write_counters(os.path.join(d, "fetch", "x", "f_counter_collection.csv"), "FETCH_SIZE",
                    fetch_rows)
    _write_counters(os.path.join(d, "write", "x", "w_counter_collection.csv"), "WRITE_SIZE",
                    write_rows)


def _cal(n=2):
    return {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "dispatches": n}


def test_calibration_and_per_call_bytes(tmp_path):
    # the copy reads 1 GiB; FETCH_SIZE reports half the KiB (factor 2), WRITE_SIZE all
    man = {"impl": "fused", "calls": 2, "calibration": _cal(),
           "entries": [{"N": 1024, "causal": 1, "dispatches_per_call": 1,
                        "algorithmic_bytes": 123, "one_score_matrix_16bit_all_heads": 0}]}
    fetch = [(MUL, 524288.0), (MUL, 524288.0), (FUSED, 1000.0), (FUSED, 1200.0)]
    write = [(MUL, 1048576.0), (MUL, 1048576.0), (FUSED, 300.0), (FUSED, 300.0)]
    _make_run(str(tmp_path), "fused", man, fetch, write)
    _, cal, entries = traffic._load_run(str(tmp_path), "fused")
    assert cal["fetch_factor"] == pytest.approx(2.0) and cal["write_factor"] == pytest.approx(1.0)
    e = entries[0]
    assert e["read_bytes"] == pytest.approx((1000 + 1200) * 1024 * 2 / 2)
    assert e["write_bytes"] == pytest.approx(300 * 1024)
    assert e["per_kernel"][FUSED][0] == pytest.approx(e["read_bytes"])


def test_dispatches_split_between_entries_and_kernels(tmp_path):
    # two entries of a two-launch path (split kernel + merge), two calls each
    man = {"impl": "decode", "calls": 2, "calibration": _cal(1),
           "entries": [{"Nk": 8192, "dispatches_per_call": 2, "algorithmic_bytes": 1},
                       {"Nk": 16384, "dispatches_per_call": 2, "algorithmic_bytes": 1}]}
    fetch = [(MUL, 1048576.0)] + [(SPLIT, 100.0), (MERGE, 1.0)] * 2 + [(SPLIT, 200.0),
                                                                      (MERGE, 2.0)] * 2
    write = [(MUL, 1048576.0)] + [(SPLIT, 10.0), (MERGE, 4.0)] * 4
    _make_run(str(tmp_path), "decode", man, fetch, write)
    _, cal, entries = traffic._load_run(str(tmp_path), "decode")
    assert cal["fetch_factor"] == pytest.approx(1.0)
    assert [e["read_bytes"] for e in entries] == pytest.approx([101 * 1024, 202 * 1024])
    assert entries[1]["per_kernel"][SPLIT][0] == pytest.approx(200 * 1024)
    assert entries[1]["per_kernel"][MERGE][1] == pytest.approx(4 * 1024)


def test_calibration_must_come_first(tmp_path):
    man = {"impl": "fused", "calls": 1, "calibration": _cal(1),
           "entries": [{"N": 1, "causal": 0, "dispatches_per_call": 1, "algorithmic_bytes": 1,
                        "one_score_matrix_16bit_all_heads": 0}]}
    _make_run(str(tmp_path), "fused", man, [(FUSED, 1.0), (MUL, 1.0)],
              [(FUSED, 1.0), (MUL, 1.0)])
    with pytest.raises(SystemExit, match="calibration"):
        traffic._load_run(str(tmp_path), "fused")


def test_summarize_decode_writes_records(tmp_path):
    man = {"impl": "decode", "calls": 1, "calibration": _cal(1), "kernel_source_hash": "abc",
           "entries": [{"B": 1, "H": 8, "Nq": 1, "Nk": 65536, "D": 128, "num_splits": 64,
                        "dispatches_per_call": 2, "algorithmic_bytes": 256 << 20}]}
    _make_run(str(tmp_path), "decode", man,
              [(MUL, 1048576.0), (SPLIT, 256.0 * 1024), (MERGE, 270.0)],
              [(MUL, 1048576.0), (SPLIT, 256.0), (MERGE, 0.0)])
    out_json, out_md = tmp_path / "d.json", tmp_path / "d.md"
    traffic.cmd_summarize_decode(argparse.Namespace(dir=str(tmp_path), out_json=str(out_json),
                                                    out_md=str(out_md), command=["cmd"]))
    rec = json.load(open(out_json))
    assert rec["kernel_source_hash"] == "abc"
    e = rec["entries"][0]
    assert e["read_bytes"] == pytest.approx((256 * 1024 + 270) * 1024)
    assert "| 1 | 8 | 1 | 65536 | 128 | 64 |" in out_md.read_text()


def test_source_hashes_cover_the_kernel_files():
    # a traffic record is tied to the sources of the kernels it measured
    assert len(traffic._kernel_hash()) == 16
    assert traffic._kernel_hash() != traffic._fp8_hash() != traffic._decode_hash()
