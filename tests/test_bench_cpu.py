"""Host logic of bench.py that needs no GPU: the HBM traffic record is reported only while
it was taken on the current LM-head sources, and its counter arithmetic."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_record_follows_the_kernel_sources(tmp_path, monkeypatch):
    path = tmp_path / "lmhead_x_traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(path))
    assert bench.traffic_record("x") is None                      # no record
    rec = dict(source_sha256_16=bench.source_hash(*bench.LMHEAD_SOURCES), hbm_bytes_per_launch=123.0)
    path.write_text(json.dumps(rec))
    assert bench.traffic_record("x") == 123.0                     # taken on these sources
    rec["source_sha256_16"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.traffic_record("x") is None                      # sources changed since
    path.write_text("not json")
    assert bench.traffic_record("x") is None


def test_source_hash_covers_every_listed_file():
    names = bench.LMHEAD_SOURCES
    assert len({bench.source_hash(n) for n in names}) == len(names)
    assert bench.source_hash(*names) != bench.source_hash(*names[:-1])


def _counter_csv(path, rows):
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    path.write_text(head + "".join(f'{d},"{k}",{c},{v},0,{t}\n' for d, k, c, v, t in rows))


def test_write_traffic_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    # Three working LM-head dispatches, one that exits at once, and the calibration
    # kernels of a 256 MiB copy: FETCH_SIZE books half of the bytes the elementwise
    # kernel reads, WRITE_SIZE all it writes.
    out = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload: str(out))
    kib = 256 * 1024
    mul = "void at::native::vectorized_elementwise_kernel<4, at::native::BinaryFunctor<float, float, float, " \
          "at::native::binary_internal::MulFunctor<float> > >"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    lm = [(1, 262144.0, 64.0), (2, 262150.0, 64.0), (3, 262140.0, 64.0), (4, 1.0, 0.0)]
    _counter_csv(fetch, [(d, "lmhead_lds_kernel", "FETCH_SIZE", f, 90000) for d, f, _ in lm]
                 + [(5, mul, "FETCH_SIZE", kib / 2, 50000), (6, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib, 50000)])
    _counter_csv(write, [(d, "lmhead_lds_kernel", "WRITE_SIZE", w_, 90000) for d, _, w_ in lm]
                 + [(5, mul, "WRITE_SIZE", kib, 50000), (6, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib, 50000)])
    rec = bench.write_traffic("x", str(fetch), str(write), 256)
    assert abs(rec["fetch"]["factor"] - 2.0) < 1e-9 and abs(rec["write"]["factor"] - 1.0) < 1e-9
    assert rec["working_launches"] == 3                           # the exiting dispatch is left out
    assert abs(rec["hbm_bytes_per_launch"] - (262144.0 * 1024 * 2 + 64.0 * 1024)) < 1.0
    assert rec["source_sha256_16"] == bench.source_hash(*bench.LMHEAD_SOURCES)
    assert json.loads(out.read_text())["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"]


def test_cpu_baseline_repeats_whole_block_loops():
    from synth import get_workload
    w = get_workload("tiny_fp32")
    r = bench.cpu_baseline(w, 0.3)       # floor min(0.3 s, 10 s): whole loops, none past 0.3 s
    assert r["kind"] == "oracle" and r["unit"] == "committed tokens/s" and r["cores"] >= 1
    assert r["seconds"] >= 0.3 or "cut at the time budget" in r["sample"]
    blocks = int(r["sample"].split(": ")[1].split(" whole")[0])
    adopted = int(r["sample"].split("), ")[1].split(" positions")[0])
    assert blocks >= 1
    cut = "cut at the time budget" in r["sample"]
    assert adopted == blocks * w.B or (cut and blocks * w.B < adopted < (blocks + 1) * w.B)
    assert abs(r["value"] - adopted / r["seconds"]) < 1e-6 * r["value"]
