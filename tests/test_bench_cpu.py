"""Host logic of bench.py that needs no GPU: the per-launch work model, the mapping of a
tagged profile onto steps, the rooflines, the HBM traffic records (reported only while
they were taken on the current sources) and their counter arithmetic, and the CPU
baseline's accounting."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import get_workload  # noqa: E402


def test_step_activity_from_step_counts_and_adoption_steps():
    steps = np.array([2, 3, 1])
    cstep = np.array([[0, 1, 1], [0, 2, 1], [0, 0, 0]])
    act = bench.step_activity(steps, cstep)
    assert len(act) == 3
    assert act[0][0].tolist() == [True, True, True] and act[0][1] == 9
    assert act[1][0].tolist() == [True, True, False] and act[1][1] == 4   # rows adopted at step >= 1
    assert act[2][0].tolist() == [False, True, False] and act[2][1] == 1


def test_class_work_counts_active_sequences_and_masked_rows():
    w = get_workload("sweep64_b32")
    plens = np.arange(1, w.n + 1) * 100
    act = np.zeros(w.n, bool)
    act[[3, 7]] = True
    nb, fl = bench.class_work(w, plens, "attention", act, 10)
    assert nb == (400 + 800) * 2 * w.Hkv * w.hd * 2
    assert fl == sum(4.0 * w.B * (p + w.B) * w.hd * w.H for p in (400, 800))
    nb, fl = bench.class_work(w, plens, "gemm_mlp_up", act, 10)
    assert nb == w.F * w.d * 2 and fl == 2 * w.B * 2 * w.F * w.d
    nb, fl = bench.class_work(w, plens, "lm_head", act, 10)
    assert nb == w.V * w.d * 2 and fl == 2.0 * 10 * w.V * w.d
    assert bench.class_work(w, plens, "commit", act, 10) == (0.0, 0.0)


def _tagged_block(w, S, B):
    """Records of one block issued B steps: embed, per layer qkv / attention / merge / out /
    up / down, LM head, commit; steps >= S take 0.001 ms per launch."""
    recs = []
    for t in range(B):
        d = 1.0 if t < S else 0.001
        recs.append((d * 0.01, (bench.K_EMBED, 0, 0)))
        for l in range(w.L):
            recs += [(d * 0.1, (bench.K_GEMM, 0, l)), (d * 0.2, (bench.K_ATTN, 0, l)), (d * 0.01, (bench.K_MERGE, 0, l)),
                     (d * 0.05, (bench.K_GEMM, 1, l)), (d * 0.15, (bench.K_GEMM, 2, l)), (d * 0.15, (bench.K_GEMM, 3, l))]
        recs += [(d * 0.5, (bench.K_LMHEAD, 0, 0)), (d * 0.01, (bench.K_COMMIT, 0, 0))]
    return recs


def test_summarize_maps_launches_to_steps():
    w = get_workload("sweep64_b8")
    plens = np.full(w.n, 1000)
    steps = np.full(w.n, 5)
    steps[0] = 3
    cstep = np.tile(np.arange(w.B) % 5, (w.n, 1))
    act = bench.step_activity(steps, cstep)
    recs = _tagged_block(w, 5, w.B) * 2
    classes, empty, nblk = bench.summarize(w, plens, recs, act, w.B)
    assert nblk == 2
    assert classes["attention"]["launches"] == 2 * 5 * w.L
    assert abs(classes["attention"]["ms"] - 2 * 5 * w.L * 0.2) < 1e-9
    # prefix bytes: all 64 sequences at steps 0..2, 63 at steps 3..4
    per_seq = 1000 * 2 * w.Hkv * w.hd * 2
    assert classes["attention"]["bytes"] == 2 * w.L * per_seq * (3 * 64 + 2 * 63)
    assert abs(empty - 2 * (w.B - 5) * 0.001 * (0.01 + w.L * 0.66 + 0.51)) < 1e-9
    r = bench.roofline_of(w, "attention", classes["attention"], {})
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["frac"] - classes["attention"]["bytes"] / (classes["attention"]["ms"] * 1e-3) / 1e9 / 8000.0) < 1e-4
    g = bench.roofline_of(w, "gemm_mlp_up", classes["gemm_mlp_up"], {"mfma_bf16_tflops": 2000.0})
    assert g["bound"] == "mfma" and g["unit"] == "TFLOP/s" and abs(g["issued_frac"] - 2 * g["frac"]) < 1e-3


def test_traffic_record_follows_the_kernel_sources(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload, cls: str(path))
    assert bench.traffic_record("x", "attention") is None                      # no record
    rec = dict(source_sha256_16=bench.source_hash(*bench.TRAFFIC_SOURCES["attention"]), ratio=1.02)
    path.write_text(json.dumps(rec))
    assert bench.traffic_record("x", "attention")["ratio"] == 1.02             # taken on these sources
    assert bench.traffic_record("x", "lm_head") is None                        # another kernel's sources
    rec["source_sha256_16"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.traffic_record("x", "attention") is None                      # sources changed since
    path.write_text("not json")
    assert bench.traffic_record("x", "attention") is None


def test_source_hash_covers_every_listed_file():
    names = bench.TRAFFIC_SOURCES["lm_head"]
    assert len({bench.source_hash(n) for n in names}) == len(names)
    assert bench.source_hash(*names) != bench.source_hash(*names[:-1])


def _counter_csv(path, rows):
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    path.write_text(head + "".join(f'{d},"{k}",{c},{v},0,{t}\n' for d, k, c, v, t in rows))


def test_write_traffic_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    # Three working attention dispatches, one that exits at once, and the calibration
    # kernels of a 256 MiB copy: FETCH_SIZE books half of the bytes the elementwise
    # kernel reads, WRITE_SIZE all it writes.
    out = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda workload, cls: str(out))
    kib = 256 * 1024
    mul = "void at::native::vectorized_elementwise_kernel<4, at::native::BinaryFunctor<float, float, float, " \
          "at::native::binary_internal::MulFunctor<float> > >"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    att = "void td::(anonymous namespace)::attn_direct_kernel<unsigned short, 128, 2, 4, 2>(td::AttnArgs)"
    ks = [(1, 262144.0, 64.0), (2, 262150.0, 64.0), (3, 262140.0, 64.0), (4, 1.0, 0.0)]
    _counter_csv(fetch, [(d, att, "FETCH_SIZE", f, 90000) for d, f, _ in ks]
                 + [(5, mul, "FETCH_SIZE", kib / 2, 50000), (6, "__amd_rocclr_copyBuffer", "FETCH_SIZE", kib, 50000)])
    _counter_csv(write, [(d, att, "WRITE_SIZE", w_, 90000) for d, _, w_ in ks]
                 + [(5, mul, "WRITE_SIZE", kib, 50000), (6, "__amd_rocclr_copyBuffer", "WRITE_SIZE", kib, 50000)])
    alg = 262144.0 * 1024 * 2
    rec = bench.write_traffic("x", "attention", str(fetch), str(write), 256, alg)
    assert abs(rec["fetch"]["factor"] - 2.0) < 1e-9 and abs(rec["write"]["factor"] - 1.0) < 1e-9
    assert rec["fetch"]["dispatches"] == 3                        # the exiting dispatch is left out
    assert abs(rec["hbm_bytes_per_launch"] - (262144.0 * 1024 * 2 + 64.0 * 1024)) < 1.0
    assert abs(rec["ratio"] - rec["hbm_bytes_per_launch"] / alg) < 1e-12
    assert rec["source_sha256_16"] == bench.source_hash(*bench.TRAFFIC_SOURCES["attention"])
    assert json.loads(out.read_text())["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"]


def test_cpu_baseline_repeats_whole_block_loops():
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
    assert "batch_step0" not in r                                 # batch of one: no whole-batch step


def test_cpu_baseline_times_one_whole_batch_step_for_large_batches():
    from tests.helpers import mini_workload
    w = mini_workload(n=6, V=64)
    r = bench.cpu_baseline(w, 0.2)
    assert r["batch_step0"]["sequences"] == 6 and r["batch_step0"]["positions_adopted"] >= 6
    assert "sequences 0..3" in r["sample"]


def test_multi_gpu_request_exits_with_a_message(capsys):
    try:
        bench.main(["--gpus", "2"])
    except SystemExit as e:
        assert e.code == 2
    assert "one GPU" in capsys.readouterr().err
