"""The benchmark's host-side contract (CPU only): one GPU only, a clear exit
without a GPU, the documented flags, and the rule that the recorded HBM
traffic is reported only while the files it was taken on are unchanged."""
import json
import os
import shutil

import pytest

import bench


def test_more_than_one_gpu_exits_with_a_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    err = capsys.readouterr().err
    assert "one GPU" in err and "--gpus 2" in err


def test_no_gpu_exits_cleanly(capsys):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert bench.main([]) == 2
    assert "needs a GPU" in capsys.readouterr().err


def test_documented_flags_parse():
    a = bench.parse_args(["--gpus", "1", "--steps", "5", "--warmup", "3", "--workload", "llama3_70b_layer",
                          "--rotate-gib", "0.5", "--eager", "--no-cpu-baseline", "--no-secondary",
                          "--calibrate-copy", "1024", "--detail"])
    assert (a.gpus, a.steps, a.warmup, a.workload, a.rotate_gib) == (1, 5, 3, "llama3_70b_layer", 0.5)
    assert a.eager and a.no_cpu_baseline and a.no_secondary and a.detail and a.calibrate_copy == 1024
    for flag in ("--quantizer-only", "--w8a8-only", "--kv-only", "--fp16-only"):
        assert getattr(bench.parse_args([flag]), flag[2:].replace("-", "_"))
    d = bench.parse_args([])
    assert d.gpus == 1 and d.steps == 0 and d.warmup == 0 and d.workload == "llama3_8b_decode"


def test_recorded_traffic_follows_the_hashed_files(tmp_path, monkeypatch):
    rec_path = os.path.join(bench.ROOT, "profiles", "decode_llama3_8b_hbm_traffic.json")
    rec = json.load(open(rec_path))
    # a copy of the tree holding exactly the hashed files and the record
    root = tmp_path / "tree"
    for rel in list(rec["sources_sha256"]) + ["profiles/decode_llama3_8b_hbm_traffic.json"]:
        dst = root / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copyfile(os.path.join(bench.ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.recorded_traffic("llama3_70b_layer") is None  # recorded for the 8B decode step only
    live = bench.recorded_traffic("llama3_8b_decode")
    # the committed record either matches the committed sources or is stale
    assert live is None or live == pytest.approx(float(rec["traffic_bytes_per_launch"]))
    # forge a record for the copied files: reported while they match...
    import hashlib
    rec["sources_sha256"] = {rel: hashlib.sha256((root / rel).read_bytes()).hexdigest()
                             for rel in rec["sources_sha256"]}
    (root / "profiles" / "decode_llama3_8b_hbm_traffic.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("llama3_8b_decode") == pytest.approx(float(rec["traffic_bytes_per_launch"]))
    # ...and null once any of them changes
    first = root / next(iter(rec["sources_sha256"]))
    first.write_bytes(first.read_bytes() + b"\n")
    assert bench.recorded_traffic("llama3_8b_decode") is None
