"""Host-side parts of bench.py that need no GPU: the one-GPU refusal, and the
rule that a committed HBM-traffic record is reported only while the kernel
it was taken on (its source, the headers it includes and the source's extra
compile flags) is the one being built."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from softmax_sink_amd import build  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _records():
    return json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))


def test_every_record_names_existing_sources():
    for workload, rec in _records().items():
        assert rec["kernel"].endswith("_kernel"), workload
        for name in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, "softmax_sink_amd", "csrc", name)), name
        assert rec["hbm_bytes_per_launch"] > 0


def test_record_follows_source_and_flags(monkeypatch, tmp_path):
    rec = dict(_records()["train_varlen"])
    live = bench.traffic_record("train_varlen", rec["kernel"])
    if live is None:
        pytest.skip("the committed train_varlen record predates the current kernel")
    assert live == rec["hbm_bytes_per_launch"]
    # another kernel name for the workload: no record
    assert bench.traffic_record("train_varlen", "bwd_dq_kernel") is None
    # other compile flags for the kernel's source: no record
    flags = dict(build.SOURCE_FLAGS)
    flags[rec["sources"][0]] = flags.get(rec["sources"][0], []) + ["-mllvm", "-some-other-flag"]
    monkeypatch.setattr(build, "SOURCE_FLAGS", flags)
    assert bench.traffic_record("train_varlen", rec["kernel"]) is None
    monkeypatch.undo()
    # an edited source: no record (a copy of the tree's csrc with one byte added)
    csrc = tmp_path / "softmax_sink_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in rec["sources"]:
        data = open(os.path.join(ROOT, "softmax_sink_amd", "csrc", name), "rb").read()
        (csrc / name).write_bytes(data + (b" " if name == rec["sources"][0] else b""))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"train_varlen": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_record("train_varlen", rec["kernel"]) is None
