"""Host logic of bench.py that runs without a GPU: the refusal of more than one GPU, and
the rule that HBM traffic comes from a committed counter record only while that record
names the current kernel build (source and hipcc flags)."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "exactly one GPU" in json.loads(res.stdout.strip().splitlines()[-1])["error"]


def test_digest_covers_source_and_flags(monkeypatch):
    from gqa_causal_prefill_amd import build

    d = bench.source_digest()
    assert len(d) == 16 and int(d, 16) >= 0
    monkeypatch.setattr(build, "HIPCC_FLAGS", build.HIPCC_FLAGS + ["-DANOTHER_BUILD"])
    assert bench.source_digest() != d


def test_traffic_only_for_the_build_it_was_taken_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_longkv_4096x32768.json")
    with open(path) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "source_digest", lambda: rec["kernel_build_sha256_16"])
    assert bench.load_traffic("longkv_4096x32768") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.load_traffic("longkv_4096x32768") is None
    assert bench.load_traffic("no_such_workload") is None



def test_counter_record_carries_mfma_busy_for_its_build(monkeypatch):
    """The counter record is gated like the traffic: the MFMA busy share (and the traffic
    the HBM rate is computed from) come only from a record of the current build."""
    path = os.path.join(ROOT, "profiles", "traffic_longkv_4096x32768.json")
    with open(path) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "source_digest", lambda: rec["kernel_build_sha256_16"])
    got = bench.load_counters("longkv_4096x32768")
    assert got is not None and got.get("mfma_busy") == rec.get("mfma_busy")
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 16)
    assert bench.load_counters("longkv_4096x32768") is None
