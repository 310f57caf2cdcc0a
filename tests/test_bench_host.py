"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard and
the rule that counter-measured HBM bytes are reported only for unchanged
kernel sources."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU path")
def test_without_a_gpu_it_exits_before_any_work():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "GPU" in r.stderr
    assert r.stdout == ""


def _fake_tree(tmp_path, sources: dict, recorded: dict, kernels: dict):
    csrc = tmp_path / "delayed_scaling_linear_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name, text in sources.items():
        (csrc / name).write_text(text)
    (tmp_path / "profiles").mkdir()
    rec = {"source_sha256": recorded, "kernels": kernels}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    return str(tmp_path)


def _sha(text: str) -> str:
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def test_traffic_is_reported_only_while_every_source_is_unchanged(tmp_path):
    src = {"a.hip": "kernel a", "b.h": "shared header", "c.hip": "kernel c, edited"}
    recorded = {"a.hip": _sha("kernel a"), "b.h": _sha("shared header"),
                "c.hip": _sha("kernel c")}                       # c changed since
    kernels = {"ka": {"sources": ["a.hip", "b.h"], "bytes": 10},
               "kc": {"sources": ["c.hip", "b.h"], "bytes": 20},
               "kn": {"sources": [], "bytes": 30},                 # names no source
               "km": {"sources": ["missing.hip"], "bytes": 40}}    # source gone
    root = _fake_tree(tmp_path, src, recorded, kernels)
    got = bench.traffic_record(root)
    assert set(got) == {"ka"}
    assert got["ka"]["bytes"] == 10


def test_no_record_means_no_traffic(tmp_path):
    assert bench.traffic_record(str(tmp_path)) is None


def test_the_committed_record_matches_the_committed_sources():
    """profiles/hbm_traffic.json names the sources it was measured on; every
    kernel it lists must name sources that exist."""
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    csrc = os.path.join(ROOT, "delayed_scaling_linear_amd", "csrc")
    for name, k in rec["kernels"].items():
        assert k["sources"], name
        for s in k["sources"]:
            assert os.path.exists(os.path.join(csrc, s)), (name, s)
