"""Host logic of bench.py that needs no GPU: the one-GPU contract and the traffic record's source digest."""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def _copy_sources(dst):
    os.makedirs(os.path.join(dst, "hierarchical_memory_amd", "csrc"))
    for f in ("hs_kernels.hip", "hs_internal.h"):
        shutil.copy(os.path.join(ROOT, "hierarchical_memory_amd", "csrc", f),
                    os.path.join(dst, "hierarchical_memory_amd", "csrc", f))
    return os.path.join(dst, "hierarchical_memory_amd", "csrc", "hs_kernels.hip")


def _digest_of(root):
    saved = bench.ROOT
    bench.ROOT = root
    try:
        return bench.kernel_source_digest()
    finally:
        bench.ROOT = saved


def test_source_digest_ignores_comments_only(tmp_path):
    """A comment or blank-line edit keeps the digest (the code is the same); a code edit changes it."""
    base = _digest_of(ROOT)
    src = _copy_sources(str(tmp_path / "a"))
    assert _digest_of(str(tmp_path / "a")) == base
    with open(src, "a") as fh:
        fh.write("\n// a trailing comment\n\n/* and a block\n   comment */\n")
    assert _digest_of(str(tmp_path / "a")) == base
    src_b = _copy_sources(str(tmp_path / "b"))
    with open(src_b) as fh:
        text = fh.read()
    with open(src_b, "w") as fh:
        fh.write(text.replace("constexpr int kCommitUnroll = 2;", "constexpr int kCommitUnroll = 3;", 1))
    assert _digest_of(str(tmp_path / "b")) != base


def test_traffic_record_is_used_only_for_its_sources_and_workload(tmp_path):
    """The committed PMC record gives bytes for its own workload on the current sources and None otherwise."""
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as fh:
        rec = json.load(fh)
    wl = rec["workload"]
    if rec["kernel_source_digest"] != bench.kernel_source_digest():
        pytest.skip("the committed traffic record was taken on other kernel code")
    t = bench.measured_traffic(wl, "resolve_plan")
    assert t is not None and t > 0
    assert bench.measured_traffic("another_workload", "resolve_plan") is None
    assert bench.measured_traffic(wl, "no_such_kernel") is None
    f = bench.traffic_fields(wl, "resolve_plan", 1.0e6)
    assert f["traffic"] == t and f["traffic_ratio"] == pytest.approx(t / 1.0e6) and f["traffic_source"]
