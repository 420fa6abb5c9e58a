"""The benchmark's contract that holds without a GPU: one GPU only, known
workload names, and the committed traffic records it reads."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_exits(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_workload_cases_build_on_the_host():
    # one workload of each kind (GQA, split, MQA, MLA), built on the host
    for w in ["gqa_b64_hm", "gqa_b1_split_hm", "mqa_b64_8k_hm", "mla_b16_320"]:
        c = bench.make_case(w)
        assert c.kv_layout == (1 if w.endswith("_hm") else 0) or c.mla
    with pytest.raises(SystemExit):
        bench.make_case("no_such_workload")


@pytest.mark.parametrize("name", ["gqa_b64_hm", "mla_b16"])
def test_committed_traffic_records(name):
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    t = json.load(open(path))
    # FETCH_SIZE scaled by the copy kernel's reading covers the algorithmic
    # bytes, and the kernel re-reads nothing
    assert 1.0 <= t["fetch_over_algorithmic"] < 1.02
    assert t["bytes_per_launch"] == pytest.approx(t["fetch_bytes"] + t["write_bytes"], rel=1e-6)
    assert t["command"] and t["source_files"]


def test_cpu_baseline_times_one_thread_and_all_threads():
    """The oracle baseline reports the all-thread and the one-thread rate
    (each a median of 3 runs), the thread count and the host's CPU model."""
    from decode_attention_paged_02_amd import workloads as W
    r = bench.cpu_baseline(W.tiny_gqa(), budget_s=0.3)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] >= 1 and r["one_thread"]["value"] > 0
    assert "median of 3" in r["sample"]
    assert r["host"]["cpu_model"] and r["host"]["nproc"] >= 1
