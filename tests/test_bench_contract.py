"""bench.py's output contract: one JSON line with the fields the benchmark
driver reads, and the refusal of more than one GPU (this path is one rank on
one GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_share_uses_every_cpu_of_the_affinity_mask(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    affinity = len(os.sched_getaffinity(0))
    quota = bench.cgroup_cpus()
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    threads, counts = bench.cpu_share()
    assert threads == (affinity if quota is None else min(affinity, quota))
    assert counts["affinity_cpus"] == affinity and counts["os_cpu_count"] == os.cpu_count()
    assert counts["omp_num_threads"] is None
    # an explicit OMP_NUM_THREADS caps it; nothing else does (no fixed ceiling)
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.cpu_share()[0] == min(3, threads)
    monkeypatch.setenv("OMP_NUM_THREADS", "100000")
    assert bench.cpu_share()[0] == threads


def test_defaults_are_the_headline_workload_and_the_one_pass_pipeline(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS
    assert bench.DEFAULT_WORKLOAD == "llama3_8b"
    # the largest shard among the workloads
    shard = {k: sum(sum(g.numels) for g in w.groups) // w.n_d for k, w in WORKLOADS.items()}
    assert max(shard, key=shard.get) == "llama3_8b"
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert args.workload == "llama3_8b" and args.pipeline == "optimistic"
    assert args.cpu_single == 1 << 28


@pytest.mark.gpu
@pytest.mark.parametrize("args", [["--workload", "tiny", "--cpu-sample", "65536"],
                                  ["--workload", "13b_nd8", "--pipeline", "optimistic", "--cpu-sample", "0"]])
def test_json_line_has_the_contract_fields(args):
    print(f"bench {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--quiet", *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)]:
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["vs_baseline"] is None and d["higher_is_better"] is True
    assert "workload" in d["config"] and "model" not in d["config"]
    assert d["config"]["arena"].split(":")[0] in ("whole", "sized", "none")
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert rf["traffic"] is None or rf["traffic"] > 0
    cc = d["copy_ceiling"]   # a plain copy in the step's arena; none when the arena has no room (tiny)
    if "13b_nd8" in args:
        assert cc["gbps"] > 1000 and abs(cc["achieved_frac"] - rf["achieved"] / cc["gbps"]) < 1e-12
    else:
        assert cc is None
    cpu = d["cpu_baseline"]
    if "--cpu-sample" in args and args[args.index("--cpu-sample") + 1] != "0":
        assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["unit"] == "params/s"
        assert cpu["cores"] <= cpu["affinity_cpus"] and cpu["single_thread_value"] > 0
    else:
        assert cpu is None
