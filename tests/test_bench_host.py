"""Host-side checks of the benchmark's contract and the workload table (CPU only).

bench.py must refuse more than one GPU with a JSON message before touching
torch, take the committed HBM byte counts only while the kernel sources they
were measured on are unchanged, and name every workload it can run.
"""
import json
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                         capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert res.returncode == 2
    line = res.stdout.strip().splitlines()[-1]
    rec = json.loads(line)
    assert rec["n_gpus"] == n and "one GPU" in rec["error"]


def test_measured_traffic_follows_the_kernel_source_hash(tmp_path, monkeypatch):
    bench = _bench()
    name = "unit-test-workload"
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / f"qgemm_traffic_{name}.json").write_text(
        json.dumps({"kernel_source_hash": "0123456789abcdef", "bytes_per_launch": 12345}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(name, "0123456789abcdef") == 12345
    assert bench.measured_traffic(name, "fedcba9876543210") is None   # kernels changed since the counters
    assert bench.measured_traffic("no-such-workload", "0123456789abcdef") is None


def test_committed_traffic_records_name_a_known_workload():
    prof = os.path.join(ROOT, "profiles")
    for f in os.listdir(prof):
        if f.startswith("qgemm_traffic_") and f.endswith(".json"):
            name = f[len("qgemm_traffic_"):-len(".json")]
            assert name in synth.WORKLOADS
            rec = json.load(open(os.path.join(prof, f)))
            assert rec["workload"] == name
            assert len(rec["kernel_source_hash"]) == 16 and rec["bytes_per_launch"] > 0


def test_workloads_by_name_and_position():
    names = list(synth.WORKLOADS)
    assert names == [synth.TINY, synth.LLAMA2_7B_PREFILL, synth.LLAMA2_7B_DECODE,
                     synth.LLAMA3_8B_W3A3, synth.LLAMA2_70B_PREFILL]
    for i, name in enumerate(names, 1):
        w = synth.workload(name)
        assert w.name == name
        assert synth.workload(i) is w and synth.workload(str(i)) is w and synth.workload(w) is w
    for bad in (0, 6, "7", "llama", ""):
        with pytest.raises(KeyError):
            synth.workload(bad)


def test_workload_shapes():
    w = synth.WORKLOADS[synth.LLAMA2_7B_PREFILL]
    assert (w.D, w.F, w.r, w.n, w.bits) == (4096, 11008, 32, 2048, 4)
    shapes = {l.name: (l.N, l.K) for l in synth.layer_linears(w)}
    assert shapes == {"qkv": (12288, 4096), "o": (4096, 4096), "gate_up": (22016, 4096), "down": (4096, 11008)}
    w = synth.WORKLOADS[synth.LLAMA3_8B_W3A3]
    shapes = {l.name: (l.N, l.K) for l in synth.layer_linears(w)}
    assert shapes == {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}
    # the decode workload draws the prefill workload's inputs
    assert synth.WORKLOADS[synth.LLAMA2_7B_DECODE].seed_id == synth.WORKLOADS[synth.LLAMA2_7B_PREFILL].seed_id
