"""bench.py's host-only modes (no GPU): the one-GPU guard and the offline
planner report."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_planner_report_lines():
    r = _run("--planner")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [json.loads(x) for x in r.stdout.strip().splitlines()]
    assert [x["planner"] for x in lines] == ["planned-16k", "ouro2.6b-32k"]
    for x in lines:
        k = x["kinds"]
        assert k["q4"] + k["q2"] + k["reuse"] == x["cells"]
        assert x["damage"] <= x["damage_budget"] * (1 + 1e-12)
        assert x["storage_units"] <= x["storage_budget_units"]


def test_default_extra_workloads_exist(monkeypatch):
    """Every workload the default run times beside the primary one is a known
    workload (a misspelt name would only fail on the GPU, after the primary
    line's timing)."""
    monkeypatch.syspath_prepend(ROOT)
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    import bench
    from loop_aware_quantized_amd import inputs as wl
    names = [x for x in bench.parse().extra.split(",") if x]
    assert names, "the default run times extra workloads"
    for n in names:
        assert n in wl.WORKLOADS or n in wl.VQ_WORKLOADS, n
    # a swept workload's entry is its own plan tau, which must be a sweep point
    for n in names:
        w = wl.WORKLOADS.get(n)
        if w is not None and w.tau_sweep:
            assert float(w.taus[0]) in [float(t) for t in w.tau_sweep]
