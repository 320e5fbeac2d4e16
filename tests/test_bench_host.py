"""Host-side checks of bench.py that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stdout


def test_every_workload_names_its_profiles_and_sources():
    sys.path.insert(0, ROOT)
    import bench
    for w, (stats_name, traffic_name, frag, label) in bench.WORKLOADS.items():
        assert w in bench.WORKLOAD_TITLES
        assert w in bench.KERNEL_SOURCES
        for f in bench.KERNEL_SOURCES[w]:
            assert os.path.exists(os.path.join(ROOT, "prompt_token_importance_amd", "csrc", f)), f
        cmds = bench.profile_commands(w, "out")
        assert set(cmds) == {"trace", "FETCH_SIZE", "WRITE_SIZE"}
        assert all(c.startswith("rocprofv3 ") and " -- python3 bench.py " in c for c in cmds.values())
        assert len(bench.source_hash(w)) == 16


def test_cpu_baselines_run_on_a_small_layer():
    """The oracle legs of the bench (all cores and one) on small inputs."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    ly = synth.gaussian_layer(3, L=2048, W=32, d_k=64, H_q=8, H_kv=2, n_spans=2, span_len=64)
    for sel in ({"kind": "cluster", "P": 16, "theta": 2e-3, "r": 3, "budget": 100},
                {"kind": "pool", "pool_k": 7, "budget": 100}):
        out = bench.cpu_baseline_softmax(ly, sel, min_seconds=0.0, max_reps=1)
        assert out["value"] > 0 and out["one_core_value"] > 0 and 1 <= out["cores"] <= 2
        assert out["kind"] == "oracle" and out["cpu_model"]
    layers = [synth.cross_layer(l, L=1024, n_spans=2, span_len=64) for l in range(2)]
    out = bench.cpu_baseline_cross(layers, 200)
    assert out["value"] > 0 and out["cores"] >= 1
