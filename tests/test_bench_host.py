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
