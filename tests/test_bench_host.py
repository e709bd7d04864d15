"""Host-side logic of bench.py that runs without a GPU: the one-GPU guard of the command
line, and the staleness check that keeps a counter-measured traffic figure out of the
JSON line once the kernel sources it was measured on have changed."""
import hashlib
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def _tree(tmp_path, sources, profile_text):
    csrc = tmp_path / "gated_delta_rule_18_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name, body in sources.items():
        (csrc / name).write_bytes(body)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "k.txt").write_text(profile_text)
    return csrc


def test_measured_traffic_follows_the_source_hash(tmp_path):
    bench = _bench_module()
    sources = {"a.hip": b"kernel a\n", "b.h": b"helpers\n"}
    h = hashlib.sha256()
    for name in ("a.hip", "b.h"):
        h.update(sources[name])
    text = (f"summary\nkernel source sha256[:16] (a.hip + b.h): {h.hexdigest()[:16]}\n"
            "traffic_bytes: 8307000000\nsnapshots_traffic_bytes: 9078000000\n")
    csrc = _tree(tmp_path, sources, text)
    bench.ROOT = str(tmp_path)
    assert bench.measured_traffic("k.txt", ["a.hip", "b.h"]) == 8307000000
    assert bench.measured_traffic("k.txt", ["a.hip", "b.h"], key="snapshots_traffic_bytes") == 9078000000
    # a key the summary does not hold, a missing summary, the sources hashed in another order
    assert bench.measured_traffic("k.txt", ["a.hip", "b.h"], key="gated_traffic_bytes") is None
    assert bench.measured_traffic("missing.txt", ["a.hip", "b.h"]) is None
    assert bench.measured_traffic("k.txt", ["b.h", "a.hip"]) is None
    # a kernel source edited after the counters were taken
    (csrc / "a.hip").write_bytes(b"kernel a, changed\n")
    assert bench.measured_traffic("k.txt", ["a.hip", "b.h"]) is None
