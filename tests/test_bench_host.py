"""Host logic of bench.py, no GPU: the one-GPU guard, and the rule that a
committed rocprofv3 counter figure is used only while the kernel sources it
was taken from are unchanged."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert not r.stdout.lstrip().startswith("{"), "no bench line"


def test_counter_figures_follow_the_source_digest(tmp_path):
    bench = _bench()
    digest = bench._source_digest(bench.GEMM_SOURCES)
    assert len(digest) == 16 and digest == bench._source_digest(bench.GEMM_SOURCES)
    assert digest != bench._source_digest(bench.RQ_SOURCES)
    table = {"gemm_kernel|x": {"source_digest": digest, "bytes_per_launch": 1234},
             "gemm_kernel|stale": {"source_digest": "0" * 16, "bytes_per_launch": 99}}
    path = tmp_path / "hbm_traffic.json"
    path.write_text(json.dumps(table))
    bench.PROFILE_COUNTERS = str(path)
    assert bench._traffic("gemm_kernel|x", bench.GEMM_SOURCES) == 1234
    assert bench._traffic("gemm_kernel|x", bench.RQ_SOURCES) is None       # other sources
    assert bench._traffic("gemm_kernel|stale", bench.GEMM_SOURCES) is None  # taken before a change
    assert bench._traffic("gemm_kernel|absent", bench.GEMM_SOURCES) is None
    path.write_text("not json")
    assert bench._traffic("gemm_kernel|x", bench.GEMM_SOURCES) is None
    bench.PROFILE_COUNTERS = str(tmp_path / "missing.json")
    assert bench._traffic("gemm_kernel|x", bench.GEMM_SOURCES) is None


def test_committed_counter_table_is_well_formed():
    """Every entry of the committed summary names its kernel, workload, digest
    and per-launch bytes, with the copy-kernel scale factors it was derived with."""
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        table = json.load(f)
    assert table
    for key, rec in table.items():
        for field in ("kernel", "workload", "source_digest", "fetch_size_kib_per_launch",
                      "write_size_kib_per_launch", "fetch_scale", "write_scale", "bytes_per_launch",
                      "algorithmic_bytes_per_launch"):
            assert field in rec, (key, field)
        kib = rec["fetch_size_kib_per_launch"] * rec["fetch_scale"] + rec["write_size_kib_per_launch"] * \
            rec["write_scale"]
        assert abs(kib * 1024 - rec["bytes_per_launch"]) <= 1024, key
        assert rec["bytes_per_launch"] >= 0.9 * rec["algorithmic_bytes_per_launch"], key
