"""Host-side checks of the benchmark script: the one-GPU guard and the committed
counter summaries it reads its traffic and MFMA-busy figures from."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("path,key", [
    (bench.TRAFFIC_PROFILE, "traffic_bytes_per_launch"),
    (bench.MFMA_PROFILE, "headline_forward_mfma_busy_pct"),
    (bench.MERGE_PROFILE, "merge_traffic_bytes_per_launch"),
])
def test_counter_summaries_carry_their_figure_and_source_digest(path, key):
    with open(path) as f:
        text = f.read()
    assert f"\n{key}:" in text
    assert "kernel_source_sha256:" in text
    assert "rocprofv3 --pmc" in text          # the command that produced it


def test_counter_figures_are_plausible_or_withheld():
    t = bench.measured_traffic()
    if t is not None:                          # withheld (None) once the kernel changed
        algorithmic = 16384 * 16 * (4 * 128 + 4) + 16384 * 16 * 4 * 128
        assert algorithmic <= t <= 10 * algorithmic
    m = bench.measured_mfma_busy()
    if m is not None:
        assert 0.0 < m <= 100.0
    mt = bench.measured_merge_traffic()
    if mt is not None:                         # 8 partials + result, O bf16 and LSE fp32
        algorithmic = 9 * 8192 * 32 * (2 * 128 + 4)
        assert algorithmic <= mt <= 1.05 * algorithmic


def test_digest_follows_the_kernel_sources(tmp_path, monkeypatch):
    d0 = bench.kernel_digest()
    src = tmp_path / "k.hip"
    src.write_text("// a different kernel\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", (str(src),))
    monkeypatch.setattr(bench, "ROOT", "/")
    assert bench.kernel_digest() != d0
    assert bench.measured_traffic() is None
    assert bench.measured_mfma_busy() is None


def test_per_workload_counters_cover_every_reference_workload():
    with open(bench.COUNTERS_PROFILE) as f:
        text = f.read()
    assert "rocprofv3 --pmc" in text and "bench.py --counter-pass" in text
    c = bench.measured_workload_counters()
    if not c:                                  # withheld once the kernels changed
        return
    from block_sparse_flash_csr_amd import workloads as W
    names = [W.WORKLOADS[i](with_inputs=False).name for i in (1, 2, 3, 4, 5)]
    # forward and merge entries are withheld separately, each once its kernel changed
    expect = (names if any(n in c for n in names) else []) + [n for n in [names[-1] + "_merge"] if n in c]
    for name in expect:
        assert name in c, name
        assert 0.0 <= c[name]["mfma_busy_pct"] <= 100.0
        assert 0.0 <= c[name]["l2_hit_pct"] <= 100.0
        assert c[name]["hbm_bytes_per_launch"] > 0


def test_per_workload_counters_are_withheld_when_the_kernel_changes(monkeypatch):
    monkeypatch.setattr(bench, "kernel_digest", lambda: "0" * 64)
    c = bench.measured_workload_counters()
    assert all(name.endswith("_merge") for name in c)
