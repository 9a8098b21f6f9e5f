"""bench.py's host logic without a GPU: the one-GPU contract, the guards on workload/option combinations, and
the counters file that fills roofline.traffic only for the kernel sources it was taken with."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=120, env={**os.environ, **env})
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("args", [["--workload", "decode_T1", "--with-conv1d"],
                                  ["--workload", "swimba_decode_T8", "--with-conv1d"],
                                  ["--workload", "swimba_decode_T1", "--backward"],
                                  ["--workload", "tiny_f32", "--backward"]])
def test_option_workload_combinations_without_a_kernel_are_rejected(args):
    r = _run(*args)
    assert r.returncode == 2 and r.stdout == "" and "bench.py:" in r.stderr, r.stderr


def test_counters_file_is_used_only_for_its_kernel_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    good = tmp_path / "counters_in_proj_demo.txt"
    good.write_text(f"# comment = ignored\nsource_sha256 = {h}\ntraffic_bytes_per_launch = 12345\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "counters_in_proj_{workload}.txt"))
    assert bench.measured_traffic("demo") == 12345.0
    good.write_text("source_sha256 = 0000000000000000\ntraffic_bytes_per_launch = 12345\n")
    assert bench.measured_traffic("demo") is None          # taken with other kernel sources
    assert bench.measured_traffic("absent") is None        # no counters for this workload
    good.write_text(f"source_sha256 = {h}\n")
    assert bench.measured_traffic("demo") is None          # no figure in the file


def test_committed_counters_match_the_current_sources():
    """The skewed block's committed counters were taken with the kernel sources in the tree, so the benchmark
    line reports roofline.traffic."""
    assert bench.measured_traffic("skewed") is not None
