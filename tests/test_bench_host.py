"""CPU tests of bench.py's host-side parts: the modelled floor uses the oracle's pinned
phase-aware cost model, the committed HBM counter summaries belong to the current gate/up
kernel source, and the bench refuses more than one GPU before touching any."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle.qstar import phased_step_time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_modelled_floor_is_the_oracle_cost_model():
    b = _bench()
    rng = np.random.default_rng(5)
    for _ in range(2000):
        m = int(rng.integers(0, 17))
        q = int(rng.integers(0, m + 1))
        S = float(rng.uniform(1e6, 6e7))
        B_P = float(rng.uniform(5e9, 7e10))
        B_H = float(rng.uniform(1e9, 3e11))
        assert b.phased_time(m, q, S, B_P, B_H) == pytest.approx(phased_step_time(m, q, S, B_P, B_H), rel=1e-12)


@pytest.mark.parametrize("workload", ["decode-L43-d4096-E256-top6", "decode-L40-d2048-E128-top8"])
def test_committed_counters_match_the_current_kernel(workload):
    """bench.py reports `traffic` only from counters taken on the current gate/up kernel
    source; the committed summaries must be those."""
    b = _bench()
    h = b.kernel_source_hash("ffn_gateup_rows_kernel")
    assert h is not None and len(h) == 16
    traffic = b.stored_traffic("ffn_gateup_rows_kernel", workload)
    assert traffic is not None and traffic > 1e7


def test_unknown_kernel_or_workload_has_no_counters():
    b = _bench()
    assert b.kernel_source_hash("no_such_kernel") is None
    assert b.stored_traffic("ffn_gateup_rows_kernel", "no-such-workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_trace_reuse_counts_experts_kept_from_the_step_before():
    b = _bench()
    # one layer, one stream, k = 2: step 1 keeps one of step 0's two experts, step 2 none
    tr = np.array([[[[1, 2]]], [[[2, 3]]], [[[4, 5]]]], dtype=np.int16)
    assert b.trace_reuse(tr) == pytest.approx(0.25)
    # the same expert set in another order counts as fully reused
    tr = np.array([[[[7, 9, 3]]], [[[3, 7, 9]]]], dtype=np.int16)
    assert b.trace_reuse(tr) == pytest.approx(1.0)


def test_profile_commands_run_committed_files_with_current_options():
    """Every rocprofv3 command written in profiles/ runs bench.py (a committed file) with
    options bench.py still accepts, so each summary can be re-made from the tree."""
    import glob
    import shlex
    b = _bench()
    seen = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        for line in open(path):
            if "rocprofv3 " not in line or " -- " not in line:
                continue
            prog = shlex.split(line.split(" -- ", 1)[1])
            assert prog[:2] == ["python3", "-u"] and prog[2] == "bench.py", (path, line)
            assert os.path.exists(os.path.join(ROOT, prog[2]))
            try:
                b.arg_parser().parse_args(prog[3:])
            except SystemExit:
                pytest.fail(f"{os.path.basename(path)}: bench.py no longer takes {' '.join(prog[3:])}")
            seen += 1
    assert seen >= 8
