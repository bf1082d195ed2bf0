"""Host-side parts of the benchmark: the one-GPU contract and the measurement helpers that need
no GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_record_is_tied_to_the_kernel_sources():
    # a stored counter summary is reported only while its kernel sources are unchanged
    assert bench.kernel_source_sha("prefill.hip") != bench.kernel_source_sha("gemv_mx.hip", "mx_common.hpp")
    assert bench.stored_traffic("no_such_kernel", ["prefill.hip"], 1.0) is None
    # the prefill record against another kernel's sources: a hash mismatch, so nothing reported
    assert bench.stored_traffic("prefill_kernel", ["gemv_mx.hip", "mx_common.hpp"], 1.0) is None
