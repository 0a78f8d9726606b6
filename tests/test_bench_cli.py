"""Host-side checks of bench.py (no GPU): it refuses more than one GPU
before touching a device, and reports the counter-measured HBM traffic only
for the kernel source the counters were taken on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_traffic_only_for_the_profiled_source():
    import bench
    sha = bench.source_sha("gemv.hip", "ql_device.h")
    key = "gemv_w4_chunked_kernel<64,1,8,0,0>"
    t = bench.traffic_for(key, sha)
    if t is not None:  # counters current for this source: close to the algorithmic bytes
        assert 0.99 < t / 174895104 < 1.05
    assert bench.traffic_for(key, "0" * 16) is None
    assert bench.traffic_for("no_such_kernel", sha) is None


def test_lds_probe_host_side():
    """The LDS probe's bindings load and its host-side arithmetic and argument
    checks hold without a device (no launch is made)."""
    import ctypes
    import bench
    L = bench.probe_lib()
    assert L.ql_probe_lds_blocks() == 256
    assert L.ql_probe_lds_bytes(0, 4096) == 8 * 4096 * 8 * 1024
    assert L.ql_probe_lds_bytes(3, 4096) == 8 * 4096 * 8 * 512
    assert L.ql_probe_lds(0, 4096, None, None, None) == 1          # no buffers
    assert L.ql_probe_lds(0, 0, ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 1  # no iterations
    assert [m for m, _ in bench.LDS_PROBE_MODES] == [0, 1, 2, 3]
