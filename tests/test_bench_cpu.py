"""Host-side checks of bench.py's contract (no GPU): one GPU only, the peaks it reports against,
and the recorded byte counts tied to the kernel sources they were taken on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_peaks_are_the_published_figures():
    b = _bench()
    assert b.PEAK_BF16_TFLOPS == 2500.0
    assert b.PEAK_HBM_GBS == 8000.0
    # 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz lane operations, the 157.3 TFLOP/s fp32 vector peak
    # counted as two-flop FMAs
    assert abs(2 * b.PEAK_VALU_LANE_OPS / 1e12 - 157.3) < 0.1


def test_traffic_is_reported_only_for_the_recorded_sources():
    b = _bench()
    for kernel, (digest, fetch_kib, write_kib) in b.TRAFFIC.items():
        assert kernel in b.KERNEL_SOURCES
        assert fetch_kib > 0 and write_kib > 0
        got = b.traffic_bytes(kernel)
        if b.source_digest(b.KERNEL_SOURCES[kernel]) == digest:
            assert got == int(fetch_kib * 1024 * b.FETCH_SCALE + write_kib * 1024 * b.WRITE_SCALE)
        else:
            assert got is None
    assert b.traffic_bytes("no_such_kernel") is None


def test_valu_counts_leave_out_the_matrix_instructions():
    # SQ_INSTS_VALU counts MFMA issues too; every record carries both counts, MFMA below VALU
    b = _bench()
    for name, (digest, valu, mfma) in b.VALU_INSTS.items():
        assert 0 < mfma < valu, name
