"""bench.py's command line on a CPU-only machine: more than one GPU is
refused with a message, before anything touches a GPU."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_one_call_is_refused_outside_the_fused_16bit_step():
    for extra in (["--separate-append"], ["--kv", "fp8"], ["--op", "rows"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--one-call", *extra],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, extra
        assert "--one-call" in r.stderr


def test_help_lists_the_workload_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for opt in ("--config", "--op", "--kv", "--reuse-blocks", "--separate-append", "--one-call"):
        assert opt in r.stdout


def test_probe_library_exports_the_measurement_helpers():
    """bench.py times launches with events from the probe library built beside
    libpagedkv (no GPU is needed to load it and look the symbols up)."""
    import ctypes
    from paged_kv_cache_119_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libpkvprobe.so not built")
    lib = ctypes.CDLL(PROBE_LIB)
    for name in ("pkvprobe_stream_read", "pkvprobe_event_create", "pkvprobe_event_record",
                 "pkvprobe_event_elapsed", "pkvprobe_event_destroy"):
        assert hasattr(lib, name), name
