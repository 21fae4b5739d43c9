"""Host-side checks of the benchmark tooling (no GPU)."""

import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLOOR_LIB = os.path.join(ROOT, "grouped_query_attention_prefill_amd", "libgqa_readfloor.so")


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: the request is refused before torch or the GPU is touched
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_lists_the_traffic_runs():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--traffic-commands", "/tmp/out"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    lines = r.stdout.splitlines()
    assert lines and all(ln.startswith("rocprofv3 --pmc ") for ln in lines)
    # a FETCH_SIZE and a WRITE_SIZE run for the copy calibration and for every row
    assert sum("FETCH_SIZE" in ln for ln in lines) == sum("WRITE_SIZE" in ln for ln in lines) == len(lines) // 2


@pytest.mark.skipif(not os.path.exists(FLOOR_LIB), reason="libgqa_readfloor.so not built")
def test_read_floor_library_exports_and_checks_arguments():
    lib = ctypes.CDLL(FLOOR_LIB)
    lib.gqa_read_floor.restype = ctypes.c_int
    lib.gqa_read_floor.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    # null buffers and sizes that are not whole 16-byte words are refused before any launch
    assert lib.gqa_read_floor(None, 16, None, None) == 1
    assert lib.gqa_read_floor(ctypes.c_void_p(16), 15, ctypes.c_void_p(16), None) == 1
