"""Host-side parts of the benchmark: byte and flop accounting, the one-GPU rule."""
import dataclasses
import subprocess
import sys
from pathlib import Path

import pytest

import bench  # noqa: E402
from quantized_recurrent_state_packed_amd import workloads as W

ROOT = Path(__file__).resolve().parents[1]


def test_serving_step_bytes_match_the_byte_model():
    """Serving shape (B=512, H=48, 128x128, 6.0-bit budget with one FP16 pivot
    head), row scales refitted every step: 679.15 MB per step -- codes
    2 x 302 MB, binary16 row and column scales 2 x 6.2 MB, q/k/v/o 50.3 MB,
    beta/gate/slot 0.2 MB.  Calibrated row scales are layout constants, so only
    the column half of the scales moves: 12.3 MB less."""
    lay = W.make_layout(3)
    refit = bench.step_bytes(dataclasses.replace(lay, row_mode=0))
    assert refit["total"] * 512 == 679_151_616
    assert refit["codes"] * 512 == 2 * 512 * 48 * 128 * 128 * 6 // 8
    cal = bench.step_bytes(lay)
    assert cal["total"] * 512 == 679_151_616 - 512 * 47 * 2 * 2 * 128


def test_step_flops_counts_integer_and_float_rows():
    lay = W.make_layout(3)
    n_piv = int((lay.unit_bits == 16).sum())
    for mode, l in (("calibrated", lay), ("refit", dataclasses.replace(lay, row_mode=0))):
        expect = ((48 - n_piv) * 128 * 128 * bench.FLOPS_INT_ELEM[mode]
                  + n_piv * 128 * 128 * bench.FLOPS_FLOAT_ELEM)
        assert bench.step_flops(l) == expect


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workloads_are_chosen_by_name_or_index():
    for i, c in W.CONFIGS.items():
        assert W.workload_id(c["name"]) == i and W.workload_id(str(i)) == i
    with pytest.raises(ValueError, match="kimi-kda-b64"):
        W.workload_id("kda")
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--workload", "no-such-workload"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "--workload" in r.stderr


def test_stream_probe_library_loads_and_rejects_bad_arguments():
    """The benchmark's bandwidth probe is built in bench_probe/, outside the
    library package; argument checks return hipErrorInvalidValue (1) before
    any device call."""
    import ctypes
    from pathlib import Path
    lib = ctypes.CDLL(str(Path(__file__).resolve().parents[1] / "bench_probe" / "libstreamprobe.so"))
    f = lib.stepq_stream_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_size_t, ctypes.c_int] + [ctypes.POINTER(ctypes.c_double)] * 3
    x = ctypes.c_double()
    assert f(0, 1, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == 1          # too small
    assert f((64 << 20) + 8, 1, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == 1   # not a multiple of 16
    assert f(64 << 20, 0, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == 1     # no repetitions
    assert f(64 << 20, 1, None, ctypes.byref(x), ctypes.byref(x)) == 1                # missing output
