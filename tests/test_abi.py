"""The C-ABI library loads and exports every entry point include/stepq.h
declares; argument checks that run before any launch (no GPU needed)."""
import re
from pathlib import Path

import numpy as np
import pytest

from quantized_recurrent_state_packed_amd import build_lib
from quantized_recurrent_state_packed_amd import stepq as S

HEADER = Path(__file__).resolve().parents[1] / "include" / "stepq.h"


@pytest.fixture(scope="module")
def lib():
    if not S.LIB_PATH.exists():
        build_lib.build()
    return S.lib()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(stepq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(S.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(5):
        assert S.stepq_status_string(st)
    assert S.stepq_status_string(99) == "unknown status"


def _desc(H=2, D=32, mode=0, bits=None, omega=None):
    bits = np.full(H if mode == 0 else H * D, 6, np.uint8) if bits is None else np.asarray(bits, np.uint8)
    omega = np.ones(H * D, np.float32) if omega is None else np.asarray(omega, np.float32)
    return (H, D, D, mode, bits, omega)


@pytest.mark.parametrize("bad,status", [
    (dict(H=0), S.STEPQ_ERR_INVALID_ARG),
    (dict(mode=2), S.STEPQ_ERR_INVALID_ARG),
    (dict(bits=[6, 5]), S.STEPQ_ERR_INVALID_ARG),
    (dict(bits=[6, 12]), S.STEPQ_ERR_INVALID_ARG),
    (dict(omega=np.r_[np.ones(63), 0.0]), S.STEPQ_ERR_INVALID_ARG),
    (dict(omega=np.r_[np.ones(63), np.nan]), S.STEPQ_ERR_INVALID_ARG),
    (dict(D=48), S.STEPQ_ERR_UNSUPPORTED),
])
def test_layout_validation_before_any_device_call(lib, bad, status):
    args = dict(H=2, D=32, mode=0)
    args.update({k: v for k, v in bad.items() if k in ("H", "D", "mode")})
    H, D, mode = args["H"], args["D"], args["mode"]
    bits = bad.get("bits")
    omega = bad.get("omega")
    if H >= 1 and omega is None:
        omega = np.ones(max(H, 1) * D, np.float32)
    with pytest.raises(S.StepqError) as e:
        S.stepq_layout_create(H, D, D, mode, np.full(max(H, 1), 6, np.uint8) if bits is None else bits,
                              np.ones(max(H, 1) * D, np.float32) if omega is None else omega, S.ROW_SCALES_REFIT)
    assert e.value.status == status


def test_unequal_key_value_dims_unsupported(lib):
    with pytest.raises(S.StepqError) as e:
        S.stepq_layout_create(1, 64, 32, 0, np.full(1, 6, np.uint8), np.ones(64, np.float32), S.ROW_SCALES_REFIT)
    assert e.value.status == S.STEPQ_ERR_UNSUPPORTED


def test_binding_defaults_to_calibrated_row_scales(lib):
    """The binding's default row-scale mode is the calibrated one, which needs
    row magnitudes: without them the call is rejected before any device call,
    so the per-step refit (ROW_SCALES_REFIT) is only ever chosen explicitly."""
    import inspect
    assert inspect.signature(S.stepq_layout_create).parameters["row_scale_mode"].default == S.ROW_SCALES_CALIBRATED
    assert inspect.signature(S.Layout).parameters["row_scale_mode"].default == S.ROW_SCALES_CALIBRATED
    with pytest.raises(S.StepqError) as e:
        S.stepq_layout_create(2, 32, 32, 0, np.full(2, 6, np.uint8), np.ones(64, np.float32))
    assert e.value.status == S.STEPQ_ERR_INVALID_ARG


def test_null_handle_paths(lib):
    assert S.stepq_slot_pool_bytes(None) == 0
    assert S.stepq_slot_scale_bytes(None) == 0
    S.stepq_layout_destroy(None)
    st = lib.stepq_decode_step(None, 1, None, 1, None, None, None, None, None, None, None, None, None)
    assert st == S.STEPQ_ERR_INVALID_ARG
    st = lib.stepq_pack(None, 1, None, 1, None, None, None, None)
    assert st == S.STEPQ_ERR_INVALID_ARG


@pytest.mark.parametrize("mode,mag", [
    (3, None),                                   # unknown row-scale mode
    (S.ROW_SCALES_CALIBRATED, None),             # calibrated mode needs magnitudes
    (S.ROW_SCALES_CALIBRATED, np.r_[np.ones(63), 0.0]),
    (S.ROW_SCALES_CALIBRATED, np.r_[np.ones(63), -1.0]),
    (S.ROW_SCALES_CALIBRATED, np.r_[np.ones(63), np.inf]),
])
def test_row_scale_mode_validation_before_any_device_call(lib, mode, mag):
    with pytest.raises(S.StepqError) as e:
        S.stepq_layout_create(2, 32, 32, 0, np.full(2, 6, np.uint8), np.ones(64, np.float32), mode, mag)
    assert e.value.status == S.STEPQ_ERR_INVALID_ARG


@pytest.mark.parametrize("gate_mode,bits", [
    (0, [6, 16]),                                # a pivot head
    (0, [6, 32]),                                # a binary32 head
    (1, [6] * 31 + [8] + [6] * 32),              # two widths inside one head
])
def test_uniform_tile_scale_needs_one_integer_width_per_head(lib, gate_mode, bits):
    with pytest.raises(S.StepqError) as e:
        S.stepq_layout_create(2, 32, 32, gate_mode, np.asarray(bits, np.uint8), np.ones(64, np.float32),
                              S.UNIFORM_TILE_SCALE)
    assert e.value.status == S.STEPQ_ERR_INVALID_ARG


@pytest.mark.parametrize("case", ["short_bits", "short_omega", "wide_bits", "short_magnitude"])
def test_binding_checks_host_array_lengths(lib, case):
    """The library reads H (per-head gate) or H*d_k widths and H*d_k weights
    from host arrays it cannot size; the binding rejects another length, and a
    width that does not fit the byte it is passed as, before the call."""
    H, D = 2, 32
    bits, omega, mode, rs, mag = np.full(H, 6), np.ones(H * D, np.float32), 0, S.ROW_SCALES_REFIT, None
    if case == "short_bits":
        mode = 1                                   # the per-key-channel gate needs H*D widths
    elif case == "short_omega":
        omega = np.ones(H * D - 1, np.float32)
    elif case == "wide_bits":
        bits = np.array([6, 264])                  # would wrap to 8 as a byte
    else:
        rs, mag = S.ROW_SCALES_CALIBRATED, np.ones(H, np.float32)
    with pytest.raises(S.StepqError, match="must fit in a byte" if case == "wide_bits" else "entries") as e:
        S.stepq_layout_create(H, D, D, mode, bits, omega, rs, mag)
    assert e.value.status == S.STEPQ_ERR_INVALID_ARG


def test_binding_rejects_host_tensors_before_the_library(lib, monkeypatch):
    """Tensor arguments of a known layout are checked before their pointers
    reach the library.  The shape is registered under the null handle, for
    which the library itself only returns a status."""
    import torch
    monkeypatch.setitem(S._layouts, None, (64, 2, 2, 1024, 256, 32))
    x = torch.zeros(2 * 64)
    slots = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(S.StepqError, match="slot_ids must be a device tensor") as e:
        S.stepq_decode_step(None, 1, slots, 1, x, x, x, x, x, x, x, x)
    assert e.value.status == S.STEPQ_ERR_INVALID_ARG
    S.set_argument_checks(False)
    try:   # unchecked, the null handle reaches the library, which rejects it
        with pytest.raises(S.StepqError) as e:
            S.stepq_decode_step(None, 1, slots, 1, x, x, x, x, x, x, x, x, stream=0)
        assert e.value.status == S.STEPQ_ERR_INVALID_ARG and "device tensor" not in str(e.value)
    finally:
        S.set_argument_checks(True)
