"""Thin Python binding of libstepq.so (include/stepq.h), same names as the C ABI.

Argument marshalling only: torch tensors (device memory) become raw pointers,
torch streams become hipStream_t handles, status codes become exceptions.
Tensor arguments are checked against the sizes the call implies before the
library sees their pointers (StepqError with STEPQ_ERR_INVALID_ARG).
Every step of the path runs in the library's HIP kernels; there is no
fallback, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

# STEPQ_LIBRARY names another build of libstepq.so to load instead (the host
# sanitizer test loads an instrumented build of the host side).
LIB_PATH = Path(os.environ.get("STEPQ_LIBRARY", Path(__file__).resolve().parent / "libstepq.so"))

STEPQ_OK = 0
STEPQ_ERR_INVALID_ARG = 1
STEPQ_ERR_UNSUPPORTED = 2
STEPQ_ERR_HIP = 3
STEPQ_ERR_NO_MEMORY = 4

EXPORTED = ("stepq_layout_create", "stepq_layout_destroy", "stepq_slot_pool_bytes",
            "stepq_slot_scale_bytes", "stepq_pack", "stepq_unpack", "stepq_decode_step", "stepq_readout",
            "stepq_status_string")


class StepqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        msg = f"{where}: {stepq_status_string(status)} (status {status})"
        super().__init__(f"{msg}: {detail}" if detail else msg)
        self.status = status


class stepq_layout_desc(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("unit_bits", ctypes.c_void_p),
                ("row_impact", ctypes.c_void_p), ("row_scale_mode", ctypes.c_int32),
                ("row_magnitude", ctypes.c_void_p)]


ROW_SCALES_REFIT = 0
ROW_SCALES_CALIBRATED = 1
UNIFORM_TILE_SCALE = 2          # comparison baseline: one absmax scale per tile


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = ctypes.CDLL(str(LIB_PATH))
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.stepq_layout_create.restype = ctypes.c_int
        L.stepq_layout_create.argtypes = [ctypes.POINTER(stepq_layout_desc), ctypes.POINTER(P)]
        L.stepq_layout_destroy.restype = None
        L.stepq_layout_destroy.argtypes = [P]
        L.stepq_slot_pool_bytes.restype = sz
        L.stepq_slot_pool_bytes.argtypes = [P]
        L.stepq_slot_scale_bytes.restype = sz
        L.stepq_slot_scale_bytes.argtypes = [P]
        L.stepq_pack.restype = ctypes.c_int
        L.stepq_pack.argtypes = [P, i32, P, i32, P, P, P, P]
        L.stepq_unpack.restype = ctypes.c_int
        L.stepq_unpack.argtypes = [P, i32, P, i32, P, P, P, P]
        L.stepq_decode_step.restype = ctypes.c_int
        L.stepq_decode_step.argtypes = [P, i32, P, i32, P, P, P, P, P, P, P, P, P]
        L.stepq_readout.restype = ctypes.c_int
        L.stepq_readout.argtypes = [P, i32, P, i32, P, P, P, P, P, P, P, P, P]
        L.stepq_status_string.restype = ctypes.c_char_p
        L.stepq_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != STEPQ_OK:
        raise StepqError(status, where)


# Shape of every live layout handle created through this module: the C ABI
# takes raw device pointers and cannot see buffer sizes, so tensor arguments
# are checked here (a buffer shorter than the call implies would otherwise be
# read or written out of bounds on the device).  Raw integer pointers and
# handles created elsewhere pass through unchecked.
_layouts: dict[int, tuple] = {}     # handle -> (H*D, H, gate floats per request, slot bytes, scale bytes, D)
_checks = True


def set_argument_checks(enabled: bool) -> None:
    """Turns the tensor argument checks of pack / unpack / decode_step /
    readout on or off (on by default; about half a microsecond per tensor).
    Off suits a loop that reuses buffers already checked by an earlier call."""
    global _checks
    _checks = bool(enabled)


def _bad(where: str, name: str, t, nbytes: int, dtype) -> None:
    import torch
    if not isinstance(t, torch.Tensor):
        detail = f"{name} must be a torch tensor or an integer pointer"
    elif not t.is_cuda:
        detail = f"{name} must be a device tensor (got {t.device})"
    elif not t.is_contiguous():
        detail = f"{name} must be contiguous"
    elif dtype is not None and t.dtype != dtype:
        detail = f"{name} must be {dtype} (got {t.dtype})"
    else:
        detail = f"{name} holds {t.nbytes} bytes, the call needs {nbytes}"
    raise StepqError(STEPQ_ERR_INVALID_ARG, where, detail)


def _validate(where: str, layout: int, batch: int, num_slots: int, slot_ids, pool, scales,
              q=None, k=None, v=None, beta=None, gate=None, o=None, state=None) -> None:
    if not _checks:
        return
    meta = _layouts.get(layout)
    if meta is None or batch <= 0 or num_slots < 1 or slot_ids is None:
        return                       # the library returns the status for these
    import torch
    f32 = torch.float32
    hd, h, gate_n, slot_bytes, scale_bytes, d = meta
    for name, t, nbytes, dt in (("slot_ids", slot_ids, 4 * batch, torch.int32),
                                ("pool", pool, num_slots * slot_bytes, None),
                                ("scales", scales, num_slots * scale_bytes, None),
                                ("q", q, 4 * batch * hd, f32), ("k", k, 4 * batch * hd, f32),
                                ("v", v, 4 * batch * hd, f32), ("o", o, 4 * batch * hd, f32),
                                ("beta", beta, 4 * batch * h, f32), ("gate", gate, 4 * batch * gate_n, f32),
                                ("state", state, 4 * batch * hd * d, f32)):
        if t is None or isinstance(t, int):
            continue
        try:
            ok = t.is_cuda and t.is_contiguous() and (dt is None or t.dtype == dt) and t.nbytes >= nbytes
        except AttributeError:
            ok = False
        if not ok:
            _bad(where, name, t, nbytes, dt)


def stepq_status_string(status: int) -> str:
    return lib().stepq_status_string(int(status)).decode()


def stepq_layout_create(num_heads: int, d_k: int, d_v: int, gate_mode: int, unit_bits, row_impact,
                        row_scale_mode: int = ROW_SCALES_CALIBRATED, row_magnitude=None) -> int:
    """Returns the layout handle (an int).  unit_bits/row_impact/row_magnitude:
    host arrays (row_magnitude only with the calibrated row-scale mode, the
    default; the per-step refit of row scales, ROW_SCALES_REFIT, is chosen
    explicitly)."""
    ub_in = np.asarray(unit_bits)
    if ub_in.size and (ub_in.min() < 0 or ub_in.max() > 255):
        raise StepqError(STEPQ_ERR_INVALID_ARG, "stepq_layout_create", "unit_bits must fit in a byte")
    ub = np.ascontiguousarray(ub_in, dtype=np.uint8)
    ri = np.ascontiguousarray(np.asarray(row_impact), dtype=np.float32)
    rm = None if row_magnitude is None else np.ascontiguousarray(np.asarray(row_magnitude), dtype=np.float32)
    # the library reads H (per-head gate) or H*d_k widths and H*d_k weights from these host arrays
    if int(num_heads) >= 1 and int(d_k) >= 1 and int(gate_mode) in (0, 1):
        rows = int(num_heads) * int(d_k)
        for name, arr, n in (("unit_bits", ub, int(num_heads) if int(gate_mode) == 0 else rows),
                             ("row_impact", ri, rows), ("row_magnitude", rm, rows)):
            if arr is not None and arr.size != n:
                raise StepqError(STEPQ_ERR_INVALID_ARG, "stepq_layout_create",
                                 f"{name} has {arr.size} entries, the layout needs {n}")
    desc = stepq_layout_desc(int(num_heads), int(d_k), int(d_v), int(gate_mode),
                             ub.ctypes.data_as(ctypes.c_void_p).value,
                             ri.ctypes.data_as(ctypes.c_void_p).value, int(row_scale_mode),
                             None if rm is None else rm.ctypes.data_as(ctypes.c_void_p).value)
    h = ctypes.c_void_p()
    _check(lib().stepq_layout_create(ctypes.byref(desc), ctypes.byref(h)), "stepq_layout_create")
    L = lib()
    H, D = int(num_heads), int(d_k)
    _layouts[h.value] = (H * D, H, H * D if int(gate_mode) == 1 else H, int(L.stepq_slot_pool_bytes(h.value)),
                         int(L.stepq_slot_scale_bytes(h.value)), D)
    return h.value


def stepq_layout_destroy(layout: int) -> None:
    _layouts.pop(layout, None)
    lib().stepq_layout_destroy(layout)


def stepq_slot_pool_bytes(layout: int) -> int:
    return int(lib().stepq_slot_pool_bytes(layout))


def stepq_slot_scale_bytes(layout: int) -> int:
    return int(lib().stepq_slot_scale_bytes(layout))


def stepq_pack(layout: int, batch: int, slot_ids, num_slots: int, state, pool, scales, stream=None) -> None:
    _validate("stepq_pack", layout, batch, num_slots, slot_ids, pool, scales, state=state)
    _check(lib().stepq_pack(layout, int(batch), _ptr(slot_ids), int(num_slots), _ptr(state), _ptr(pool),
                            _ptr(scales), _stream(stream)), "stepq_pack")


def stepq_unpack(layout: int, batch: int, slot_ids, num_slots: int, pool, scales, state, stream=None) -> None:
    _validate("stepq_unpack", layout, batch, num_slots, slot_ids, pool, scales, state=state)
    _check(lib().stepq_unpack(layout, int(batch), _ptr(slot_ids), int(num_slots), _ptr(pool), _ptr(scales),
                              _ptr(state), _stream(stream)), "stepq_unpack")


def stepq_decode_step(layout: int, batch: int, slot_ids, num_slots: int, q, k, v, beta, gate, pool, scales, o,
                      stream=None) -> None:
    _validate("stepq_decode_step", layout, batch, num_slots, slot_ids, pool, scales, q, k, v, beta, gate, o)
    _check(lib().stepq_decode_step(layout, int(batch), _ptr(slot_ids), int(num_slots), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(beta), _ptr(gate), _ptr(pool), _ptr(scales), _ptr(o), _stream(stream)),
           "stepq_decode_step")


def stepq_readout(layout: int, batch: int, slot_ids, num_slots: int, q, k, v, beta, gate, pool, scales, o,
                  stream=None) -> None:
    _validate("stepq_readout", layout, batch, num_slots, slot_ids, pool, scales, q, k, v, beta, gate, o)
    _check(lib().stepq_readout(layout, int(batch), _ptr(slot_ids), int(num_slots), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(beta), _ptr(gate), _ptr(pool), _ptr(scales), _ptr(o), _stream(stream)),
           "stepq_readout")


class Layout:
    """Owns a layout handle; sizes of pool and scale buffers for num_slots slots."""

    def __init__(self, num_heads: int, d: int, gate_mode: int, unit_bits, row_impact,
                 row_scale_mode: int = ROW_SCALES_CALIBRATED, row_magnitude=None):
        self.H, self.D, self.gate_mode = int(num_heads), int(d), int(gate_mode)
        self.row_scale_mode = int(row_scale_mode)
        self.handle = stepq_layout_create(num_heads, d, d, gate_mode, unit_bits, row_impact,
                                          row_scale_mode, row_magnitude)
        self.slot_bytes = stepq_slot_pool_bytes(self.handle)
        self.scale_bytes = stepq_slot_scale_bytes(self.handle)

    @classmethod
    def from_workload(cls, lay) -> "Layout":
        return cls(lay.H, lay.D, lay.gate_mode, lay.unit_bits, lay.row_impact, lay.row_mode,
                   lay.row_magnitude if lay.row_mode == ROW_SCALES_CALIBRATED else None)

    def alloc(self, num_slots: int, device="cuda"):
        """Zeroed pool and scale buffers (torch uint8 / int16 device tensors)."""
        import torch
        pool = torch.zeros(num_slots * self.slot_bytes, dtype=torch.uint8, device=device)
        scales = torch.zeros(num_slots * self.scale_bytes // 2, dtype=torch.int16, device=device)
        return pool, scales

    def close(self) -> None:
        if getattr(self, "handle", None):
            stepq_layout_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
