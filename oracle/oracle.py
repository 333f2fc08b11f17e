"""Python handle on the CPU oracle of the STEPQuant packed-state decode step.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  The arithmetic
lives in stepq_oracle.cpp (float64, one element at a time); this file only
builds it with g++ and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "stepq_oracle.cpp"
DEFAULT_LIB = HERE / "libstepq_oracle.so"
# STEPQ_ORACLE_LIB names another build of the same source (the sanitizer test
# builds one with -fsanitize=address,undefined); it is loaded as it is.
LIB = Path(os.environ.get("STEPQ_ORACLE_LIB", DEFAULT_LIB))

_lib = None


COMPILE_FLAGS = ["-std=c++17", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = False) -> Path:
    """Compile the oracle (g++, OpenMP, no FMA contraction, no fast-math)."""
    if LIB != DEFAULT_LIB:
        return LIB
    if force or not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
        tmp = LIB.with_suffix(".so.tmp")
        cmd = ["g++", "-O2", *COMPILE_FLAGS, str(SRC), "-o", str(tmp)]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(str(LIB))
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        sig = {
            "ora_layout_check": (i32, [i32, i32, i32, P, P, P]),
            "ora_slot_bytes": (i64, [i32, i32, i32, P]),
            "ora_head_word_offset": (i64, [i32, i32, i32, P, i32]),
            "ora_half_from_double": (ctypes.c_uint16, [f64]),
            "ora_double_from_half": (f64, [ctypes.c_uint16]),
            "ora_encode_fields": (None, [i32, P, P, P, i64]),
            "ora_decode_fields": (None, [i32, P, P, P]),
            "ora_quantize_tile": (i32, [i32, i32, i32, P, P, P, i32, P, P, P, P, P, P, P, P]),
            "ora_reconstruct_tile": (i32, [i32, i32, i32, P, i32, P, P, P, P]),
            "ora_fit_columns_for_codes": (i32, [i32, i32, i32, P, P, P, i32, P, P, P]),
            "ora_pack": (i32, [i32, i32, i32, P, P, P, i32, P, P, P, P]),
            "ora_unpack": (i32, [i32, i32, i32, P, i32, P, P, P, P]),
            "ora_step": (i32, [i32, i32, i32, P, P, P, i32, P, P, P, P, P, P, P, P, P, P, P, P, i64]),
            "ora_step_tile_diag": (i32, [i32, i32, i32, P, P, P, i32, P, P, P, f32, P, P, P, P, P,
                                         P, P, P, P]),
            "ora_tile_decode": (i32, [i32, i32, i32, P, i32, P, P]),
            "ora_tile_encode": (i32, [i32, i32, i32, P, i32, P, P]),
            "ora_uniform_step": (i32, [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P]),
            "ora_uniform_pack": (i32, [i32, i32, i32, i32, P, P, P]),
            "ora_num_threads": (i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


class OracleLayout:
    """The oracle's own reading of a layout description (H, D, gate mode, widths,
    impact weights, and -- for the calibrated row-scale reading -- the calibrated
    row magnitudes; row_mag None selects the per-step refit of row scales)."""

    def __init__(self, H: int, D: int, gate_mode: int, unit_bits, row_impact, row_mag=None):
        self.H, self.D, self.gate_mode = int(H), int(D), int(gate_mode)
        self.unit_bits = _c(unit_bits, np.uint8)
        self.row_impact = _c(row_impact, np.float32)
        self.row_mag = None if row_mag is None else _c(row_mag, np.float32)
        if lib().ora_layout_check(self.H, self.D, self.gate_mode, _p(self.unit_bits), _p(self.row_impact),
                                  _p(self.row_mag)):
            raise ValueError("invalid layout description")
        self.slot_bytes = int(lib().ora_slot_bytes(self.H, self.D, self.gate_mode, _p(self.unit_bits)))
        self.scale_halves = self.H * 2 * self.D
        self._head_off = [int(lib().ora_head_word_offset(*self._args(), h)) for h in range(self.H + 1)]

    @classmethod
    def from_workload(cls, lay) -> "OracleLayout":
        return cls(lay.H, lay.D, lay.gate_mode, lay.unit_bits, lay.row_impact,
                   lay.row_magnitude if lay.row_mode == 1 else None)

    def _args(self):
        return (self.H, self.D, self.gate_mode, _p(self.unit_bits))

    def head_word_offset(self, h: int) -> int:
        return self._head_off[h]

    def head_words(self, h: int) -> int:
        return self.head_word_offset(h + 1) - self.head_word_offset(h)

    def row_bits(self) -> np.ndarray:
        if self.gate_mode == 0:
            return np.repeat(self.unit_bits.reshape(self.H, 1), self.D, axis=1).astype(np.int32)
        return self.unit_bits.reshape(self.H, self.D).astype(np.int32)

    def new_pool(self, num_slots: int):
        return (np.zeros(num_slots * self.slot_bytes, np.uint8),
                np.zeros(num_slots * self.scale_halves, np.uint16))

    def pack(self, slot_ids, state, pool, scales):
        slot_ids = _c(slot_ids, np.int32)
        state = _c(state, np.float32)
        B = slot_ids.size
        assert state.shape == (B, self.H, self.D, self.D)
        rc = lib().ora_pack(*self._args(), _p(self.row_impact), _p(self.row_mag), B, _p(slot_ids), _p(state), _p(pool), _p(scales))
        assert rc == 0

    def unpack(self, slot_ids, pool, scales) -> np.ndarray:
        slot_ids = _c(slot_ids, np.int32)
        B = slot_ids.size
        out = np.empty((B, self.H, self.D, self.D), np.float32)
        rc = lib().ora_unpack(*self._args(), B, _p(slot_ids), _p(pool), _p(scales), _p(out))
        assert rc == 0
        return out

    def step(self, slot_ids, inp: dict, pool_in, scales_in, pool_out=None, scales_out=None,
             tiles=None):
        """One decode step; returns o [B, H, D].  Writes pool_out/scales_out
        (default: in place).  tiles: optional tile indices b*H + h to process."""
        slot_ids = _c(slot_ids, np.int32)
        B = slot_ids.size
        q, k, v = (_c(inp[n], np.float32) for n in ("q", "k", "v"))
        beta, gate = _c(inp["beta"], np.float32), _c(inp["gate"], np.float32)
        assert q.shape == (B, self.H, self.D) and beta.shape == (B, self.H)
        pool_out = pool_in if pool_out is None else pool_out
        scales_out = scales_in if scales_out is None else scales_out
        o = np.zeros((B, self.H, self.D), np.float32)
        tl = None if tiles is None else _c(tiles, np.int32)
        rc = lib().ora_step(*self._args(), _p(self.row_impact), _p(self.row_mag), B, _p(slot_ids), _p(q), _p(k), _p(v),
                            _p(beta), _p(gate), _p(pool_in), _p(scales_in), _p(pool_out),
                            _p(scales_out), _p(o), _p(tl), 0 if tl is None else tl.size)
        assert rc == 0
        return o

    def quantize_tile(self, h: int, Mp: np.ndarray) -> dict:
        D = self.D
        Mp = _c(Mp, np.float64)
        words = np.zeros(self.head_words(h), np.uint32)
        rhat = np.zeros(D, np.uint16)
        chat = np.zeros(D, np.uint16)
        r, c0, c = np.zeros(D), np.zeros(D), np.zeros(D)
        codes = np.zeros((D, D), np.int32)
        rc = lib().ora_quantize_tile(*self._args(), _p(self.row_impact), _p(self.row_mag), h, _p(Mp), _p(words),
                                     _p(rhat), _p(chat), _p(r), _p(c0), _p(c), _p(codes))
        assert rc == 0
        return dict(words=words, rhat=rhat, chat=chat, r=r, c0=c0, c=c, codes=codes)

    def fit_columns_for_codes(self, h: int, Mp, codes) -> np.ndarray:
        """binary16 column scales the rule gives for M' (float64) and the given codes."""
        chat = np.zeros(self.D, np.uint16)
        rc = lib().ora_fit_columns_for_codes(*self._args(), _p(self.row_impact), _p(self.row_mag), h, _p(_c(Mp, np.float64)),
                                             _p(_c(codes, np.int32)), _p(chat))
        assert rc == 0
        return chat

    def reconstruct_tile(self, h: int, words, rhat, chat) -> np.ndarray:
        M = np.zeros((self.D, self.D))
        rc = lib().ora_reconstruct_tile(*self._args(), h, _p(_c(words, np.uint32)),
                                        _p(_c(rhat, np.uint16)), _p(_c(chat, np.uint16)), _p(M))
        assert rc == 0
        return M

    def step_tile_diag(self, h, q, k, v, beta, gate_rows, words, rhat, chat):
        D = self.D
        wo = np.zeros(self.head_words(h), np.uint32)
        ro, co = np.zeros(D, np.uint16), np.zeros(D, np.uint16)
        o = np.zeros(D, np.float32)
        Mp = np.zeros((D, D))
        rc = lib().ora_step_tile_diag(*self._args(), _p(self.row_impact), _p(self.row_mag), h, _p(_c(q, np.float32)),
                                      _p(_c(k, np.float32)), _p(_c(v, np.float32)), float(beta),
                                      _p(_c(gate_rows, np.float32)), _p(_c(words, np.uint32)),
                                      _p(_c(rhat, np.uint16)), _p(_c(chat, np.uint16)), _p(wo),
                                      _p(ro), _p(co), _p(o), _p(Mp))
        assert rc == 0
        return dict(words=wo, rhat=ro, chat=co, o=o, Mp=Mp)

    def decode_tile(self, h: int, words) -> np.ndarray:
        """Fields [D, D] (row-major by original row) of one tile's words."""
        fields = np.zeros((self.D, self.D), np.uint32)
        assert lib().ora_tile_decode(*self._args(), h, _p(_c(words, np.uint32)), _p(fields)) == 0
        return fields

    def encode_tile(self, h: int, fields) -> np.ndarray:
        words = np.zeros(self.head_words(h), np.uint32)
        assert lib().ora_tile_encode(*self._args(), h, _p(_c(fields, np.uint32)), _p(words)) == 0
        return words

    # tile views into a pool
    def tile_words(self, pool: np.ndarray, slot: int, h: int) -> np.ndarray:
        base = slot * self.slot_bytes // 4 + self.head_word_offset(h)
        return pool.view(np.uint32)[base: base + self.head_words(h)]

    def tile_scales(self, scales: np.ndarray, slot: int, h: int):
        base = (slot * self.H + h) * 2 * self.D
        return scales[base: base + self.D], scales[base + self.D: base + 2 * self.D]


def half_from_double(x: float) -> int:
    return int(lib().ora_half_from_double(float(x)))


def double_from_half(h: int) -> float:
    return float(lib().ora_double_from_half(int(h)))


def encode_fields(row_bits, fields) -> np.ndarray:
    row_bits = _c(row_bits, np.int32)
    D = row_bits.size
    fields = _c(fields, np.uint32)
    assert fields.shape == (D, D)
    nw = ((int(row_bits.sum()) + 31) // 32) * D
    words = np.zeros(nw, np.uint32)
    lib().ora_encode_fields(D, _p(row_bits), _p(fields), _p(words), nw)
    return words


def decode_fields(row_bits, words) -> np.ndarray:
    row_bits = _c(row_bits, np.int32)
    D = row_bits.size
    fields = np.zeros((D, D), np.uint32)
    lib().ora_decode_fields(D, _p(row_bits), _p(_c(words, np.uint32)), _p(fields))
    return fields


def uniform_pack(state, bits: int):
    state = _c(state, np.float32)
    B, H, D, _ = state.shape
    codes = np.zeros(state.shape, np.int32)
    scale = np.zeros((B, H), np.float32)
    assert lib().ora_uniform_pack(B, H, D, bits, _p(state), _p(codes), _p(scale)) == 0
    return codes, scale


def uniform_step(codes, scale, inp: dict, bits: int, gate_mode: int):
    B, H, D, _ = codes.shape
    q, k, v = (_c(inp[n], np.float32) for n in ("q", "k", "v"))
    beta, gate = _c(inp["beta"], np.float32), _c(inp["gate"], np.float32)
    o = np.zeros((B, H, D), np.float32)
    assert lib().ora_uniform_step(B, H, D, gate_mode, bits, _p(q), _p(k), _p(v), _p(beta), _p(gate),
                                  _p(codes), _p(scale), _p(o)) == 0
    return o


def num_threads() -> int:
    return int(lib().ora_num_threads())
