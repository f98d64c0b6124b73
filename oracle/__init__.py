"""ctypes wrapper over the plain-C CPU oracle (``oracle/cfz_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The library product never imports this
package, and this package imports nothing from the library product.

Arrays are numpy arrays on the host: bf16 is carried as ``uint16`` bit patterns.
Every call works in place on the state arrays it is given, like the C code.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

DELTA, LITERAL, OFF, OPENLOOP = 0, 1, 2, 3
SENDER, RECEIVER = 0, 1

_libs = {}            # "serial" / "openmp" -> loaded library
_active = "serial"


def _load():
    """The active build of the oracle: the serial one unless inside ``parallel()``."""
    lib = _libs.get(_active)
    if lib is not None:
        return lib
    path = _build.LIB_OMP if _active == "openmp" else _build.LIB
    if not os.path.exists(path):
        _build.build()
    lib = C.CDLL(path)
    p = C.c_void_p
    i64, i32 = C.c_int64, C.c_int
    lib.oracle_pack_codes.argtypes = [i64, i32, p, p]
    lib.oracle_unpack_codes.argtypes = [i64, i32, p, p]
    lib.oracle_quantize.argtypes = [i64, i32, i32, p, p, p]
    lib.oracle_warmup.argtypes = [i64, i32, i32, i32, p, p, p, p]
    lib.oracle_compress.argtypes = [i64, i32, i32, i32, i32, p, p, p, p, p, p]
    lib.oracle_decompress.argtypes = [i64, i32, i32, i32, p, p, p, p]
    lib.oracle_bf16_to_f32.argtypes = [i64, p, p]
    lib.oracle_f32_to_bf16.argtypes = [i64, p, p]
    lib.oracle_qr.argtypes = [i64, i32, p, p, p]
    lib.oracle_qr.restype = i32
    lib.oracle_lowrank.argtypes = [i64, i64, i32, i32, p, p, p, p, p]
    lib.oracle_lowrank_ef_update.argtypes = [i64, i64, i32, p, p, p, C.c_double, p]
    lib.oracle_lowrank_ef_compress.argtypes = [i64, i64, i32, i32, p, p, p, p, p, p, p, p]
    lib.oracle_lowrank_ef_decompress.argtypes = [i64, i64, i32, p, p, p, p, p]
    lib.oracle_qmax.argtypes = [i32]
    lib.oracle_qmax.restype = i32
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = i32
    _libs[_active] = lib
    return lib


class parallel:
    """Within ``with oracle.parallel():`` every call goes to the OpenMP build of the same C
    source (identical results; used to time the oracle on all host cores)."""

    def __enter__(self):
        global _active
        self._prev, _active = _active, "openmp"
        return self

    def __exit__(self, *exc):
        global _active
        _active = self._prev
        return False


def threads() -> int:
    """Threads the active build's loops use (1 for the serial build)."""
    return _load().oracle_threads()


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def qmax(bits: int) -> int:
    return _load().oracle_qmax(bits)


def codes_bytes(n: int, bits: int) -> int:
    return n * bits // 8


def _check_codec(n, bits, group):
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    if group <= 0 or n % group or group % 8:
        raise ValueError("group must be a positive multiple of 8 dividing the element count")


# ---------------------------------------------------------------- packing

def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.zeros(q.size * bits // 8, dtype=np.uint8)
    _load().oracle_pack_codes(q.size, bits, _ptr(q), _ptr(out))
    return out


def unpack_codes(codes: np.ndarray, n: int, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros(n, dtype=np.int8)
    _load().oracle_unpack_codes(n, bits, _ptr(codes), _ptr(out))
    return out


# ---------------------------------------------------------------- codec

def quantize(r: np.ndarray, bits: int, group: int):
    """Stateless group quantization of an fp32 array: returns (codes, scales)."""
    r = np.ascontiguousarray(r, dtype=np.float32).reshape(-1)
    _check_codec(r.size, bits, group)
    codes = np.zeros(r.size * bits // 8, dtype=np.uint8)
    scales = np.zeros(r.size // group, dtype=np.float32)
    _load().oracle_quantize(r.size, bits, group, _ptr(r), _ptr(codes), _ptr(scales))
    return codes, scales


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.zeros(h.shape, dtype=np.float32)
    _load().oracle_bf16_to_f32(h.size, _ptr(h), _ptr(out))
    return out


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.zeros(f.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16(f.size, _ptr(f), _ptr(out))
    return out


class Sender:
    """Sender-side codec state: P (bf16 previous activation), E (carried error), X-hat (base).

    E and X-hat are fp32 arrays, or bf16 bit patterns (uint16) with ``state_bf16``."""

    def __init__(self, n, bits=4, group=64, mode=DELTA, x0=None, state_bf16=False):
        _check_codec(n, bits, group)
        self.n, self.bits, self.group, self.mode = n, bits, group, mode
        self.state_bf16 = bool(state_bf16)
        sdt = np.uint16 if state_bf16 else np.float32
        self.prev = np.zeros(n, np.uint16) if mode in (DELTA, OPENLOOP) else None
        self.err = np.zeros(n, sdt) if mode in (DELTA, LITERAL) else None
        self.base = np.zeros(n, sdt) if mode in (LITERAL, OFF) else None
        x0 = None if x0 is None else np.ascontiguousarray(x0, np.uint16).reshape(-1)
        _load().oracle_warmup(n, mode, SENDER, self.state_bf16, _ptr(x0), _ptr(self.prev),
                              _ptr(self.base), _ptr(self.err))

    def compress(self, x: np.ndarray):
        x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
        assert x.size == self.n
        codes = np.zeros(self.n * self.bits // 8, dtype=np.uint8)
        scales = np.zeros(self.n // self.group, dtype=np.float32)
        _load().oracle_compress(self.n, self.bits, self.group, self.mode, self.state_bf16,
                                _ptr(x), _ptr(self.prev), _ptr(self.base), _ptr(self.err),
                                _ptr(codes), _ptr(scales))
        return codes, scales


class Receiver:
    """Receiver-side codec state: X-hat (fp32 base, or bf16 bit patterns with ``state_bf16``)."""

    def __init__(self, n, bits=4, group=64, x0=None, state_bf16=False):
        _check_codec(n, bits, group)
        self.n, self.bits, self.group = n, bits, group
        self.state_bf16 = bool(state_bf16)
        self.base = np.zeros(n, np.uint16 if state_bf16 else np.float32)
        x0 = None if x0 is None else np.ascontiguousarray(x0, np.uint16).reshape(-1)
        _load().oracle_warmup(n, DELTA, RECEIVER, self.state_bf16, _ptr(x0), None,
                              _ptr(self.base), None)

    def decompress(self, codes: np.ndarray, scales: np.ndarray, want_xhat=False):
        codes = np.ascontiguousarray(codes, np.uint8)
        scales = np.ascontiguousarray(scales, np.float32)
        xhat = np.zeros(self.n, np.uint16) if want_xhat else None
        _load().oracle_decompress(self.n, self.bits, self.group, self.state_bf16, _ptr(codes),
                                  _ptr(scales), _ptr(self.base), _ptr(xhat))
        return xhat


# ---------------------------------------------------------------- low rank

def qr(M: np.ndarray):
    """Thin QR (fp64 Householder, diag(R) > 0).  Returns (Q, R, dropped_columns)."""
    M = np.ascontiguousarray(M, dtype=np.float64)
    rows, cols = M.shape
    Q = np.zeros((rows, cols), np.float64)
    R = np.zeros((cols, cols), np.float64)
    dropped = _load().oracle_qr(rows, cols, _ptr(M), _ptr(Q), _ptr(R))
    return Q, R, dropped


def lowrank(A_bf16: np.ndarray, Q0: np.ndarray, T: int):
    """Algorithm 3 on one m x n bf16 matrix: returns (U, V, R_U) in fp64."""
    A_bf16 = np.ascontiguousarray(A_bf16, dtype=np.uint16)
    Q0 = np.ascontiguousarray(Q0, dtype=np.float32)
    m, n = A_bf16.shape
    r = Q0.shape[1]
    assert Q0.shape[0] == n
    U = np.zeros((m, r), np.float64)
    V = np.zeros((n, r), np.float64)
    RU = np.zeros((r, r), np.float64)
    _load().oracle_lowrank(m, n, r, T, _ptr(A_bf16), _ptr(Q0), _ptr(U), _ptr(V), _ptr(RU))
    return U, V, RU


# ---------------------------------------------------------------- low rank inside error feedback

def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def lowrank_ef_update(U, V, RU, sign, Y):
    """Y (m x n fp32, in place) += sign * (U R_U) V^T, each element rounded once from fp64."""
    U, V, RU = _f64(U), _f64(V), _f64(RU)
    m, r = U.shape
    n = V.shape[0]
    assert Y.dtype == np.float32 and Y.size == m * n and Y.flags["C_CONTIGUOUS"]
    _load().oracle_lowrank_ef_update(m, n, r, _ptr(U), _ptr(V), _ptr(RU), float(sign), _ptr(Y))
    return Y


class LowrankSender:
    """Sender state of the rank-r compressor inside error feedback: prev (bf16 bits) and the
    fp32 carried error, warmed up like the quantizer's DELTA mode."""

    def __init__(self, m, n, x0=None):
        self.m, self.n = m, n
        self.prev = np.zeros(m * n, np.uint16)
        self.err = np.zeros(m * n, np.float32)
        if x0 is not None:
            self.prev[:] = np.ascontiguousarray(x0, np.uint16).reshape(-1)

    def compress(self, x, Q0, T):
        """One step: returns (U, V, RU) in fp64 and A, the bf16 residual that was compressed."""
        x = np.ascontiguousarray(x, np.uint16).reshape(-1)
        Q0 = np.ascontiguousarray(Q0, np.float32)
        r = Q0.shape[1]
        assert x.size == self.m * self.n and Q0.shape[0] == self.n
        A = np.zeros(self.m * self.n, np.uint16)
        U = np.zeros((self.m, r), np.float64)
        V = np.zeros((self.n, r), np.float64)
        RU = np.zeros((r, r), np.float64)
        _load().oracle_lowrank_ef_compress(self.m, self.n, r, T, _ptr(x), _ptr(self.prev),
                                           _ptr(self.err), _ptr(Q0), _ptr(A), _ptr(U), _ptr(V),
                                           _ptr(RU))
        return U, V, RU, A


class LowrankReceiver:
    """Receiver state: the fp32 base, warmed up to x0."""

    def __init__(self, m, n, x0=None):
        self.m, self.n = m, n
        self.base = np.zeros(m * n, np.float32)
        if x0 is not None:
            self.base[:] = bf16_to_f32(np.ascontiguousarray(x0, np.uint16).reshape(-1))

    def decompress(self, U, V, RU, want_xhat=False):
        U, V, RU = _f64(U), _f64(V), _f64(RU)
        r = U.shape[1]
        xhat = np.zeros(self.m * self.n, np.uint16) if want_xhat else None
        _load().oracle_lowrank_ef_decompress(self.m, self.n, r, _ptr(U), _ptr(V), _ptr(RU),
                                             _ptr(self.base), _ptr(xhat))
        return xhat
