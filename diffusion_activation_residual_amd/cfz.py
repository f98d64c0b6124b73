"""Thin ctypes binding over libcfz (``include/cfz.h``): argument marshalling only.

Every step of the codec and of the subspace iteration runs in the HIP kernels
of ``libcfz.so``; this module converts torch tensors into raw device pointers
and the current HIP stream, calls the C entry point of the same name, and
turns a non-OK status into ``CfzError``.  Because it sees tensor sizes, which
the C ABI cannot, it also refuses (``ValueError``, before any device work) a
tensor smaller than the call would touch.  torch supplies device memory and
streams, nothing else.  There is no fallback: if the library is not built,
importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcfz.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "cfz.h")

CFZ_OK, CFZ_ERR_NULL, CFZ_ERR_SHAPE, CFZ_ERR_UNSUPPORTED = 0, 1, 2, 3
CFZ_ERR_ALIGN, CFZ_ERR_MODE, CFZ_ERR_WORKSPACE, CFZ_ERR_HIP = 4, 5, 6, 7
CFZ_EF_DELTA, CFZ_EF_LITERAL, CFZ_EF_OFF = 0, 1, 2
CFZ_SENDER, CFZ_RECEIVER = 0, 1
CFZ_STATE_F32, CFZ_STATE_BF16 = 0, 1
MODES = {"delta": CFZ_EF_DELTA, "literal": CFZ_EF_LITERAL, "off": CFZ_EF_OFF}


class cfz_desc(C.Structure):
    _fields_ = [("rows", C.c_int64), ("cols", C.c_int64), ("bits", C.c_int32),
                ("group", C.c_int32), ("ef_mode", C.c_int32), ("role", C.c_int32),
                ("state_dtype", C.c_int32), ("reserved", C.c_int32)]


class cfz_buffers(C.Structure):
    _fields_ = [("prev_bf16", C.c_void_p), ("base", C.c_void_p), ("err", C.c_void_p)]


class CfzError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = _lib.cfz_last_error().decode(errors="replace")
        name = _lib.cfz_status_string(status).decode()
        super().__init__(f"{where}: {name} (status {status}): {detail}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libcfz.so is not built ({LIB_PATH}); build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` at the repository root")
    lib = C.CDLL(LIB_PATH)
    p, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
    sig = {
        "cfz_state_create": ([C.POINTER(cfz_desc), C.POINTER(cfz_buffers), p, p, C.POINTER(p)], i32),
        "cfz_state_resume": ([C.POINTER(cfz_desc), C.POINTER(cfz_buffers), i64, C.POINTER(p)], i32),
        "cfz_state_destroy": ([p], i32),
        "cfz_state_steps": ([p], i64),
        "cfz_codes_bytes": ([C.POINTER(cfz_desc)], sz),
        "cfz_scales_bytes": ([C.POINTER(cfz_desc)], sz),
        "cfz_compress": ([p, p, p, p, p], i32),
        "cfz_decompress": ([p, p, p, p, p], i32),
        "cfz_compress_group": ([i32, p, p, p, p, p], i32),
        "cfz_decompress_group": ([i32, p, p, p, p, p], i32),
        "cfz_lowrank_workspace_bytes": ([i64, i64, i64, i32], sz),
        "cfz_lowrank": ([i64, i64, i64, i32, i32, p, p, p, p, p, p, sz, p], i32),
        "cfz_lowrank_noalloc": ([i64, i64, i64, i32, i32, p, p, p, p, p, p], i32),
        "cfz_lowrank_noalloc_max_bytes": ([], sz),
        "cfz_lowrank_ef_workspace_bytes": ([i64, i64, i64, i32], sz),
        "cfz_lowrank_ef_warmup": ([i64, p, p, p, p, p], i32),
        "cfz_lowrank_ef_compress": ([i64, i64, i64, i32, i32, p, p, p, p, p, p, p, p, sz, p], i32),
        "cfz_lowrank_ef_compress_deferred": ([i64, i64, i64, i32, i32, i32, p, p, p, p, p, p, p,
                                              p, sz, p], i32),
        "cfz_lowrank_ef_flush": ([i64, i64, i64, i32, p, p, p, p, p], i32),
        "cfz_lowrank_ef_decompress": ([i64, i64, i64, i32, p, p, p, p, p, p], i32),
        "cfz_stream_copy": ([p, p, sz, p], i32),
        "cfz_stream_mix": ([p, sz, p, sz, p], i32),
        "cfz_status_string": ([i32], C.c_char_p),
        "cfz_last_error": ([], C.c_char_p),
        "cfz_abi_version": ([], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def header_functions():
    """Names of the functions ``include/cfz.h`` declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cfz_[a-z_0-9]+)\s*\(", text)))


def _check(status, where):
    if status != CFZ_OK:
        raise CfzError(status, where)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libcfz takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libcfz takes contiguous tensors")
    return t.data_ptr()


# handle -> sizes its calls touch (elements, codes bytes, scales bytes), for the size checks
_sizes = {}


def _need(t, nbytes, what):
    """Raise before any device work when a tensor is smaller than the call will touch (raw
    integer pointers are the caller's responsibility, as in C)."""
    if t is None or isinstance(t, int):
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: tensor holds {have} bytes, the call touches {nbytes}")


def _need_dtype(t, dtypes, what):
    """The same host-side guard for element types the kernels read as fp32 or bf16."""
    if t is None or isinstance(t, int):
        return
    if t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise TypeError(f"{what}: {str(t.dtype).replace('torch.', '')} tensor, expected {names}")


_F32 = (torch.float32,)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _record(handle, desc):
    n = max(desc.rows * desc.cols, 0)
    _sizes[handle] = (n, _lib.cfz_codes_bytes(C.byref(desc)), _lib.cfz_scales_bytes(C.byref(desc)))


def _check_state_buffers(desc, prev, base, err, x0=None):
    n = max(desc.rows * desc.cols, 0)
    w = 2 if desc.state_dtype == CFZ_STATE_BF16 else 4
    sdt = _BF16 if desc.state_dtype == CFZ_STATE_BF16 else _F32
    _need_dtype(base, sdt, "base")
    _need_dtype(err, sdt, "err")
    _need(prev, 2 * n, "prev")
    _need(base, w * n, "base")
    _need(err, w * n, "err")
    _need(x0, 2 * n, "x0")


def _check_payload(handle, x=None, codes=None, scales=None, xhat=None):
    if handle not in _sizes:
        return
    n, cb, sb = _sizes[handle]
    _need_dtype(scales, _F32, "scales")
    _need(x, 2 * n, "x")
    _need(codes, cb, "codes")
    _need(scales, sb, "scales")
    _need(xhat, 2 * n, "xhat")


def _check_lowrank(batch, m, n, r, A=None, Q0=None, U=None, V=None, RU=None):
    b, m, n, r = (max(int(v), 0) for v in (batch, m, n, r))
    for t, what in ((Q0, "Q0"), (U, "U"), (V, "V"), (RU, "RU")):
        _need_dtype(t, _F32, what)
    _need(A, 2 * b * m * n, "A")
    _need(Q0, 4 * b * n * r, "Q0")
    _need(U, 4 * b * m * r, "U")
    _need(V, 4 * b * n * r, "V")
    _need(RU, 4 * b * r * r, "RU")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _bf16_ptr(t):
    if t is not None and not isinstance(t, int) and t.dtype not in (torch.bfloat16, torch.int16,
                                                                    torch.uint16):
        raise TypeError("bf16 data must be a bfloat16 (or 16-bit bit-pattern) tensor")
    return _ptr(t)


# ------------------------------------------------------------------ raw entry points

def cfz_abi_version() -> int:
    return _lib.cfz_abi_version()


def cfz_status_string(status: int) -> str:
    return _lib.cfz_status_string(status).decode()


def cfz_last_error() -> str:
    return _lib.cfz_last_error().decode(errors="replace")


def make_desc(rows, cols, bits=4, group=64, ef_mode=CFZ_EF_DELTA, role=CFZ_SENDER,
              state_dtype=CFZ_STATE_F32) -> cfz_desc:
    return cfz_desc(rows, cols, bits, group, ef_mode, role, state_dtype, 0)


def cfz_codes_bytes(desc: cfz_desc) -> int:
    return _lib.cfz_codes_bytes(C.byref(desc))


def cfz_scales_bytes(desc: cfz_desc) -> int:
    return _lib.cfz_scales_bytes(C.byref(desc))


def cfz_state_create(desc: cfz_desc, prev=None, base=None, err=None, x0=None, stream=None):
    _check_state_buffers(desc, prev, base, err, x0)
    bufs = cfz_buffers(_bf16_ptr(prev), _ptr(base), _ptr(err))
    out = C.c_void_p()
    _check(_lib.cfz_state_create(C.byref(desc), C.byref(bufs), _bf16_ptr(x0), _stream(stream),
                                 C.byref(out)), "cfz_state_create")
    _record(out.value, desc)
    return out.value


def cfz_state_resume(desc: cfz_desc, prev=None, base=None, err=None, steps=0):
    _check_state_buffers(desc, prev, base, err)
    bufs = cfz_buffers(_bf16_ptr(prev), _ptr(base), _ptr(err))
    out = C.c_void_p()
    _check(_lib.cfz_state_resume(C.byref(desc), C.byref(bufs), steps, C.byref(out)),
           "cfz_state_resume")
    _record(out.value, desc)
    return out.value


def cfz_state_destroy(handle) -> None:
    _sizes.pop(handle, None)
    _check(_lib.cfz_state_destroy(handle), "cfz_state_destroy")


def cfz_state_steps(handle) -> int:
    return _lib.cfz_state_steps(handle)


def cfz_compress(handle, x, codes, scales, stream=None) -> None:
    _check_payload(handle, x=x, codes=codes, scales=scales)
    _check(_lib.cfz_compress(handle, _bf16_ptr(x), _ptr(codes), _ptr(scales), _stream(stream)),
           "cfz_compress")


def cfz_decompress(handle, codes, scales, xhat=None, stream=None) -> None:
    _check_payload(handle, codes=codes, scales=scales, xhat=xhat)
    _check(_lib.cfz_decompress(handle, _ptr(codes), _ptr(scales), _bf16_ptr(xhat),
                               _stream(stream)), "cfz_decompress")


def _ptr_array(items, fn=_ptr):
    arr = (C.c_void_p * max(len(items), 1))()
    for i, t in enumerate(items):
        arr[i] = fn(t)
    return arr


def cfz_compress_group(handles, xs, codes, scales, stream=None) -> None:
    """One grouped compress over len(handles) tensors (entry i: handles[i], xs[i], ...)."""
    n = len(handles)
    if not (len(xs) == len(codes) == len(scales) == n):
        raise ValueError("all lists must have one entry per state")
    for i in range(n):
        _check_payload(handles[i], x=xs[i], codes=codes[i], scales=scales[i])
    _check(_lib.cfz_compress_group(n, _ptr_array(handles, lambda h: h), _ptr_array(xs, _bf16_ptr),
                                   _ptr_array(codes), _ptr_array(scales), _stream(stream)),
           "cfz_compress_group")


def cfz_decompress_group(handles, codes, scales, xhats=None, stream=None) -> None:
    n = len(handles)
    if not (len(codes) == len(scales) == n) or (xhats is not None and len(xhats) != n):
        raise ValueError("all lists must have one entry per state")
    for i in range(n):
        _check_payload(handles[i], codes=codes[i], scales=scales[i],
                       xhat=None if xhats is None else xhats[i])
    xa = None if xhats is None else _ptr_array(xhats, _bf16_ptr)
    _check(_lib.cfz_decompress_group(n, _ptr_array(handles, lambda h: h), _ptr_array(codes),
                                     _ptr_array(scales), xa, _stream(stream)),
           "cfz_decompress_group")


def cfz_lowrank_workspace_bytes(batch, m, n, r) -> int:
    return _lib.cfz_lowrank_workspace_bytes(batch, m, n, r)


def cfz_lowrank(batch, m, n, r, T, A, Q0, U, V, RU, workspace, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check_lowrank(batch, m, n, r, A, Q0, U, V, RU)
    _need(workspace, ws_bytes, "workspace")
    _check(_lib.cfz_lowrank(batch, m, n, r, T, _bf16_ptr(A), _ptr(Q0), _ptr(U), _ptr(V),
                            _ptr(RU), _ptr(workspace), ws_bytes, _stream(stream)), "cfz_lowrank")


def cfz_lowrank_noalloc_max_bytes() -> int:
    return _lib.cfz_lowrank_noalloc_max_bytes()


def cfz_lowrank_noalloc(batch, m, n, r, T, A, Q0, U, V, RU, stream=None) -> None:
    """cfz_lowrank on the library's built-in scratch: no workspace argument, no allocation."""
    _check_lowrank(batch, m, n, r, A, Q0, U, V, RU)
    _check(_lib.cfz_lowrank_noalloc(batch, m, n, r, T, _bf16_ptr(A), _ptr(Q0), _ptr(U), _ptr(V),
                                    _ptr(RU), _stream(stream)), "cfz_lowrank_noalloc")


def cfz_lowrank_ef_workspace_bytes(batch, m, n, r) -> int:
    return _lib.cfz_lowrank_ef_workspace_bytes(batch, m, n, r)


def cfz_lowrank_ef_warmup(count, x0=None, prev=None, err=None, base=None, stream=None) -> None:
    c = max(int(count), 0)
    _need_dtype(err, _F32, "err")
    _need_dtype(base, _F32, "base")
    _need(x0, 2 * c, "x0")
    _need(prev, 2 * c, "prev")
    _need(err, 4 * c, "err")
    _need(base, 4 * c, "base")
    _check(_lib.cfz_lowrank_ef_warmup(count, _bf16_ptr(x0), _bf16_ptr(prev), _ptr(err), _ptr(base),
                                      _stream(stream)), "cfz_lowrank_ef_warmup")


def cfz_lowrank_ef_compress(batch, m, n, r, T, x, prev, err, Q0, U, V, RU, workspace,
                            ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check_lowrank(batch, m, n, r, None, Q0, U, V, RU)
    c = max(int(batch), 0) * max(int(m), 0) * max(int(n), 0)
    _need_dtype(err, _F32, "err")
    _need(x, 2 * c, "x")
    _need(prev, 2 * c, "prev")
    _need(err, 4 * c, "err")
    _need(workspace, ws_bytes, "workspace")
    _check(_lib.cfz_lowrank_ef_compress(batch, m, n, r, T, _bf16_ptr(x), _bf16_ptr(prev), _ptr(err),
                                        _ptr(Q0), _ptr(U), _ptr(V), _ptr(RU), _ptr(workspace),
                                        ws_bytes, _stream(stream)), "cfz_lowrank_ef_compress")


def cfz_lowrank_ef_compress_deferred(batch, m, n, r, T, pending, x, prev, err, Q0, U, V, RU,
                                     workspace, ws_bytes=None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check_lowrank(batch, m, n, r, None, Q0, U, V, RU)
    c = max(int(batch), 0) * max(int(m), 0) * max(int(n), 0)
    _need_dtype(err, _F32, "err")
    _need(x, 2 * c, "x")
    _need(prev, 2 * c, "prev")
    _need(err, 4 * c, "err")
    _need(workspace, ws_bytes, "workspace")
    _check(_lib.cfz_lowrank_ef_compress_deferred(batch, m, n, r, T, int(pending), _bf16_ptr(x),
                                                 _bf16_ptr(prev), _ptr(err), _ptr(Q0), _ptr(U),
                                                 _ptr(V), _ptr(RU), _ptr(workspace), ws_bytes,
                                                 _stream(stream)),
           "cfz_lowrank_ef_compress_deferred")


def cfz_lowrank_ef_flush(batch, m, n, r, U, V, RU, err, stream=None) -> None:
    _check_lowrank(batch, m, n, r, None, None, U, V, RU)
    c = max(int(batch), 0) * max(int(m), 0) * max(int(n), 0)
    _need_dtype(err, _F32, "err")
    _need(err, 4 * c, "err")
    _check(_lib.cfz_lowrank_ef_flush(batch, m, n, r, _ptr(U), _ptr(V), _ptr(RU), _ptr(err),
                                     _stream(stream)), "cfz_lowrank_ef_flush")


def cfz_lowrank_ef_decompress(batch, m, n, r, U, V, RU, base, xhat=None, stream=None) -> None:
    _check_lowrank(batch, m, n, r, None, None, U, V, RU)
    c = max(int(batch), 0) * max(int(m), 0) * max(int(n), 0)
    _need_dtype(base, _F32, "base")
    _need(base, 4 * c, "base")
    _need(xhat, 2 * c, "xhat")
    _check(_lib.cfz_lowrank_ef_decompress(batch, m, n, r, _ptr(U), _ptr(V), _ptr(RU), _ptr(base),
                                          _bf16_ptr(xhat), _stream(stream)),
           "cfz_lowrank_ef_decompress")


def cfz_stream_copy(src, dst, nbytes=None, stream=None) -> None:
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _need(src, nbytes, "src")
    _need(dst, nbytes, "dst")
    _check(_lib.cfz_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "cfz_stream_copy")


def cfz_stream_mix(src, src_bytes, dst, dst_bytes, stream=None) -> None:
    """Reads src_bytes of src and writes dst_bytes of dst, the writes spread evenly through
    the reads (a plain stream with a given read:write ratio)."""
    _need(src, src_bytes, "src")
    _need(dst, dst_bytes, "dst")
    _check(_lib.cfz_stream_mix(_ptr(src), src_bytes, _ptr(dst), dst_bytes, _stream(stream)),
           "cfz_stream_mix")


# ------------------------------------------------------------------ torch-owned state helpers

def _state_torch_dtype(state_bf16):
    return torch.bfloat16 if state_bf16 else torch.float32


class Sender:
    """A sender's codec state with its buffers held in torch device tensors.

    ``state_bf16`` keeps the carried error and the base in bf16 instead of fp32."""

    def __init__(self, rows, cols, bits=4, group=64, mode=CFZ_EF_DELTA, x0=None,
                 device="cuda", stream=None, state_bf16=False):
        self.desc = make_desc(rows, cols, bits, group, mode, CFZ_SENDER,
                              CFZ_STATE_BF16 if state_bf16 else CFZ_STATE_F32)
        n = rows * cols
        sdt = _state_torch_dtype(state_bf16)
        self.prev = torch.empty(n, dtype=torch.bfloat16, device=device) if mode == CFZ_EF_DELTA else None
        self.base = torch.empty(n, dtype=sdt, device=device) if mode != CFZ_EF_DELTA else None
        self.err = torch.empty(n, dtype=sdt, device=device) if mode != CFZ_EF_OFF else None
        self.codes = torch.empty(cfz_codes_bytes(self.desc), dtype=torch.uint8, device=device)
        self.scales = torch.empty(n // group, dtype=torch.float32, device=device)
        self.handle = cfz_state_create(self.desc, self.prev, self.base, self.err, x0, stream)

    def compress(self, x, codes=None, scales=None, stream=None):
        codes = self.codes if codes is None else codes
        scales = self.scales if scales is None else scales
        cfz_compress(self.handle, x, codes, scales, stream)
        return codes, scales

    def close(self):
        if self.handle:
            cfz_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Receiver:
    """A receiver's codec state (the running base) held in a torch device tensor."""

    def __init__(self, rows, cols, bits=4, group=64, x0=None, device="cuda", stream=None,
                 state_bf16=False):
        self.desc = make_desc(rows, cols, bits, group, CFZ_EF_DELTA, CFZ_RECEIVER,
                              CFZ_STATE_BF16 if state_bf16 else CFZ_STATE_F32)
        self.base = torch.empty(rows * cols, dtype=_state_torch_dtype(state_bf16), device=device)
        self.handle = cfz_state_create(self.desc, None, self.base, None, x0, stream)

    def decompress(self, codes, scales, xhat=None, stream=None):
        cfz_decompress(self.handle, codes, scales, xhat, stream)
        return xhat

    def close(self):
        if self.handle:
            cfz_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LowrankSender:
    """Sender of the rank-r compressor inside error feedback, for ``batch`` tensors of m x n:
    prev (bf16), err (fp32), the workspace and the payload (U, V, RU) in torch tensors.

    deferred=True: each step leaves its error update pending and the next step applies it inside
    its residual pass (same results, one pass over err fewer per step); err holds the carried
    error only after ``flush()``."""

    def __init__(self, batch, m, n, r, x0=None, device="cuda", stream=None, deferred=False):
        self.batch, self.m, self.n, self.r = batch, m, n, r
        self.deferred, self.pending = deferred, False
        count = batch * m * n
        self.prev = torch.empty(count, dtype=torch.bfloat16, device=device)
        self.err = torch.empty(count, dtype=torch.float32, device=device)
        self.ws = torch.empty(max(cfz_lowrank_ef_workspace_bytes(batch, m, n, r), 1),
                              dtype=torch.uint8, device=device)
        self.U = torch.empty((batch, m, r), dtype=torch.float32, device=device)
        self.V = torch.empty((batch, n, r), dtype=torch.float32, device=device)
        self.RU = torch.empty((batch, r, r), dtype=torch.float32, device=device)
        cfz_lowrank_ef_warmup(count, x0, self.prev, self.err, None, stream)

    def residual_bf16(self):
        """The bf16 residual A of the last step, left at the start of the workspace."""
        return self.ws[: self.batch * self.m * self.n * 2].view(torch.bfloat16)

    def compress(self, x, Q0, T, stream=None):
        if self.deferred:
            cfz_lowrank_ef_compress_deferred(self.batch, self.m, self.n, self.r, T, self.pending,
                                             x, self.prev, self.err, Q0, self.U, self.V, self.RU,
                                             self.ws, stream=stream)
            self.pending = True
        else:
            cfz_lowrank_ef_compress(self.batch, self.m, self.n, self.r, T, x, self.prev, self.err,
                                    Q0, self.U, self.V, self.RU, self.ws, stream=stream)
        return self.U, self.V, self.RU

    def flush(self, stream=None):
        """Applies a pending update, so that err holds the carried error."""
        if self.pending:
            cfz_lowrank_ef_flush(self.batch, self.m, self.n, self.r, self.U, self.V, self.RU,
                                 self.err, stream)
            self.pending = False


class LowrankReceiver:
    """Receiver of the rank-r compressor inside error feedback: the fp32 base."""

    def __init__(self, batch, m, n, r, x0=None, device="cuda", stream=None):
        self.batch, self.m, self.n, self.r = batch, m, n, r
        self.base = torch.empty(batch * m * n, dtype=torch.float32, device=device)
        cfz_lowrank_ef_warmup(batch * m * n, x0, None, None, self.base, stream)

    def decompress(self, U, V, RU, xhat=None, stream=None):
        cfz_lowrank_ef_decompress(self.batch, self.m, self.n, self.r, U, V, RU, self.base, xhat,
                                  stream)
        return xhat
