"""Python binding of libswm.so, the MI355X sparse-weight matmul library.

Argument marshalling only: every step of the product runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream; the
binding passes raw pointers, leading dimensions and the stream handle through
the C ABI declared in ``include/swm.h``.  There is no fallback: if the library
is not built or a call fails, an exception is raised.

Layout conventions (as in the C header): W is (M, K) fp16 row-major; X and Y
are token-major, X (N, K) and Y (N, M); Y = X @ (W * mask).T per token.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswm.so")

STATUS = {
    0: "SWM_OK", 1: "SWM_ERR_INVALID_ARG", 2: "SWM_ERR_SHAPE", 3: "SWM_ERR_ALIGN", 4: "SWM_ERR_OOM",
    5: "SWM_ERR_OVERFLOW", 6: "SWM_ERR_FORMAT", 7: "SWM_ERR_HIP", 8: "SWM_ERR_UNSUPPORTED",
}

# Every symbol include/swm.h declares, with its ctypes signature.
_i64, _u64, _i32, _sz, _vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p


SWM_CFG_SKIPPING = 1
SWM_CFG_SMFMAC = 2


class TileCfg(ctypes.Structure):
    _fields_ = [("tm", ctypes.c_int32), ("tk", ctypes.c_int32), ("flags", ctypes.c_int32)]


class FormatInfo(ctypes.Structure):
    _fields_ = [("m", _i64), ("k", _i64), ("tm", _i32), ("tk", _i32), ("mt", _i64), ("kt", _i64),
                ("nnz", _u64), ("padded_len", _u64), ("max_tile", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("bytes_header", _u64), ("bytes_tile_ptr", _u64),
                ("bytes_bits", _u64), ("bytes_values", _u64), ("bytes_total", _u64)]

    def as_dict(self):
        return {f[0]: getattr(self, f[0]) for f in self._fields_ if f[0] != "reserved"}


_PP = ctypes.POINTER(_vp)
SIGNATURES = {
    "swm_sparse_compress": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, ctypes.POINTER(TileCfg), _vp, _PP]),
    "swm_encode_blob": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, ctypes.POINTER(TileCfg), _vp, _sz,
                               ctypes.POINTER(_sz)]),
    "swm_format_export": (_i32, [_vp, _vp, _sz, ctypes.POINTER(_sz)]),
    "swm_format_import": (_i32, [_vp, _sz, _vp, _PP]),
    "swm_format_validate_blob": (_i32, [_vp, _sz]),
    "swm_format_query": (_i32, [_vp, ctypes.POINTER(FormatInfo)]),
    "swm_size_dry_run": (_i32, [_i64, _i64, _u64, ctypes.POINTER(TileCfg), ctypes.POINTER(FormatInfo)]),
    "swm_format_destroy": (_i32, [_vp]),
    "swm_decompress": (_i32, [_vp, _vp, _i64, _vp]),
    "swm_spmm": (_i32, [_vp, _vp, _i64, _vp, _i64, _i64, _vp]),
    "swm_spmm_workspace_bytes": (_sz, [_vp, _i64]),
    "swm_spmm_ws": (_i32, [_vp, _vp, _i64, _vp, _i64, _i64, _vp, _sz, _vp]),
    "swm_spmspv": (_i32, [_vp, _vp, _i64, _vp, _i64, _i32, _vp]),
    "swm_spmspv_noalloc": (_i32, [_vp, _vp, _i64, _vp, _i64, _i32, _vp]),
    "swm_spmspv_threshold": (_i32, [_vp, _vp, _i64, _vp, _i64, _i32, ctypes.c_float, _vp]),
    "swm_gate_up_silu": (_i32, [_vp, _vp, _vp, _i64, _vp, _i64, _i32, ctypes.c_float, _vp]),
    "swm_gate_up_silu_workspace_bytes": (_sz, [_vp, _vp, _i64]),
    "swm_gate_up_silu_ws": (_i32, [_vp, _vp, _vp, _i64, _vp, _i64, _i64, ctypes.c_float, _vp, _sz, _vp]),
    "swm_dense_gate_up_silu": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, ctypes.c_float, _vp]),
    "swm_format_enable_skipping": (_i32, [_vp, _vp, ctypes.POINTER(_u64)]),
    "swm_format_enable_smfmac": (_i32, [_vp, _vp, ctypes.POINTER(_u64)]),
    "swm_colruns_encode_blob": (_i32, [_vp, _sz, _vp, _sz, ctypes.POINTER(_sz)]),
    "swm_dense_gemm": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp]),
    "swm_hbm_stream": (_i32, [_vp, _sz, _i32, _i32, _vp, _vp]),
    "swm_status_str": (ctypes.c_char_p, [_i32]),
    "swm_last_hip_error": (_i32, []),
    "swm_version": (_i32, []),
}

_lib = None


class SwmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = STATUS.get(code, str(code))
        if code == 7 and _lib is not None:
            msg += f" (hipError {_lib.swm_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def load():
    """Load libswm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run python -m sparse_weight_matmul_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int, where: str):
    if code != 0:
        raise SwmError(code, where)


def _cfg(tile, flags=0):
    if tile is None and not flags:
        return None
    tm, tk = tile if tile is not None else (16, 64)
    c = TileCfg(int(tm), int(tk), int(flags))
    return ctypes.byref(c)


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _host_u16(W):
    a = W.detach().cpu().numpy() if hasattr(W, "detach") else np.asarray(W)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16 or a.ndim != 2:
        raise TypeError("W must be a 2-D fp16 (or uint16 bit-pattern) array")
    return np.ascontiguousarray(a)


def _host_mask(mask, shape):
    if mask is None:
        return None
    m = mask.detach().cpu().numpy() if hasattr(mask, "detach") else np.asarray(mask)
    if m.shape != shape:
        raise ValueError("mask shape mismatch")
    return np.ascontiguousarray(m.astype(np.uint8))


def _dev2d(t, name, rows=None, cols=None):
    """(pointer, leading dimension) of a 2-D fp16 CUDA tensor with unit column stride."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float16 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float16 CUDA tensor")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    if rows is not None and t.shape[0] != rows:
        raise ValueError(f"{name} has {t.shape[0]} rows, expected {rows}")
    if cols is not None and t.shape[1] != cols:
        raise ValueError(f"{name} has {t.shape[1]} columns, expected {cols}")
    return ctypes.c_void_p(t.data_ptr()), max(int(t.stride(0)), int(t.shape[1]), 1)


class Format:
    """A compressed weight resident on the current device (owns its memory)."""

    def __init__(self, handle: ctypes.c_void_p):
        self._h = handle
        self.info = self.query()

    @property
    def M(self):
        return self.info["m"]

    @property
    def K(self):
        return self.info["k"]

    def query(self) -> dict:
        lib = load()
        inf = FormatInfo()
        _check(lib.swm_format_query(self._h, ctypes.byref(inf)), "swm_format_query")
        return inf.as_dict()

    def export(self) -> bytes:
        lib = load()
        size = ctypes.c_size_t(0)
        _check(lib.swm_format_export(self._h, None, 0, ctypes.byref(size)), "swm_format_export")
        buf = ctypes.create_string_buffer(size.value)
        _check(lib.swm_format_export(self._h, buf, size.value, ctypes.byref(size)), "swm_format_export")
        return buf.raw[:size.value]

    def enable_skipping(self, stream=None) -> int:
        """Attach the column-run encoding used by spmspv for n <= 4; returns its bytes."""
        lib = load()
        nbytes = _u64(0)
        _check(lib.swm_format_enable_skipping(self._h, _stream_ptr(stream), ctypes.byref(nbytes)),
               "swm_format_enable_skipping")
        return int(nbytes.value)

    def enable_smfmac(self, stream=None) -> int:
        """Attach the 2:4 layers of the sparse-matrix-core prefill route; returns their bytes."""
        lib = load()
        nbytes = _u64(0)
        _check(lib.swm_format_enable_smfmac(self._h, _stream_ptr(stream), ctypes.byref(nbytes)),
               "swm_format_enable_smfmac")
        return int(nbytes.value)

    def close(self):
        if self._h:
            load().swm_format_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sparse_compress(W, mask=None, tile=(16, 64), stream=None, skipping=False, smfmac=False) -> Format:
    """Compress a host fp16 W (M, K) with an optional host mask; upload to the
    current device.  skipping=True also builds the column-run encoding that
    lets spmspv skip zero activations (SWM_CFG_SKIPPING); smfmac=True also
    keeps W compacted into 2:4 layers, which spmm and spmm_ws multiply on the
    sparse matrix cores at prefill token counts (SWM_CFG_SMFMAC)."""
    lib = load()
    w = _host_u16(W)
    m = _host_mask(mask, w.shape)
    h = ctypes.c_void_p()
    code = lib.swm_sparse_compress(w.ctypes.data, w.shape[1], None if m is None else m.ctypes.data,
                                   w.shape[1], w.shape[0], w.shape[1],
                                   _cfg(tile, (SWM_CFG_SKIPPING if skipping else 0) | (SWM_CFG_SMFMAC if smfmac else 0)),
                                   _stream_ptr(stream),
                                   ctypes.byref(h))
    _check(code, "swm_sparse_compress")
    return Format(h)


def encode_blob(W, mask=None, tile=(16, 64)) -> bytes:
    """Host-only encoder: the export blob of compress(W, mask) without any GPU."""
    lib = load()
    w = _host_u16(W)
    m = _host_mask(mask, w.shape)
    mp = None if m is None else m.ctypes.data
    size = ctypes.c_size_t(0)
    _check(lib.swm_encode_blob(w.ctypes.data, w.shape[1], mp, w.shape[1], w.shape[0], w.shape[1],
                               _cfg(tile), None, 0, ctypes.byref(size)), "swm_encode_blob")
    buf = ctypes.create_string_buffer(max(size.value, 1))
    _check(lib.swm_encode_blob(w.ctypes.data, w.shape[1], mp, w.shape[1], w.shape[0], w.shape[1],
                               _cfg(tile), buf, size.value, ctypes.byref(size)), "swm_encode_blob")
    return buf.raw[:size.value]


def colruns_encode_blob(tcb_blob: bytes) -> bytes:
    """Host-only: the SWM-CR v2 column-run blob derived from a SWM-TCB v2 blob."""
    lib = load()
    b = ctypes.create_string_buffer(bytes(tcb_blob), max(len(tcb_blob), 1))
    size = ctypes.c_size_t(0)
    _check(lib.swm_colruns_encode_blob(b, len(tcb_blob), None, 0, ctypes.byref(size)), "swm_colruns_encode_blob")
    out = ctypes.create_string_buffer(max(size.value, 1))
    _check(lib.swm_colruns_encode_blob(b, len(tcb_blob), out, size.value, ctypes.byref(size)),
           "swm_colruns_encode_blob")
    return out.raw[:size.value]


def validate_blob(blob: bytes) -> int:
    """Status code of the library's blob validator (0 = valid)."""
    lib = load()
    b = ctypes.create_string_buffer(bytes(blob), max(len(blob), 1))
    return int(lib.swm_format_validate_blob(b, len(blob)))


def format_import(blob: bytes, stream=None) -> Format:
    lib = load()
    b = ctypes.create_string_buffer(bytes(blob), max(len(blob), 1))
    h = ctypes.c_void_p()
    _check(lib.swm_format_import(b, len(blob), _stream_ptr(stream), ctypes.byref(h)), "swm_format_import")
    return Format(h)


def size_dry_run(M: int, K: int, nnz: int, tile=(16, 64)) -> dict:
    lib = load()
    inf = FormatInfo()
    _check(lib.swm_size_dry_run(M, K, nnz, _cfg(tile), ctypes.byref(inf)), "swm_size_dry_run")
    return inf.as_dict()


def size_dry_run_status(M: int, K: int, nnz: int, tile=(16, 64)) -> int:
    lib = load()
    inf = FormatInfo()
    return int(lib.swm_size_dry_run(M, K, nnz, _cfg(tile), ctypes.byref(inf)))


def _out(Y, N, M, like):
    import torch
    if Y is None:
        Y = torch.empty((N, M), dtype=torch.float16, device=like.device)
    return Y


def spmm(fmt: Format, X, Y=None, stream=None):
    """Y (N, M) = X (N, K) @ (W * mask).T on the device."""
    lib = load()
    N = X.shape[0]
    xp, ldx = _dev2d(X, "X", cols=fmt.K)
    Y = _out(Y, N, fmt.M, X)
    yp, ldy = _dev2d(Y, "Y", rows=N, cols=fmt.M)
    _check(lib.swm_spmm(fmt._h, xp, ldx, yp, ldy, N, _stream_ptr(stream)), "swm_spmm")
    return Y


def spmm_workspace_bytes(fmt: Format, N: int) -> int:
    """Device workspace bytes spmm(..., workspace=) uses for N tokens (0: none)."""
    return int(load().swm_spmm_workspace_bytes(fmt._h, int(N)))


def spmm_ws(fmt: Format, X, workspace, Y=None, stream=None):
    """spmm with a caller-owned device workspace (a CUDA uint8 tensor of at
    least spmm_workspace_bytes(fmt, N) bytes, or None): for large N the library
    expands W into it once and runs its dense MFMA kernel.  Same result."""
    lib = load()
    N = X.shape[0]
    xp, ldx = _dev2d(X, "X", cols=fmt.K)
    Y = _out(Y, N, fmt.M, X)
    yp, ldy = _dev2d(Y, "Y", rows=N, cols=fmt.M)
    if workspace is None:
        wp, wb = None, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor")
        wp, wb = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    _check(lib.swm_spmm_ws(fmt._h, xp, ldx, yp, ldy, N, wp, wb, _stream_ptr(stream)), "swm_spmm_ws")
    return Y


def gate_up_silu(gate: Format, up: Format, X, tau: float = 0.0, H=None, stream=None):
    """Gated FFN hidden activation for 1..32 decode tokens: H (n, M) =
    SiLU(X @ W_g.T) * (X @ W_u.T), entries with |H| < tau stored as +0."""
    lib = load()
    n = X.shape[0]
    xp, ldx = _dev2d(X, "X", cols=gate.K)
    H = _out(H, n, gate.M, X)
    hp, ldh = _dev2d(H, "H", rows=n, cols=gate.M)
    _check(lib.swm_gate_up_silu(gate._h, up._h, xp, ldx, hp, ldh, n, float(tau), _stream_ptr(stream)),
           "swm_gate_up_silu")
    return H


def gate_up_silu_workspace_bytes(gate: Format, up: Format, n: int) -> int:
    """Device workspace bytes gate_up_silu_ws uses for n tokens (0: none)."""
    return int(load().swm_gate_up_silu_workspace_bytes(gate._h, up._h, int(n)))


def gate_up_silu_ws(gate: Format, up: Format, X, workspace, tau: float = 0.0, H=None, stream=None):
    """gate_up_silu for any token count: from 33 tokens the gate and up
    weights are expanded into `workspace` (a contiguous CUDA uint8 tensor of at
    least gate_up_silu_workspace_bytes(gate, up, n) bytes; None below 33
    tokens) and one dense MFMA product forms H with the gated epilogue."""
    lib = load()
    n = X.shape[0]
    xp, ldx = _dev2d(X, "X", cols=gate.K)
    H = _out(H, n, gate.M, X)
    hp, ldh = _dev2d(H, "H", rows=n, cols=gate.M)
    if workspace is None:
        wp, wb = None, 0
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor")
        wp, wb = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    _check(lib.swm_gate_up_silu_ws(gate._h, up._h, xp, ldx, hp, ldh, n, float(tau), wp, wb, _stream_ptr(stream)),
           "swm_gate_up_silu_ws")
    return H


def dense_gate_up_silu(W2, X, tau: float = 0.0, H=None, stream=None):
    """Dense gated FFN step: W2 (2M, K) holds the gate and up weights
    interleaved by row (2m: gate row m, 2m+1: up row m); H (N, M) =
    SiLU(X @ Wg.T) * (X @ Wu.T), |H| < tau stored as +0."""
    lib = load()
    N = X.shape[0]
    if W2.shape[0] % 2:
        raise ValueError("W2 must hold an even number of rows (gate / up interleaved)")
    M, K = W2.shape[0] // 2, W2.shape[1]
    wp, ldw = _dev2d(W2, "W2", cols=K)
    xp, ldx = _dev2d(X, "X", cols=K)
    H = _out(H, N, M, X)
    hp, ldh = _dev2d(H, "H", rows=N, cols=M)
    _check(lib.swm_dense_gate_up_silu(wp, ldw, xp, ldx, hp, ldh, M, K, N, float(tau), _stream_ptr(stream)),
           "swm_dense_gate_up_silu")
    return H


def spmspv(fmt: Format, x, y=None, stream=None):
    """Zero-activation-skipping product for 1..16 tokens; x (n, K), y (n, M).
    Skips on the column-run encoding for n <= 2 when the handle carries it."""
    lib = load()
    n = x.shape[0]
    xp, ldx = _dev2d(x, "x", cols=fmt.K)
    y = _out(y, n, fmt.M, x)
    yp, ldy = _dev2d(y, "y", rows=n, cols=fmt.M)
    _check(lib.swm_spmspv(fmt._h, xp, ldx, yp, ldy, n, _stream_ptr(stream)), "swm_spmspv")
    return y


def spmspv_noalloc(fmt: Format, x, y=None, stream=None):
    """spmspv whose skipping path keeps its partial sums in the library's fixed
    device array (no allocation inside the call); same result, bitwise."""
    lib = load()
    n = x.shape[0]
    xp, ldx = _dev2d(x, "x", cols=fmt.K)
    y = _out(y, n, fmt.M, x)
    yp, ldy = _dev2d(y, "y", rows=n, cols=fmt.M)
    _check(lib.swm_spmspv_noalloc(fmt._h, xp, ldx, yp, ldy, n, _stream_ptr(stream)), "swm_spmspv_noalloc")
    return y


def spmspv_threshold(fmt: Format, x, tau: float, y=None, stream=None):
    """spmspv with activations |x| < tau counted as zero (skipping must be enabled, n <= 4)."""
    lib = load()
    n = x.shape[0]
    xp, ldx = _dev2d(x, "x", cols=fmt.K)
    y = _out(y, n, fmt.M, x)
    yp, ldy = _dev2d(y, "y", rows=n, cols=fmt.M)
    _check(lib.swm_spmspv_threshold(fmt._h, xp, ldx, yp, ldy, n, float(tau), _stream_ptr(stream)),
           "swm_spmspv_threshold")
    return y


def dense_gemm(W, X, Y=None, stream=None):
    """In-house dense baseline: Y (N, M) = X (N, K) @ W.T with dense fp16 W (M, K) on the device."""
    lib = load()
    M, K = W.shape
    N = X.shape[0]
    wp, ldw = _dev2d(W, "W")
    xp, ldx = _dev2d(X, "X", cols=K)
    Y = _out(Y, N, M, X)
    yp, ldy = _dev2d(Y, "Y", rows=N, cols=M)
    _check(lib.swm_dense_gemm(wp, ldw, xp, ldx, yp, ldy, M, K, N, _stream_ptr(stream)), "swm_dense_gemm")
    return Y


def decompress(fmt: Format, W=None, stream=None):
    """Dense fp16 W * mask (M, K) on the device, expanded by the library's kernel."""
    import torch
    lib = load()
    if W is None:
        W = torch.empty((fmt.M, fmt.K), dtype=torch.float16, device="cuda")
    wp, ldw = _dev2d(W, "W", rows=fmt.M, cols=fmt.K)
    _check(lib.swm_decompress(fmt._h, wp, ldw, _stream_ptr(stream)), "swm_decompress")
    return W


def hbm_stream(buf, unroll: int, blocks: int, out=None, stream=None):
    """Calibration read of a whole CUDA tensor `buf` (bytes a multiple of 16)."""
    import torch
    lib = load()
    if out is None:
        out = torch.empty(blocks * 4, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib.swm_hbm_stream(ctypes.c_void_p(buf.data_ptr()), nbytes, unroll, blocks,
                              ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)), "swm_hbm_stream")
    return out


def status_str(code: int) -> str:
    return load().swm_status_str(code).decode()


def version() -> int:
    return int(load().swm_version())
