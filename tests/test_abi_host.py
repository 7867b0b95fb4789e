"""Host-side checks of the C-ABI library (no GPU needed).

* the shared library loads and exports every function include/swm.h declares;
* the C++ encoder writes the same bytes as the independent numpy encoder;
* the validator rejects corrupted blobs;
* size accounting and overflow detection of the dry run;
* the library's column-run encoding (activation skipping) is byte-identical to
  the independent numpy encoder's.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import sparse_weight_matmul_amd as swm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "swm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = swm.load()
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
        assert n in swm.SIGNATURES, n
    assert swm.version() >= 100
    assert swm.status_str(0) == "ok"
    assert swm.status_str(6) == "invalid format"


def _case(seed, M, K, density, signed_zero=True):
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((M, K))).astype(np.float16)
    if signed_zero:
        W[g.random((M, K)) < 0.05] = np.float16(-0.0)
        W[g.random((M, K)) < 0.05] = np.float16(0.0)
    mask = g.random((M, K)) < density
    return W, mask


@pytest.mark.parametrize("M,K,tile,density", [
    (1, 1, (16, 64), 1.0), (3, 10, (16, 32), 0.5), (64, 64, (16, 64), 0.5), (100, 70, (16, 64), 0.5),
    (130, 300, (16, 96), 0.3), (65, 257, (16, 256), 0.01), (200, 40, (16, 32), 0.99),
    (256, 512, (16, 64), 0.0), (257, 129, (16, 128), 1.0), (17, 65, (16, 64), 0.5),
])
def test_cpp_encoder_matches_numpy_encoder_bytes(M, K, tile, density):
    W, mask = _case(M * 7 + K, M, K, density)
    a = swm.encode_blob(W, mask, tile=tile)
    b = oracle.tcb_encode(W, mask, TK=tile[1]).blob()
    assert a == b
    assert swm.validate_blob(a) == 0


def test_cpp_encoder_null_mask_matches():
    W, _ = _case(5, 90, 77, 1.0)
    a = swm.encode_blob(W, None)
    b = oracle.tcb_encode(W, None).blob()
    assert a == b


def test_cpp_encoder_tiny_workload_bytes():
    import swm_workloads as wl
    W, mask, _ = wl.tiny()
    assert swm.encode_blob(W, mask) == oracle.tcb_encode(W, mask).blob()


def _corrupt(blob: bytes, off: int, value: bytes) -> bytes:
    b = bytearray(blob)
    b[off:off + len(value)] = value
    return bytes(b)


def test_validator_rejects_corruption():
    W, mask = _case(1, 100, 130, 0.5)
    blob = swm.encode_blob(W, mask)
    f = oracle.tcb_parse(blob)
    T = f.Mt * f.Kt
    nW = f.TK // 4
    off_tp = 64
    off_bits = off_tp + 4 * (T + 1)
    off_vals = off_bits + 8 * T * nW
    assert swm.validate_blob(blob) == 0
    bad = {
        "magic": _corrupt(blob, 0, b"XXXX"),
        "version": _corrupt(blob, 4, (3).to_bytes(4, "little")),
        "reserved": _corrupt(blob, 60, (1).to_bytes(4, "little")),
        "truncated": blob[:-2],
        "extra": blob + b"\0\0",
        "nnz": _corrupt(blob, 32, (f.nnz + 1).to_bytes(8, "little")),
        "max_tile": _corrupt(blob, 56, (f.max_tile + 8).to_bytes(4, "little")),
        "tile_ptr_nonmonotone": _corrupt(blob, off_tp + 4, (int(f.tile_ptr[2]) + 8).to_bytes(4, "little")),
        # 100 rows: the last slab (rows 96..111) has 4 valid rows; bit 5 of any word is row 5
        "bit_beyond_M": _corrupt(blob, off_bits + 8 * (((f.Mt - 1) * f.Kt) * nW + 3), (1 << 5).to_bytes(8, "little")),
        # 130 columns: the last tile column starts at 128; its word 15 (step 1, e = 7) is column 128+39
        "bit_beyond_K": _corrupt(blob, off_bits + 8 * ((f.Kt - 1) * nW + 15), (1).to_bytes(8, "little")),
        "popcount_mismatch": _corrupt(blob, off_bits, (int(f.bits[0]) ^ 1).to_bytes(8, "little")),
    }
    # nonzero padding: find a tile whose run has padding
    lens = np.diff(f.tile_ptr.astype(np.int64))
    pcs = np.array([bin(int(x)).count("1") for x in f.bits]).reshape(T, nW).sum(1)
    t = int(np.nonzero(lens > pcs)[0][0])
    bad["padding"] = _corrupt(blob, off_vals + 2 * (int(f.tile_ptr[t + 1]) - 1), b"\x01\x00")
    for name, b in bad.items():
        assert swm.validate_blob(b) == 6, name


def test_dry_run_sizes_and_overflow():
    info = swm.size_dry_run(4096, 4096, 4096 * 2048)
    assert info["mt"] == 256 and info["kt"] == 64
    assert info["bytes_bits"] == 256 * 64 * 16 * 8
    assert info["padded_len"] == 4096 * 2048 + 256 * 64 * 7
    assert info["bytes_total"] == 64 + 4 * (256 * 64 + 1) + info["bytes_bits"] + 2 * info["padded_len"]
    assert swm.size_dry_run_status(1 << 20, 1 << 20, 1 << 33) == 5  # padded length >= 2^32
    assert swm.size_dry_run_status(10, 10, 101) == 1  # nnz > M*K
    assert swm.size_dry_run_status(-1, 10, 0) == 1
    assert swm.size_dry_run_status(64, 64, 0, tile=(32, 64)) == 1  # tm must be 16
    assert swm.size_dry_run_status(64, 64, 0, tile=(16, 48)) == 1  # tk not a multiple of 32


def test_dry_run_bounds_the_real_format():
    W, mask = _case(3, 300, 200, 0.5)
    info = swm.size_dry_run(300, 200, int(mask.sum()))
    f = oracle.tcb_encode(W, mask)
    assert f.padded_len <= info["padded_len"]
    assert len(f.blob()) <= info["bytes_total"]


def test_encoder_rejects_bad_arguments():
    lib = swm.load()
    size = ctypes.c_size_t(0)
    W = np.zeros((4, 4), dtype=np.uint16)
    # ldw < K
    assert lib.swm_encode_blob(W.ctypes.data, 3, None, 4, 4, 4, None, None, 0, ctypes.byref(size)) == 1
    # null W with a non-empty shape
    assert lib.swm_encode_blob(None, 4, None, 4, 4, 4, None, None, 0, ctypes.byref(size)) == 1
    # null size pointer
    assert lib.swm_encode_blob(W.ctypes.data, 4, None, 4, 4, 4, None, None, 0, None) == 1
    # bad tile shape
    cfg = swm.TileCfg(16, 12)
    assert lib.swm_encode_blob(W.ctypes.data, 4, None, 4, 4, 4, ctypes.byref(cfg), None, 0, ctypes.byref(size)) == 1
    # empty matrix is fine
    assert lib.swm_encode_blob(None, 0, None, 0, 0, 0, None, None, 0, ctypes.byref(size)) == 0
    assert size.value == 64 + 4


def test_compress_rejects_unknown_flags():
    # flag bits other than SWM_CFG_SKIPPING and SWM_CFG_SMFMAC are refused before any encoding or upload
    lib = swm.load()
    W = np.ones((4, 4), dtype=np.float16)
    h = ctypes.c_void_p()
    cfg = swm.TileCfg(16, 64, 4)
    assert lib.swm_sparse_compress(W.ctypes.data, 4, None, 4, 4, 4, ctypes.byref(cfg), None, ctypes.byref(h)) == 1
    assert not h.value


def test_null_handle_calls_are_rejected():
    lib = swm.load()
    inf = swm.FormatInfo()
    assert lib.swm_format_query(None, ctypes.byref(inf)) == 1
    assert lib.swm_spmm(None, None, 1, None, 1, 1, None) == 1
    assert lib.swm_spmspv(None, None, 1, None, 1, 1, None) == 1
    assert lib.swm_spmspv_noalloc(None, None, 1, None, 1, 1, None) == 1
    assert lib.swm_dense_gemm(None, 1, None, 1, None, 1, 1, 1, 1, None) == 1
    assert lib.swm_decompress(None, None, 1, None) == 1
    assert lib.swm_spmm_ws(None, None, 1, None, 1, 1024, None, 0, None) == 1
    assert lib.swm_spmm_workspace_bytes(None, 4096) == 0
    assert lib.swm_gate_up_silu(None, None, None, 1, None, 1, 1, 0.0, None) == 1
    assert lib.swm_gate_up_silu_ws(None, None, None, 1, None, 1, 4096, 0.0, None, 0, None) == 1
    assert lib.swm_gate_up_silu_workspace_bytes(None, None, 4096) == 0
    assert lib.swm_dense_gate_up_silu(None, 8, None, 8, None, 8, 8, 8, 64, 0.0, None) == 1
    assert lib.swm_format_destroy(None) == 0
    assert lib.swm_format_validate_blob(None, 0) == 1


@pytest.mark.parametrize("M,K,density,null_mask", [
    (1, 1, 1.0, False), (3, 10, 0.5, False), (256, 64, 0.5, False), (257, 70, 0.3, False),
    (300, 513, 0.5, True), (600, 40, 0.0, False), (513, 130, 1.0, False), (64, 700, 0.05, False),
])
def test_colruns_encoder_matches_numpy_encoder_bytes(M, K, density, null_mask):
    W, mask = _case(M * 11 + K, M, K, density)
    tcb = swm.encode_blob(W, None if null_mask else mask)
    got = swm.colruns_encode_blob(tcb)
    exp = oracle.colruns_encode(W, None if null_mask else mask).blob()
    assert got == exp


def test_colruns_encoder_rejects_bad_input():
    lib = swm.load()
    W, mask = _case(1, 40, 40, 0.5)
    tcb = bytearray(swm.encode_blob(W, mask))
    size = ctypes.c_size_t(0)
    b = ctypes.create_string_buffer(bytes(tcb), len(tcb))
    assert lib.swm_colruns_encode_blob(b, len(tcb), None, 0, ctypes.byref(size)) == 0 and size.value > 32
    small = ctypes.create_string_buffer(size.value - 1)
    assert lib.swm_colruns_encode_blob(b, len(tcb), small, size.value - 1, ctypes.byref(size)) == 1
    assert lib.swm_colruns_encode_blob(None, 0, None, 0, ctypes.byref(size)) == 1
    assert lib.swm_colruns_encode_blob(b, len(tcb), None, 0, None) == 1
    tcb[0] ^= 0xFF  # bad magic: the validator's status comes back
    bad = ctypes.create_string_buffer(bytes(tcb), len(tcb))
    assert lib.swm_colruns_encode_blob(bad, len(tcb), None, 0, ctypes.byref(size)) == 6
    assert lib.swm_format_enable_skipping(None, None, None) == 1
    assert lib.swm_format_enable_smfmac(None, None, None) == 1
