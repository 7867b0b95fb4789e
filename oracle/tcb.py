"""Independent numpy encoder / decoder of the SWM-TCB v2 format (test infra only).

The pages name a "Tiled-Column-wise Bitmap Compressed" (Tiled-CBC) format for
the static sparse weights ("Unified Static-Dynamic Pruning for Efficient LLM
Inference", abstract) but do not give its layout.  SWM-TCB v2 is this project's
reading: tiles of 16 rows x TK columns; every tile column has a 16-bit bitmap
(one bit of position metadata per entry, the low-metadata goal of
"Accelerating GPU inference of LLMs with moderately unstructured sparse weight
matrices", Sec. 3.1 and Challenge 2 of Sec. 1); the kept fp16 values are packed
column by column, so each column's values form one contiguous run.

Spec (written out here from the definition, not from the GPU library):
  1. TM = 16.  Tile grid Mt = ceil(M/16), Kt = ceil(K/TK), TK a multiple of 32.
     Tile t = i*Kt + j covers rows [16i, 16i+16) and columns [TK*j, TK*j+TK);
     tiles are stored in increasing t.
  2. Column bitmaps are stored four to a 64-bit word.  A tile has TK/32 steps
     of 32 columns and each step 8 words; word w = 8*s + e of the tile holds,
     in bits 16q .. 16q+15, the bitmap of column 32*s + 8*q + e (q = 0..3):
     bit b (LSB = 0) of the word is 1 iff position
         (row 16*i + b % 16,  column TK*j + 32*s + 8*(b // 16) + e)
     is kept.  Rows >= M and columns >= K are never kept.
  3. values: the raw fp16 bits of every kept entry of tile t, word by word
     (w = 0, 1, ...) and inside a word by increasing bit b -- i.e. column by
     column, each column's kept rows in increasing order; each tile's run is
     padded with 0x0000 to a multiple of 8 values.
  4. tile_ptr: uint32[Mt*Kt + 1], exclusive prefix of padded run lengths (in
     values); the total must stay below 2**32.
  5. Header, 64 bytes little-endian: b"SWMT", u32 version=2, i64 M, i64 K,
     u32 TM=16, u32 TK, u64 nnz (unpadded), u64 padded length, u32 Mt, u32 Kt,
     u32 largest padded tile run, u32 reserved=0.
  6. Export blob = header || tile_ptr || bits || values, no gaps.
A null mask keeps exactly the entries whose value is not +0 or -0.  A kept
entry equal to +-0 is stored with its bits; a pruned entry decodes to +0.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

import numpy as np

MAGIC = b"SWMT"
VERSION = 2
TM = 16
HEADER_BYTES = 64
_HDR = struct.Struct("<4sIqqIIQQIIII")
assert _HDR.size == HEADER_BYTES


@dataclass
class TcbFormat:
    M: int
    K: int
    TM: int
    TK: int
    nnz: int
    padded_len: int
    Mt: int
    Kt: int
    max_tile: int
    tile_ptr: np.ndarray  # uint32
    bits: np.ndarray      # uint64
    values: np.ndarray    # uint16

    def header(self) -> bytes:
        return _HDR.pack(MAGIC, VERSION, self.M, self.K, self.TM, self.TK, self.nnz,
                         self.padded_len, self.Mt, self.Kt, self.max_tile, 0)

    def blob(self) -> bytes:
        return (self.header() + self.tile_ptr.astype("<u4").tobytes()
                + self.bits.astype("<u8").tobytes() + self.values.astype("<u2").tobytes())


def _bit_positions(TK: int):
    """(row, column) inside a tile of every (word, bit) pair, in storage order."""
    W = TK // 4
    w = np.arange(W)[:, None]
    b = np.arange(64)[None, :]
    s, e = w // 8, w % 8
    rows = np.broadcast_to(b % 16, (W, 64))
    cols = 32 * s + 8 * (b // 16) + e
    return rows, cols


def tcb_encode(W: np.ndarray, mask: np.ndarray | None, TK: int = 64) -> TcbFormat:
    W = np.asarray(W, dtype=np.float16)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    M, K = W.shape
    if TK <= 0 or TK % 32:
        raise ValueError("TK must be a positive multiple of 32")
    wbits = W.view(np.uint16)
    if mask is None:
        keep = (wbits & np.uint16(0x7FFF)) != 0
    else:
        keep = np.asarray(mask, dtype=bool)
        if keep.shape != (M, K):
            raise ValueError("mask shape mismatch")
    Mt, Kt = -(-M // TM), -(-K // TK)
    kp = np.zeros((Mt * TM, Kt * TK), dtype=bool)
    kp[:M, :K] = keep
    vp = np.zeros((Mt * TM, Kt * TK), dtype=np.uint16)
    vp[:M, :K] = wbits
    rows, cols = _bit_positions(TK)
    nW = TK // 4
    weights = (np.uint64(1) << np.arange(64, dtype=np.uint64))[None, :]
    bits = np.zeros(Mt * Kt * nW, dtype=np.uint64)
    tile_ptr = np.zeros(Mt * Kt + 1, dtype=np.uint64)
    runs = []
    for i in range(Mt):
        for j in range(Kt):
            t = i * Kt + j
            kt = kp[i * TM:(i + 1) * TM, j * TK:(j + 1) * TK]
            vt = vp[i * TM:(i + 1) * TM, j * TK:(j + 1) * TK]
            kb = kt[rows, cols]  # (nW, 64) in storage order
            bits[t * nW:(t + 1) * nW] = (kb.astype(np.uint64) * weights).sum(axis=1, dtype=np.uint64)
            run = vt[rows, cols][kb]
            pad = (-run.size) % 8
            if pad:
                run = np.concatenate([run, np.zeros(pad, dtype=np.uint16)])
            runs.append(run)
            tile_ptr[t + 1] = tile_ptr[t] + run.size
    total = int(tile_ptr[-1])
    if total >= 2 ** 32:
        raise OverflowError("padded value count does not fit in 32 bits")
    values = np.concatenate(runs) if runs else np.zeros(0, dtype=np.uint16)
    lens = np.diff(tile_ptr)
    return TcbFormat(M=M, K=K, TM=TM, TK=TK, nnz=int(keep.sum()), padded_len=total,
                     Mt=Mt, Kt=Kt, max_tile=int(lens.max()) if lens.size else 0,
                     tile_ptr=tile_ptr.astype(np.uint32), bits=bits, values=values)


def tcb_parse(blob: bytes) -> TcbFormat:
    """Parse an export blob back into arrays (raises ValueError on bad input)."""
    if len(blob) < HEADER_BYTES:
        raise ValueError("blob shorter than header")
    magic, ver, M, K, tm, TK, nnz, plen, Mt, Kt, mx, _ = _HDR.unpack_from(blob, 0)
    if magic != MAGIC or ver != VERSION or tm != TM:
        raise ValueError("bad magic, version or tile height")
    T = Mt * Kt
    nW = TK // 4
    off = HEADER_BYTES
    tp = np.frombuffer(blob, dtype="<u4", count=T + 1, offset=off); off += 4 * (T + 1)
    bits = np.frombuffer(blob, dtype="<u8", count=T * nW, offset=off); off += 8 * T * nW
    vals = np.frombuffer(blob, dtype="<u2", count=plen, offset=off); off += 2 * plen
    if off != len(blob):
        raise ValueError("blob length mismatch")
    return TcbFormat(M=M, K=K, TM=tm, TK=TK, nnz=nnz, padded_len=plen, Mt=Mt, Kt=Kt,
                     max_tile=mx, tile_ptr=tp.copy(), bits=bits.copy(), values=vals.copy())


def tcb_decode(fmt: TcbFormat) -> np.ndarray:
    """Dense fp16 bits (uint16, M x K) of W (.) mask; pruned entries are 0x0000."""
    M, K, TK, Mt, Kt = fmt.M, fmt.K, fmt.TK, fmt.Mt, fmt.Kt
    nW = TK // 4
    rows, cols = _bit_positions(TK)
    out = np.zeros((Mt * TM, Kt * TK), dtype=np.uint16)
    shifts = np.arange(64, dtype=np.uint64)[None, :]
    for t in range(Mt * Kt):
        i, j = divmod(t, Kt)
        words = fmt.bits[t * nW:(t + 1) * nW][:, None]
        kb = ((words >> shifts) & np.uint64(1)).astype(bool)  # (nW, 64)
        n = int(kb.sum())
        run = fmt.values[int(fmt.tile_ptr[t]):int(fmt.tile_ptr[t]) + n]
        tile = np.zeros((TM, TK), dtype=np.uint16)
        tile[rows[kb], cols[kb]] = run
        out[i * TM:(i + 1) * TM, j * TK:(j + 1) * TK] = tile
    return out[:M, :K]
