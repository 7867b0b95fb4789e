"""Independent numpy encoder / decoder of the SWM-CR v2 column-run encoding
(test infrastructure only).

The decode kernel of "Unified Static-Dynamic Pruning for Efficient LLM
Inference" (SPDP, abstract) skips, at run time, the input channels whose
activation is zero.  "Reduced Matrix Multiplication" (blog page, Sec. 4.2)
states why this is exact: a channel whose activation is zero contributes only
zero terms, so the product over the kept channels equals the full product.
Skipping can only save memory traffic when the weights of one input channel
(one column of W) lie together in memory over many rows.  SWM-CR v2 is this
project's layout for that purpose: the same kept entries as the tiled format,
regrouped column by column inside blocks of 256 rows, with the blocks of one
column stored four at a time.

Spec (written out here from the definition, not from the GPU library):
  1. R = 256.  Row blocks b = 0 .. Mb-1, Mb = ceil(M / R); block b covers
     rows [R b, R b + R).  Blocks form groups of G = 4: block b = G g + j,
     j = 0 .. 3, and there are Gn = ceil(Mb / G) groups.  Entry
     e = (g K + k) G + j is column k inside block b; E = Gn K G entries.
     Entries of blocks b >= Mb (the last group's missing blocks) are empty.
  2. bits: uint64[E 4].  Word q of entry e has bit i set iff position
     (row R b + 64 q + i, column k) is kept.  Rows >= M are never kept.
  3. values: for every entry in increasing e, the raw fp16 bits of the kept
     entries of that column inside that block, in increasing row order,
     padded with 0x0000 to a multiple of 4 values.
  4. ptr: uint32[E + 1], exclusive prefix of padded run lengths (values);
     the total must stay below 2**32.
  5. Header, 32 bytes little-endian: b"SWMC", u32 version = 2, i64 M, i64 K,
     u32 R = 256, u32 Mb.
  6. Blob = header || ptr || bits || values, no gaps.
Which entries are kept is the tiled format's rule: the mask if one is given,
else every entry whose value is not +0 or -0; kept entries keep their bits.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass

import numpy as np

MAGIC = b"SWMC"
VERSION = 2
G = 4
R = 256
HEADER_BYTES = 32
_HDR = struct.Struct("<4sIqqII")
assert _HDR.size == HEADER_BYTES


@dataclass
class ColRuns:
    M: int
    K: int
    Mb: int
    ptr: np.ndarray     # uint32 [E + 1]
    bits: np.ndarray    # uint64 [E*4]
    values: np.ndarray  # uint16

    def blob(self) -> bytes:
        return (_HDR.pack(MAGIC, VERSION, self.M, self.K, R, self.Mb) + self.ptr.astype("<u4").tobytes()
                + self.bits.astype("<u8").tobytes() + self.values.astype("<u2").tobytes())


def colruns_encode(W: np.ndarray, mask: np.ndarray | None) -> ColRuns:
    """Spec steps 1-4 from a dense fp16 W (M, K) and an optional boolean mask."""
    W = np.asarray(W, dtype=np.float16)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    M, K = W.shape
    wbits = W.view(np.uint16)
    if mask is None:
        keep = (wbits & np.uint16(0x7FFF)) != 0
    else:
        keep = np.asarray(mask, dtype=bool)
        if keep.shape != (M, K):
            raise ValueError("mask shape mismatch")
    Mb = -(-M // R)
    Gn = -(-Mb // G)
    weights = np.uint64(1) << np.arange(64, dtype=np.uint64)
    # per block: bitmap words (K, 4) and each column's run (padded)
    blk_bits, blk_runs = [], []
    for b in range(Gn * G):
        kb = np.zeros((R, K), dtype=bool)
        vb = np.zeros((R, K), dtype=np.uint16)
        rows = max(0, min(R, M - R * b))
        kb[:rows] = keep[R * b:R * b + rows]
        vb[:rows] = wbits[R * b:R * b + rows]
        words = np.zeros((K, 4), dtype=np.uint64)
        for q in range(4):
            blk = kb[64 * q:64 * q + 64].astype(np.uint64)  # (64, K): bit i = row 64q + i
            words[:, q] = (blk * weights[:, None]).sum(axis=0, dtype=np.uint64)
        runs = []
        for k in range(K):
            run = vb[kb[:, k], k]  # increasing row order
            pad = (-run.size) % 4
            if pad:
                run = np.concatenate([run, np.zeros(pad, dtype=np.uint16)])
            runs.append(run)
        blk_bits.append(words)
        blk_runs.append(runs)
    # entries in e order: group g, column k, block j of the group
    bits, runs = [], []
    for g in range(Gn):
        for k in range(K):
            for j in range(G):
                bits.append(blk_bits[G * g + j][k])
                runs.append(blk_runs[G * g + j][k])
    lens = np.array([r.size for r in runs], dtype=np.int64)
    ptr = np.zeros(len(runs) + 1, dtype=np.int64)
    np.cumsum(lens, out=ptr[1:])
    if ptr[-1] >= 2 ** 32:
        raise OverflowError("padded value count does not fit in 32 bits")
    values = np.concatenate(runs) if runs else np.zeros(0, dtype=np.uint16)
    bits = np.concatenate(bits) if bits else np.zeros(0, dtype=np.uint64)
    return ColRuns(M=M, K=K, Mb=Mb, ptr=ptr.astype(np.uint32), bits=bits, values=values)


def colruns_parse(blob: bytes) -> ColRuns:
    if len(blob) < HEADER_BYTES:
        raise ValueError("blob shorter than header")
    magic, ver, M, K, r, Mb = _HDR.unpack_from(blob, 0)
    if magic != MAGIC or ver != VERSION or r != R or Mb != -(-M // R):
        raise ValueError("bad header")
    E = -(-Mb // G) * K * G
    off = HEADER_BYTES
    ptr = np.frombuffer(blob, dtype="<u4", count=E + 1, offset=off).astype(np.uint32)
    off += 4 * (E + 1)
    bits = np.frombuffer(blob, dtype="<u8", count=4 * E, offset=off).astype(np.uint64)
    off += 32 * E
    n = int(ptr[-1])
    values = np.frombuffer(blob, dtype="<u2", count=n, offset=off).astype(np.uint16)
    if off + 2 * n != len(blob):
        raise ValueError("blob size mismatch")
    return ColRuns(M=M, K=K, Mb=Mb, ptr=ptr, bits=bits, values=values)


def colruns_decode(c: ColRuns) -> tuple[np.ndarray, np.ndarray]:
    """(W bits with pruned entries +0, keep mask), both (M, K), from the encoding."""
    Gn = -(-c.Mb // G)
    W = np.zeros((Gn * G * R, c.K), dtype=np.uint16)
    keep = np.zeros((Gn * G * R, c.K), dtype=bool)
    for g in range(Gn):
        for k in range(c.K):
            for j in range(G):
                e = (g * c.K + k) * G + j
                b = G * g + j
                rows = []
                for q in range(4):
                    w = int(c.bits[4 * e + q])
                    rows += [R * b + 64 * q + i for i in range(64) if (w >> i) & 1]
                p = int(c.ptr[e])
                W[rows, k] = c.values[p:p + len(rows)]
                keep[rows, k] = True
    return W[:c.M], keep[:c.M]
