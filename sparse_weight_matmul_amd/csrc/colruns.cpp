// Host side of the SWM-CR v2 column-run encoding used by activation skipping.
//
// The decode kernel of "Unified Static-Dynamic Pruning for Efficient LLM
// Inference" (SPDP, abstract) skips at run time the input channels whose
// activation is zero; "Reduced Matrix Multiplication" (blog page, Sec. 4.2)
// gives the reason this is exact (a zero channel adds only zero terms).  The
// tiled format keeps at most 16 rows of one column together (at most 32
// bytes), so an inactive column shares its memory sectors with active ones
// and skipping it saves nothing.  This encoding regroups the same kept
// entries column by column inside blocks of R = 256 rows, so a column's run is
// about 256 bytes at 50% sparsity and skipping it skips whole cache lines.
// Blocks are stored in groups of four per column: the four bitmap entries of
// a column (4 x 32 bytes) fill one 128-byte line and its four runs are
// adjacent, so an active column's data shares lines only with itself.
//
// Layout (block b = 4g + j, j = 0..3, rows [256b, 256b + 256); entry
// e = (g*K + k)*4 + j is column k of block b; blocks past Mb in the last
// group are empty entries):
//   bits[e][q], q = 0..3: bit i <=> row 256b + 64q + i kept;
//   values: kept fp16 bits of entry e in increasing row order, each run
//   zero-padded to a multiple of 4 values (8 bytes);
//   ptr[e] = exclusive prefix of padded run lengths (uint32).
// Blob: 32-byte header (b"SWMC", u32 version 2, i64 M, i64 K, u32 R, u32 Mb)
// || ptr || bits || values.  The encoding is derived from a validated SWM-TCB
// v2 blob, so both hold exactly the same kept entries and bits.
#include <cstring>

#include "swm_internal.h"

namespace swm {

swm_status colruns_from_tcb(const void* tcb, size_t size, ColRunsHost* out) {
  Header h;
  swm_status st = validate_blob(tcb, size, &h);
  if (st != SWM_OK) return st;
  if (h.tm != 16 || h.tk % 32 != 0) return SWM_ERR_UNSUPPORTED;
  const uint8_t* blob = static_cast<const uint8_t*>(tcb);
  const uint32_t* tile_ptr = reinterpret_cast<const uint32_t*>(blob + h.off_tile_ptr());
  const uint8_t* bits_b = blob + h.off_bits();
  const uint8_t* vals_b = blob + h.off_values();
  const int64_t M = h.m, K = h.k;
  const int64_t Mb = (M + kColRunRows - 1) / kColRunRows;
  const uint64_t wpt = h.words_per_tile();
  ColRunsHost c;
  c.m = M;
  c.k = K;
  c.mb = Mb;
  const uint64_t E = c.entries();
  auto entry_of = [&](int64_t b, int64_t col) -> uint64_t {
    return (uint64_t(b / kColRunGroup) * uint64_t(K) + uint64_t(col)) * kColRunGroup + uint64_t(b % kColRunGroup);
  };
  try {
    c.ptr.assign(E + 1, 0);
    c.bits.assign(4 * E, 0);
    std::vector<uint32_t> count(E, 0);
    // Pass 1: kept entries per (block, column) and the bitmaps.
    for (uint32_t i = 0; i < h.mt; ++i)
      for (uint32_t j = 0; j < h.kt; ++j) {
        const uint64_t t = uint64_t(i) * h.kt + j;
        for (uint64_t w = 0; w < wpt; ++w) {
          uint64_t word;
          std::memcpy(&word, bits_b + 8 * (t * wpt + w), 8);
          const uint64_t s = w / 8, e = w % 8;
          while (word) {
            const int bit = __builtin_ctzll(word);
            word &= word - 1;
            const int64_t row = int64_t(i) * 16 + bit % 16;
            const int64_t col = int64_t(j) * h.tk + 32 * s + 8 * (bit / 16) + e;
            const int64_t b = row / kColRunRows, r = row % kColRunRows;
            const uint64_t en = entry_of(b, col);
            ++count[en];
            c.bits[4 * en + r / 64] |= uint64_t(1) << (r % 64);
          }
        }
      }
    uint64_t total = 0;
    for (uint64_t en = 0; en < E; ++en) {
      c.ptr[en] = uint32_t(total);
      total += (count[en] + 3) & ~3u;
      if (total >= (uint64_t(1) << 32)) return SWM_ERR_OVERFLOW;
    }
    c.ptr[E] = uint32_t(total);
    c.values.assign(total, 0);
    // Pass 2: values.  Slabs are visited in increasing row order and, inside a
    // slab, a column's bits in increasing row order, so appending keeps every
    // run sorted by row.
    std::vector<uint32_t> cur(c.ptr.begin(), c.ptr.end() - 1);
    for (uint32_t i = 0; i < h.mt; ++i)
      for (uint32_t j = 0; j < h.kt; ++j) {
        const uint64_t t = uint64_t(i) * h.kt + j;
        uint64_t pos = tile_ptr[t];
        for (uint64_t w = 0; w < wpt; ++w) {
          uint64_t word;
          std::memcpy(&word, bits_b + 8 * (t * wpt + w), 8);
          const uint64_t s = w / 8, e = w % 8;
          while (word) {
            const int bit = __builtin_ctzll(word);
            word &= word - 1;
            const int64_t row = int64_t(i) * 16 + bit % 16;
            const int64_t col = int64_t(j) * h.tk + 32 * s + 8 * (bit / 16) + e;
            const uint64_t en = entry_of(row / kColRunRows, col);
            uint16_t v;
            std::memcpy(&v, vals_b + 2 * pos, 2);
            ++pos;
            c.values[cur[en]++] = v;
          }
        }
      }
  } catch (...) {
    return SWM_ERR_OOM;
  }
  *out = std::move(c);
  return SWM_OK;
}

size_t colruns_blob_bytes(const ColRunsHost& c) {
  const uint64_t E = c.entries();
  return kColRunHeaderBytes + 4 * (E + 1) + 32 * E + 2 * c.values.size();
}

void colruns_write_blob(const ColRunsHost& c, uint8_t* dst) {
  const uint64_t E = c.entries();
  std::memset(dst, 0, kColRunHeaderBytes);
  std::memcpy(dst, "SWMC", 4);
  const uint32_t ver = 2, r = kColRunRows, mb = uint32_t(c.mb);
  std::memcpy(dst + 4, &ver, 4);
  std::memcpy(dst + 8, &c.m, 8);
  std::memcpy(dst + 16, &c.k, 8);
  std::memcpy(dst + 24, &r, 4);
  std::memcpy(dst + 28, &mb, 4);
  size_t off = kColRunHeaderBytes;
  std::memcpy(dst + off, c.ptr.data(), 4 * (E + 1));
  off += 4 * (E + 1);
  std::memcpy(dst + off, c.bits.data(), 32 * E);
  off += 32 * E;
  if (!c.values.empty()) std::memcpy(dst + off, c.values.data(), 2 * c.values.size());
}

}  // namespace swm
