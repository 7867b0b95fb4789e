// Host side of the SWM-TCB v2 tiled column-bitmap format: encoder, blob
// header, validator and size accounting.
//
// The format is this library's reading of the "Tiled-Column-wise Bitmap
// Compressed" format named by "Unified Static-Dynamic Pruning for Efficient LLM
// Inference" (abstract), whose layout the page does not give.  One bit of
// position metadata per entry keeps metadata small at ~50% sparsity, the goal
// set in "Accelerating GPU inference of LLMs with moderately unstructured
// sparse weight matrices", Sec. 3.1 (and Challenge 2 of its Sec. 1, where
// per-nonzero indices cost as much as the values).
//
// Layout (TM = 16; tile t = i*kt + j covers rows [16i, 16i+16) and columns
// [tk*j, tk*j + tk), tk a multiple of 32):
//   a tile has tk/32 steps of 32 columns, each step eight 64-bit words; word
//   w = 8*s + e carries in bits 16q..16q+15 the 16-row bitmap of tile column
//   32*s + 8*q + e, i.e. bit b <=> (row 16i + b%16, column tk*j + 32s + 8(b/16) + e);
//   values: kept fp16 bits word by word, bit by bit (column by column, rows
//   ascending), each tile run zero-padded to a multiple of 8 values;
//   tile_ptr[t] = exclusive prefix of padded run lengths (uint32).
// This bit order puts, for lane b of a 64-wide wave, row b%16 and column
// group b/16 in the same place as the A operand of a 16x16x32 matrix-core
// product, so a decoded word feeds the matrix cores without reshuffling.
// Pattern computation is offline: the moderate-sparsity page, Sec. 2.1.
#include <algorithm>
#include <cstring>
#include <limits>

#include "swm_internal.h"

namespace swm {

namespace {

template <typename T>
void put(uint8_t* dst, size_t off, T v) {
  std::memcpy(dst + off, &v, sizeof(T));
}
template <typename T>
T get(const uint8_t* src, size_t off) {
  T v;
  std::memcpy(&v, src + off, sizeof(T));
  return v;
}

inline bool keep_entry(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm, int64_t r,
                       int64_t c) {
  if (mask) return mask[r * ldm + c] != 0;
  return (W[r * ldw + c] & 0x7FFFu) != 0;  // null mask: keep values other than +-0
}

// Row and column (inside the tile) of bit b of word w.
inline void bit_pos(uint32_t w, uint32_t b, uint32_t* row, uint32_t* col) {
  *row = b & 15u;
  *col = 32u * (w >> 3) + 8u * (b >> 4) + (w & 7u);
}

}  // namespace

void write_header(const Header& h, uint8_t* dst) {
  std::memset(dst, 0, kHeaderBytes);
  std::memcpy(dst, "SWMT", 4);
  put<uint32_t>(dst, 4, kVersion);
  put<int64_t>(dst, 8, h.m);
  put<int64_t>(dst, 16, h.k);
  put<uint32_t>(dst, 24, h.tm);
  put<uint32_t>(dst, 28, h.tk);
  put<uint64_t>(dst, 32, h.nnz);
  put<uint64_t>(dst, 40, h.padded_len);
  put<uint32_t>(dst, 48, h.mt);
  put<uint32_t>(dst, 52, h.kt);
  put<uint32_t>(dst, 56, h.max_tile);
  put<uint32_t>(dst, 60, 0u);
}

swm_status read_header(const void* buf, size_t size, Header* h) {
  if (!buf || !h) return SWM_ERR_INVALID_ARG;
  if (size < kHeaderBytes) return SWM_ERR_FORMAT;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (std::memcmp(b, "SWMT", 4) != 0) return SWM_ERR_FORMAT;
  if (get<uint32_t>(b, 4) != kVersion) return SWM_ERR_FORMAT;
  Header r;
  r.m = get<int64_t>(b, 8);
  r.k = get<int64_t>(b, 16);
  r.tm = get<uint32_t>(b, 24);
  r.tk = get<uint32_t>(b, 28);
  r.nnz = get<uint64_t>(b, 32);
  r.padded_len = get<uint64_t>(b, 40);
  r.mt = get<uint32_t>(b, 48);
  r.kt = get<uint32_t>(b, 52);
  r.max_tile = get<uint32_t>(b, 56);
  if (get<uint32_t>(b, 60) != 0) return SWM_ERR_FORMAT;
  if (r.m < 0 || r.k < 0 || r.tm != kTM || r.tk == 0 || r.tk % 32 || r.tk > 4096) return SWM_ERR_FORMAT;
  if (uint64_t(r.mt) != (uint64_t(r.m) + r.tm - 1) / r.tm) return SWM_ERR_FORMAT;
  if (uint64_t(r.kt) != (uint64_t(r.k) + r.tk - 1) / r.tk) return SWM_ERR_FORMAT;
  if (r.padded_len >= (uint64_t(1) << 32)) return SWM_ERR_FORMAT;
  // Section sizes must fit size_t without wrapping (cap at 2^50 bytes).
  const uint64_t lim = uint64_t(1) << 50;
  if (r.tiles() > lim / 64 || r.n_bits() > lim / 8) return SWM_ERR_FORMAT;
  *h = r;
  return SWM_OK;
}

swm_status plan_grid(int64_t M, int64_t K, const swm_tile_cfg* cfg, Header* h) {
  int32_t tm = cfg ? cfg->tm : int32_t(kTM), tk = cfg ? cfg->tk : 64;
  if (M < 0 || K < 0) return SWM_ERR_INVALID_ARG;
  if (tm != int32_t(kTM) || tk <= 0 || tk % 32 || tk > 4096) return SWM_ERR_INVALID_ARG;
  const int64_t lim = int64_t(1) << 40;
  if (M > lim || K > lim) return SWM_ERR_OVERFLOW;
  Header r;
  r.m = M;
  r.k = K;
  r.tm = uint32_t(tm);
  r.tk = uint32_t(tk);
  uint64_t mt = (uint64_t(M) + tm - 1) / tm, kt = (uint64_t(K) + tk - 1) / tk;
  if (mt > std::numeric_limits<uint32_t>::max() || kt > std::numeric_limits<uint32_t>::max())
    return SWM_ERR_OVERFLOW;
  r.mt = uint32_t(mt);
  r.kt = uint32_t(kt);
  if (r.tiles() > (uint64_t(1) << 40) / r.words_per_tile()) return SWM_ERR_OVERFLOW;
  *h = r;
  return SWM_OK;
}

swm_status encode_blob(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm,
                       int64_t M, int64_t K, const swm_tile_cfg* cfg, std::vector<uint8_t>* out) {
  if (!out) return SWM_ERR_INVALID_ARG;
  if ((M > 0 && K > 0) && !W) return SWM_ERR_INVALID_ARG;
  if (ldw < K || (mask && ldm < K)) return SWM_ERR_INVALID_ARG;
  Header h;
  swm_status st = plan_grid(M, K, cfg, &h);
  if (st != SWM_OK) return st;
  const uint32_t tm = h.tm, tk = h.tk, nw = uint32_t(h.words_per_tile());
  const uint64_t T = h.tiles();

  // Pass 1: kept entries per tile -> padded run lengths -> tile_ptr.
  std::vector<uint64_t> tile_nnz(T, 0);
  for (int64_t r = 0; r < M; ++r) {
    const uint64_t i = uint64_t(r) / tm;
    for (int64_t c = 0; c < K; ++c)
      if (keep_entry(W, ldw, mask, ldm, r, c)) ++tile_nnz[i * h.kt + uint64_t(c) / tk];
  }
  uint64_t total = 0, nnz = 0, max_tile = 0;
  for (uint64_t t = 0; t < T; ++t) {
    uint64_t padded = (tile_nnz[t] + kPadValues - 1) / kPadValues * kPadValues;
    nnz += tile_nnz[t];
    total += padded;
    if (padded > max_tile) max_tile = padded;
  }
  if (total >= (uint64_t(1) << 32)) return SWM_ERR_OVERFLOW;
  h.nnz = nnz;
  h.padded_len = total;
  h.max_tile = uint32_t(max_tile);

  try {
    out->assign(h.total_bytes(), 0);
  } catch (...) {
    return SWM_ERR_OOM;
  }
  uint8_t* blob = out->data();
  write_header(h, blob);
  uint8_t* tp = blob + h.off_tile_ptr();
  uint8_t* bits = blob + h.off_bits();
  uint8_t* vals = blob + h.off_values();

  // Pass 2: per tile, copy into a local (row, column) buffer, then emit words
  // and values in storage order.
  std::vector<uint16_t> tv(size_t(tm) * tk);
  std::vector<uint8_t> tkp(size_t(tm) * tk);
  uint64_t pos = 0;
  for (uint64_t i = 0; i < h.mt; ++i) {
    for (uint64_t j = 0; j < h.kt; ++j) {
      const uint64_t t = i * h.kt + j;
      put<uint32_t>(tp, 4 * t, uint32_t(pos));
      std::fill(tkp.begin(), tkp.end(), 0);
      const int64_t r0 = int64_t(i * tm), c0 = int64_t(j * tk);
      const int64_t r1 = std::min<int64_t>(r0 + tm, M), c1 = std::min<int64_t>(c0 + tk, K);
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          const size_t li = size_t(r - r0) * tk + size_t(c - c0);
          tkp[li] = keep_entry(W, ldw, mask, ldm, r, c) ? 1 : 0;
          tv[li] = W[r * ldw + c];
        }
      for (uint32_t w = 0; w < nw; ++w) {
        uint64_t word = 0;
        for (uint32_t b = 0; b < 64; ++b) {
          uint32_t row, col;
          bit_pos(w, b, &row, &col);
          const size_t li = size_t(row) * tk + col;
          if (tkp[li]) {
            word |= uint64_t(1) << b;
            put<uint16_t>(vals, 2 * pos, tv[li]);
            ++pos;
          }
        }
        put<uint64_t>(bits, 8 * (t * nw + w), word);
      }
      pos = (pos + kPadValues - 1) / kPadValues * kPadValues;  // padding stays 0x0000
    }
  }
  put<uint32_t>(tp, 4 * T, uint32_t(pos));
  return SWM_OK;
}

swm_status validate_blob(const void* buf, size_t size, Header* hout) {
  Header h;
  swm_status st = read_header(buf, size, &h);
  if (st != SWM_OK) return st;
  if (h.total_bytes() != size) return SWM_ERR_FORMAT;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  const uint8_t* tp = b + h.off_tile_ptr();
  const uint8_t* bits = b + h.off_bits();
  const uint8_t* vals = b + h.off_values();
  const uint64_t T = h.tiles(), nw = h.words_per_tile();
  if (get<uint32_t>(tp, 0) != 0) return SWM_ERR_FORMAT;
  uint64_t nnz = 0, max_tile = 0;
  for (uint64_t t = 0; t < T; ++t) {
    const uint64_t p0 = get<uint32_t>(tp, 4 * t), p1 = get<uint32_t>(tp, 4 * (t + 1));
    if (p1 < p0 || (p1 - p0) % kPadValues || p1 > h.padded_len) return SWM_ERR_FORMAT;
    const uint64_t i = t / h.kt, j = t % h.kt;
    const int64_t rows_valid = std::max<int64_t>(0, std::min<int64_t>(16, h.m - int64_t(16 * i)));
    const uint64_t row_ok = rows_valid >= 16 ? 0xFFFFull : ((uint64_t(1) << rows_valid) - 1);
    uint64_t pc = 0;
    for (uint64_t w = 0; w < nw; ++w) {
      const uint64_t word = get<uint64_t>(bits, 8 * (t * nw + w));
      uint64_t allowed = 0;
      for (uint32_t q = 0; q < 4; ++q) {
        const int64_t col = int64_t(j * h.tk + 32 * (w >> 3) + 8 * q + (w & 7));
        if (col < h.k) allowed |= row_ok << (16 * q);
      }
      if (word & ~allowed) return SWM_ERR_FORMAT;
      pc += uint64_t(__builtin_popcountll(word));
    }
    if (p1 - p0 < pc || p1 - p0 >= pc + kPadValues) return SWM_ERR_FORMAT;
    for (uint64_t q = p0 + pc; q < p1; ++q)
      if (get<uint16_t>(vals, 2 * q) != 0) return SWM_ERR_FORMAT;
    nnz += pc;
    if (p1 - p0 > max_tile) max_tile = p1 - p0;
  }
  if (get<uint32_t>(tp, 4 * T) != h.padded_len) return SWM_ERR_FORMAT;
  if (nnz != h.nnz || max_tile != h.max_tile) return SWM_ERR_FORMAT;
  if (hout) *hout = h;
  return SWM_OK;
}

void fill_info(const Header& h, swm_format_info* info) {
  std::memset(info, 0, sizeof(*info));
  info->m = h.m;
  info->k = h.k;
  info->tm = int32_t(h.tm);
  info->tk = int32_t(h.tk);
  info->mt = h.mt;
  info->kt = h.kt;
  info->nnz = h.nnz;
  info->padded_len = h.padded_len;
  info->max_tile = h.max_tile;
  info->bytes_header = kHeaderBytes;
  info->bytes_tile_ptr = 4 * (h.tiles() + 1);
  info->bytes_bits = 8 * h.n_bits();
  info->bytes_values = 2 * h.padded_len;
  info->bytes_total = h.total_bytes();
}

bool mask_exceeds_2_of_4(const Header& h, const uint8_t* blob) {
  // Tiles start at multiples of 32 columns, so aligned groups of 4 never
  // straddle a 32-column step.  Group a (0..7) of step s is columns
  // 32s + 4a .. +3: quarter q = a/2 of the words 8s + 4(a%2) .. +3, whose
  // bits 16q .. 16q+15 are the 16 rows.  A row keeps 3 or 4 entries of the
  // group iff three of its four bits are set.
  const uint64_t* bits = reinterpret_cast<const uint64_t*>(blob + h.off_bits());
  const uint64_t wpt = h.words_per_tile();
  for (uint64_t t = 0; t < h.tiles(); ++t)
    for (uint64_t sidx = 0; sidx < h.tk / 32; ++sidx)
      for (int a = 0; a < 8; ++a) {
        const uint64_t* w = bits + t * wpt + 8 * sidx + 4 * (a % 2);
        const int q = a / 2;
        const uint32_t f0 = uint32_t(w[0] >> (16 * q)) & 0xFFFF, f1 = uint32_t(w[1] >> (16 * q)) & 0xFFFF;
        const uint32_t f2 = uint32_t(w[2] >> (16 * q)) & 0xFFFF, f3 = uint32_t(w[3] >> (16 * q)) & 0xFFFF;
        if ((f0 & f1 & f2) | (f0 & f1 & f3) | (f0 & f2 & f3) | (f1 & f2 & f3)) return true;
      }
  return false;
}

}  // namespace swm
