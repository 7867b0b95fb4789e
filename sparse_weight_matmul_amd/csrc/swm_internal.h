// Internal declarations shared by the host format code and the HIP launchers.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "swm.h"

namespace swm {

constexpr uint32_t kVersion = 2;
constexpr uint32_t kTM = 16;  // rows per tile
constexpr size_t kHeaderBytes = 64;
constexpr int kPadValues = 8;  // each tile run is padded to a multiple of 8 values (16 B)

// Parsed SWM-TCB v2 header (little-endian on disk; this build targets x86-64 hosts).
struct Header {
  int64_t m = 0, k = 0;
  uint32_t tm = 0, tk = 0;
  uint64_t nnz = 0, padded_len = 0;
  uint32_t mt = 0, kt = 0;
  uint32_t max_tile = 0;

  uint64_t tiles() const { return uint64_t(mt) * kt; }
  uint64_t words_per_tile() const { return tk / 4; }  // 4 column bitmaps of 16 bits per word
  uint64_t n_bits() const { return tiles() * words_per_tile(); }
  size_t off_tile_ptr() const { return kHeaderBytes; }
  size_t off_bits() const { return off_tile_ptr() + 4 * (tiles() + 1); }
  size_t off_values() const { return off_bits() + 8 * n_bits(); }
  size_t total_bytes() const { return off_values() + 2 * padded_len; }
};

void write_header(const Header& h, uint8_t* dst);
swm_status read_header(const void* buf, size_t size, Header* h);

// Check tile shape and sizes; fills h.tm/tk/mt/kt/m/k.
swm_status plan_grid(int64_t M, int64_t K, const swm_tile_cfg* cfg, Header* h);

// Encode to a full export blob.
swm_status encode_blob(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm,
                       int64_t M, int64_t K, const swm_tile_cfg* cfg, std::vector<uint8_t>* out);

// Full structural validation of a blob.
swm_status validate_blob(const void* buf, size_t size, Header* h);

void fill_info(const Header& h, swm_format_info* info);

// True if some row keeps more than 2 entries in an aligned group of 4
// columns (the mask is not 2:4 along K), from a validated blob's bitmaps.
bool mask_exceeds_2_of_4(const Header& h, const uint8_t* blob);

// SWM-CR v2 column-run encoding (activation skipping): kept entries grouped
// by input column inside blocks of kColRunRows rows, the blocks of a column
// stored kColRunGroup at a time.
constexpr int kColRunRows = 256;
constexpr int kColRunGroup = 4;  // row blocks stored together per column
constexpr size_t kColRunHeaderBytes = 32;
struct ColRunsHost {
  int64_t m = 0, k = 0, mb = 0;  // mb row blocks, in ceil(mb / 4) groups
  std::vector<uint32_t> ptr;     // entries + 1
  std::vector<uint64_t> bits;    // entries * 4
  std::vector<uint16_t> values;  // padded runs
  uint64_t entries() const { return uint64_t((mb + kColRunGroup - 1) / kColRunGroup) * uint64_t(k) * kColRunGroup; }
};
// Derive the encoding from a SWM-TCB v2 blob (validated first).
swm_status colruns_from_tcb(const void* tcb, size_t size, ColRunsHost* out);
size_t colruns_blob_bytes(const ColRunsHost& c);
void colruns_write_blob(const ColRunsHost& c, uint8_t* dst);

}  // namespace swm
