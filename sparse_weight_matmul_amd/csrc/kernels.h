// Device-side view of a compressed weight and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "swm_internal.h"

namespace swm {

// Device memory of one SWM-TCB v2 handle (16-row tiles).
struct DevFormat {
  Header h;
  const uint32_t* tile_ptr = nullptr;  // mt*kt + 1
  const uint64_t* bits = nullptr;      // mt*kt*tk words
  const uint16_t* vals = nullptr;      // padded_len values (+ slack for over-reads)
  const uint16_t* zeros = nullptr;     // >= kt*tk + 64 zero halves (device)
};

// Work split of the decode kernel for one call.
struct DecodePlan {
  int waves = 1;           // waves per workgroup (one workgroup per 16-row slab)
  int tiles_per_wave = 1;  // consecutive tiles of the slab per wave
  int seg_tiles = 4;       // tiles per streamed segment
  int seg_chunks = 1;      // 1 KiB loads per segment (covers the largest segment)
  int seq_segs = 0;        // straight-line kernel: two-tile segments per wave (0 = not used)
  int seq_chunks = 1;      // 1 KiB loads per two-tile segment
  bool direct_b = false;   // 9-16 tokens: B operands loaded straight into registers
};

// Work split of the decode kernel (at least one wave per 16 tiles of a slab
// row).  `straight_line` with kxi > 0: the split for token counts the
// straight-line kernel serves with kxi 1 KiB activation loads per segment
// (N <= 4: 1, <= 8: 2, <= 16: 4), chosen for the most resident waves per CU;
// otherwise about `waves_per_cu` waves per CU.  `tile_ptr` (host, mt*kt+1
// entries) sizes the segment loads.
DecodePlan plan_decode(const Header& h, const uint32_t* tile_ptr, int num_cus, int waves_per_cu, bool straight_line,
                       int kxi = 0);

hipError_t launch_decode(const DevFormat& f, const DecodePlan& p, const uint16_t* X, int64_t ldx,
                         uint16_t* Y, int64_t ldy, int n, bool skip, hipStream_t s);

// Activation-skipping decode over the SWM-CR v2 column-run encoding.
constexpr int kCrMaxCols = 1024;  // input columns per workgroup (one per thread)
struct ColRunsPlan {
  int mb = 0;      // 256-row blocks
  int splits = 0;  // column ranges (S)
  int cps = 0;     // columns per range
};
struct DevColRuns {
  int64_t m = 0, k = 0;
  const uint32_t* ptr = nullptr;   // entries + 1 (entries = ceil(mb/4)*4*k)
  const uint64_t* bits = nullptr;  // entries * 4
  const uint16_t* vals = nullptr;  // padded runs + 16 bytes of slack
  float* partials = nullptr;       // mb*splits*4*256 per-workgroup partial sums
  ColRunsPlan plan;
  uint64_t bytes = 0;              // ptr + bits + values
};
ColRunsPlan plan_colruns(int64_t M, int64_t K);
// Floats of per-workgroup partial sums one skipping call writes.
size_t colruns_partial_floats(const ColRunsPlan& p);
// Device address and size (floats) of the library's fixed partial-sum array
// on the current device (resolved once per device).
hipError_t spmspv_scratch(float** out, size_t* floats);
// tau: activations with |x| < tau count as zero (0 = only exact zeros).
hipError_t launch_spmspv_cr(const DevColRuns& c, const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy,
                            int n, float tau, hipStream_t s);

// Gated FFN decode: H = SiLU(W_g X) * (W_u X) with |H| < tau dropped, both
// formats in one launch of the straight-line kernel (seq_segs == 0: no
// instance covers the shape).
DecodePlan plan_decode_glu(const Header& g, const Header& u, int num_cus, int n);
hipError_t launch_decode_glu(const DevFormat& g, const DevFormat& u, const DecodePlan& p, const uint16_t* X,
                             int64_t ldx, uint16_t* H, int64_t ldh, int n, float tau, hipStream_t s);

hipError_t launch_decompress(const DevFormat& f, uint16_t* W, int64_t ldw, hipStream_t s);

// HBM read-bandwidth calibration: `blocks` workgroups of 256 threads stream `bytes`.
hipError_t launch_stream(const void* src, size_t bytes, int unroll, int blocks, uint32_t* out,
                         hipStream_t s);

// Dense W (row-major) times token-major X for n <= 16 tokens.
struct DensePlan {
  int waves = 4;
  int kchunk = 512;  // columns per wave
};
DensePlan plan_dense_small(int64_t M, int64_t K, int n, int num_cus);
hipError_t launch_dense_small(const DensePlan& p, const uint16_t* W, int64_t ldw, const uint16_t* X,
                              int64_t ldx, uint16_t* Y, int64_t ldy, int64_t M, int64_t K, int n, hipStream_t s);

// Tiled MFMA GEMM for larger N: dense W, or W expanded from the format tile by tile.
hipError_t launch_prefill_dense(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx,
                                uint16_t* Y, int64_t ldy, int64_t M, int64_t K, int64_t N, int num_cus,
                                hipStream_t s);
// The same kernel with the gated-FFN epilogue: W is M2 = 2 x channels rows
// with gate and up rows interleaved (2c, 2c+1), H (N x M2/2) receives
// SiLU(g) * u rounded to fp16, +0 where |h| < tau.  Needs the LDS-direct
// kernel's 32-bit byte offsets (prefill_dense_dma_fits).
hipError_t launch_prefill_dense_glu(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx,
                                    uint16_t* H, int64_t ldh, int64_t M2, int64_t K, int64_t N, float tau,
                                    int num_cus, hipStream_t s);
bool prefill_dense_dma_fits(int64_t M, int64_t ldw, int64_t K, int64_t N, int64_t ldx);
hipError_t launch_prefill_sparse(const DevFormat& f, const uint16_t* X, int64_t ldx, uint16_t* Y,
                                 int64_t ldy, int64_t N, hipStream_t s);
// The prefill kernels need K >= 8, K % 8 == 0, ldx % 8 == 0 and a 16-byte aligned X.
bool prefill_supported(int64_t K, int64_t ldx, const void* X);
size_t prefill_sparse_lds(const Header& h);
// The sparse prefill kernel addresses X with 32-bit byte offsets.
bool prefill_sparse_fits(const Header& h, int64_t N, int64_t ldx);

// Prefill on the sparse matrix cores: W (.) mask as a 2:4 layer plus a
// residual layer (both 2:4 conforming), compacted per call into a workspace
// and multiplied with v_smfmac_f32_32x32x32_f16.
struct Sparse24Layout {
  int64_t kp = 0, ldv = 0, ldm = 0;  // K rounded up to 64; values / index leading dimensions
  size_t off_m24 = 0, off_vres = 0, off_mres = 0, bytes = 0;
};
Sparse24Layout sparse24_layout(const Header& h, bool residual);
hipError_t launch_compact24(const DevFormat& f, const Sparse24Layout& L, bool residual, void* ws, hipStream_t s);
hipError_t launch_smf(const Header& h, const Sparse24Layout& L, bool residual, const void* ws, const uint16_t* X,
                      int64_t ldx, uint16_t* Y, int64_t ldy, int64_t N, int num_cus, hipStream_t s);
// The SMFMAC kernel addresses the compacted layers and X with 32-bit byte offsets.
bool smf_fits(const Header& h, int64_t N, int64_t ldx);

}  // namespace swm
