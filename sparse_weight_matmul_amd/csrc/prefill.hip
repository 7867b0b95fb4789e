// Prefill-regime kernels (large N): Y = W X on the matrix cores, with W
// either dense (the in-house baseline) or expanded on chip from the SWM-TCB v2
// format, tile by tile, into the same LDS operand layout.
//
// Method: "Unified Static-Dynamic Pruning for Efficient LLM Inference" (SPDP),
// abstract -- a matrix-core SpMM for the compute-intense prefill phase over the
// same tiled column-bitmap format as decode.  Loading the weights sparse and
// computing dense on chip is the pattern "Accelerating GPU inference of LLMs
// with moderately unstructured sparse weight matrices" (Sec. 2.3) describes for
// its prior art; at moderate sparsity the dense-executed products are the same
// as the dense GEMM's, so the sparse kernel can at best tie once compute bound.
//
// Dense kernel: one 256-thread workgroup computes a 256 (rows of W) x 256
// (tokens) block of Y over K in steps of 64.  Four waves in a 2 x 2 layout each
// own a 128 x 128 sub-block = 4 x 4 v_mfma_f32_32x32x16_f16 accumulators (256
// fp32 per lane, in AGPRs).  A and B tiles (256 x 64 fp16 each) are double
// buffered in LDS with an XOR swizzle of the 16-byte chunks, so the 16-byte
// fragment reads of consecutive rows hit distinct banks without padding.
// Inside a step the fragments of the next 16-column slice are read while the
// current slice's 16 products issue, and the next step's global tiles are in
// flight in VGPRs.  All global loads are unconditional: rows past M and tokens
// past N read a clamped valid row (their outputs are never stored) and
// activations past K read as zero.
//
// Sparse kernel: see prefill_ws_kernel below (eight waves, two per SIMD, the
// expansion shared by all of them).  Both kernels map workgroups to tiles XCD
// aware: consecutive workgroup ids go to different XCDs, so ids are regrouped
// to give each XCD a contiguous band of output tiles that share weight rows
// in its L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "kernels.h"

namespace swm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int BM = 256, BN = 256, BK = 64;  // default block (launchers set the grid per kernel shape)

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void lds_store16(uint32_t addr, u32x4 v) {
  *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(addr)) = v;
}
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr) {
  return *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(addr));
}
// Byte offset of (row, 16-byte chunk) in a swizzled 256 x 64 fp16 tile.  The
// LDS serves a 16-byte read for 16 lanes at a time from 64 four-byte banks
// (256 bytes), i.e. two 128-byte rows: rows of one parity share a bank half,
// so the chunk is permuted by bits 1..3 of the row, and 16 consecutive rows
// reading the same logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return uint32_t(row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4));
}

struct PrefillArgs {
  const uint16_t* W;  // dense variant
  const uint32_t* tile_ptr;
  const uint64_t* bits;
  const uint16_t* vals;  // sparse variant
  const uint16_t* X;
  uint16_t* Y;
  int64_t ldw, ldx, ldy;
  int M, N, K;
  int tiles_m, tiles_n, kt, mt;
  int group_m;     // output-tile rows per L2 group
  int run_chunks;  // 512-byte run chunks per tile (1..4), sparse variant
  float tau;       // gated epilogue: |h| below tau (after fp16 rounding) is stored as +0
};

// Map the workgroup id to an output tile: regroup ids so that each XCD (id % 8)
// gets a contiguous range, then walk that range column-major inside bands of
// group_m tile rows (the band's weight rows stay hot in that XCD's L2).
__device__ __forceinline__ bool tile_of(const PrefillArgs& a, int& tm, int& tn) {
  const int total = a.tiles_m * a.tiles_n;
  const int g = int(blockIdx.x);
  const int per_xcd = (int(gridDim.x) + 7) / 8;
  const int l = (g & 7) * per_xcd + (g >> 3);
  if (l >= total) return false;
  const int band = a.group_m * a.tiles_n;
  const int first_m = (l / band) * a.group_m;
  const int gm = min(a.group_m, a.tiles_m - first_m);
  const int r = l % band;
  tm = first_m + r % gm;
  tn = r / gm;
  return true;
}

// Dense block shapes: waves in a 2 x 2 layout, each owning kWI x kWJ 32 x 32
// accumulators, so the block is 64 kWI (rows of W) x 64 kWJ (tokens).  The
// host takes the largest block that still gives every CU work.
template <int kWI, int kWJ>
__global__ __launch_bounds__(256) void dense_kernel(PrefillArgs a) {
  constexpr int kBM = 64 * kWI, kBN = 64 * kWJ;
  constexpr int kAT = kBM * BK * 2, kBT = kBN * BK * 2;  // stage bytes
  constexpr int kRA = kBM / 32, kRB = kBN / 32;         // 16-byte loads per thread
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  if (!tile_of(a, tm, tn)) return;
  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = tm * kBM, n0 = tn * kBN;

  // LDS: A stages [2][kAT] | B stages [2][kBT]
  const uint32_t sA = lds_addr(smem), sB = sA + 2 * kAT;

  // Global fetch map: thread -> (row r*32 + tid/8, chunk tid%8).
  const int frow = tid >> 3, fch = tid & 7;
  const int nsteps = (a.K + BK - 1) / BK;

  // B: tokens past N read token N-1 (never stored); columns past K read 0.
  const uint16_t* xrow[kRB];
#pragma unroll
  for (int r = 0; r < kRB; ++r) xrow[r] = a.X + int64_t(min(n0 + r * 32 + frow, a.N - 1)) * a.ldx;
  u32x4 regA[kRA], regB[kRB];
  bool bvalid = true;  // the fetched B chunk lies inside K (zeroed at the store, not at the load)
  auto fetch_B = [&](int ks) {
    const int k = ks * BK + fch * 8;
    const int kc = min(k, a.K - 8);
    bvalid = k < a.K;
#pragma unroll
    for (int r = 0; r < kRB; ++r) regB[r] = *reinterpret_cast<const u32x4*>(xrow[r] + kc);
  };
  auto store_B = [&](int stage) {
#pragma unroll
    for (int r = 0; r < kRB; ++r) {
      const u32x4 v = bvalid ? regB[r] : u32x4{0u, 0u, 0u, 0u};
      lds_store16(sB + stage * kBT + swz(r * 32 + frow, fch), v);
    }
  };
  // A: rows past M read row M-1 (never stored); columns past K are
  // multiplied by zero activations.
  auto fetch_A = [&](int ks) {
    const int kc = min(ks * BK + fch * 8, a.K - 8);
#pragma unroll
    for (int r = 0; r < kRA; ++r) {
      const int m = min(m0 + r * 32 + frow, a.M - 1);
      regA[r] = *reinterpret_cast<const u32x4*>(a.W + int64_t(m) * a.ldw + kc);
    }
  };
  auto store_A = [&](int stage) {
#pragma unroll
    for (int r = 0; r < kRA; ++r) lds_store16(sA + stage * kAT + swz(r * 32 + frow, fch), regA[r]);
  };

  f32x16 acc[kWI][kWJ];
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < kWJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Prologue: stage 0 complete in LDS.
  fetch_B(0);
  fetch_A(0);
  store_A(0);
  store_B(0);
  __syncthreads();

  // One basic block per step.  The next step's tiles are fetched
  // interleaved with the first two slices' products (the vector memory
  // path then works in the background instead of stalling the issue of a
  // burst), and stored into the free stage interleaved with the last
  // slice's products.  The last step refetches itself into the unused stage.
  constexpr int kM = kWI * kWJ;                          // products per slice
  constexpr int kW = (kRA + kRB + kM - 1) / kM;          // LDS stores per product in the last slice
  for (int ks = 0; ks < nsteps; ++ks) {
    const int st = ks & 1;
    const int kn = min(ks + 1, nsteps - 1);
    const uint32_t aBase = sA + st * kAT, bBase = sB + st * kBT;
    half8 fa[2][kWI], fb[2][kWJ];
    auto load_frags = [&](int kk, int slot) {
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < kWI; ++i)
        fa[slot][i] = __builtin_bit_cast(half8, lds_load16(aBase + swz((wm * kWI + i) * 32 + (lane & 31), ch)));
#pragma unroll
      for (int j = 0; j < kWJ; ++j)
        fb[slot][j] = __builtin_bit_cast(half8, lds_load16(bBase + swz((wn * kWJ + j) * 32 + (lane & 31), ch)));
    };
    load_frags(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int sl = kk & 1;
      if (kk < 3) load_frags(kk + 1, sl ^ 1);
      if (kk == 0) fetch_A(kn);
      if (kk == 1) fetch_B(kn);
#pragma unroll
      for (int i = 0; i < kWI; ++i)
#pragma unroll
        for (int j = 0; j < kWJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0);
      if (kk == 3) {
        store_A(st ^ 1);
        store_B(st ^ 1);
      }
      // issue pattern of this slice: next fragments first, then products
      // with the slice's global loads or LDS stores spread between them
      __builtin_amdgcn_sched_group_barrier(0x100, kWI + kWJ, 0);  // DS read
      if (kk == 0) {
        constexpr int kL = kRA < kM ? kRA : kM;
#pragma unroll
        for (int q = 0; q < kL; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, kM / kL, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, kRA / kL, 0);  // VMEM read
        }
      } else if (kk == 1) {
        constexpr int kL = kRB < kM ? kRB : kM;
#pragma unroll
        for (int q = 0; q < kL; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, kM / kL, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, kRB / kL, 0);  // VMEM read
        }
      } else if (kk == 3) {
#pragma unroll
        for (int q = 0; q < kM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x200, kW, 0);  // DS write
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  // Epilogue: fp16 round-to-nearest-even, 4 consecutive rows per 8-byte store.
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < kWJ; ++j) {
      const int n = n0 + (wn * kWJ + j) * 32 + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + (wm * kWI + i) * 32 + q * 8 + (lane >> 5) * 4;
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, _Float16(acc[i][j][q * 4 + e]));
        uint16_t* dst = a.Y + int64_t(n) * a.ldy + m;
        if (m + 3 < a.M && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
          u32x2 pk = {uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
          *reinterpret_cast<u32x2*>(dst) = pk;
        } else {
          for (int e = 0; e < 4; ++e)
            if (m + e < a.M) dst[e] = h[e];
        }
      }
    }
}

// ------------------------------------------------------------------ dense, tiles loaded straight into LDS
// Sixteen zero bytes: the source of activation chunks past K.
__device__ __attribute__((aligned(16))) uint16_t g_pf_zero[8];

// Global -> LDS without registers: lane l writes 16 bytes at lds + 16 l
// (`lds` is the same for every lane of the wave).
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// s_waitcnt: at most n vector memory operations of this wave outstanding and
// every LDS operation complete (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at 7, lgkmcnt 11:8 = 0).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (((n >> 4) & 3) << 14));
}

// kWM x kWN waves, each owning kWI x kWJ accumulators of 32 x 32: the block
// is 32 kWI kWM rows of W by 32 kWJ kWN tokens.
template <int kWI, int kWJ, int kWM, int kWN>
struct DmaShape {
  static constexpr int kNW = kWM * kWN;                              // waves
  static constexpr int kBR = 32 * kWI * kWM, kBT = 32 * kWJ * kWN;  // block rows, tokens
  static constexpr int kAT = kBR * BK * 2, kBTB = kBT * BK * 2;     // stage bytes
  // three stages where the block is alone on its CU anyway; the 128x128
  // block keeps two, so that two blocks share a CU
  static constexpr int kStages = kBR * kBT >= 256 * 128 && 3 * (kAT + kBTB) <= 160 * 1024 ? 3 : 2;
  static constexpr int kIA = kAT / (1024 * kNW), kIB = kBTB / (1024 * kNW);  // 1 KiB loads per wave per step
  static_assert(kIA * 1024 * kNW == kAT && kIB * 1024 * kNW == kBTB, "whole loads per wave");
  // the stages, or the per-wave epilogue regions (a padded token row each) if larger
  static constexpr int kEpi = kNW * (32 * kWJ) * (64 * kWI + 8);
  static constexpr int kLds = kStages * (kAT + kBTB) > kEpi ? kStages * (kAT + kBTB) : kEpi;
  static_assert(kLds <= 160 * 1024, "LDS");
};

// The dense product with the A and B tiles loaded by global_load_lds_dwordx4
// into kStages LDS stages (no staging registers, no LDS store instructions):
// instruction i of wave w fills LDS bytes (w n + i) KiB + 16 lane of its
// tile, row r = 8 (w n + i) + lane/8, stored chunk lane%8, so the lane loads
// the logical chunk (lane%8) ^ ((r >> 1) & 7) of the swizzled layout.  One
// barrier per step, in its last 16-column slice, once every wave holds that
// slice's fragments: after it the first fragments of step ks + 1 and the
// loads of step ks + kStages (into the stage just released) are spread
// between the slice's products, so a load has kStages - 1 steps to arrive
// and the matrix cores do not wait for the first fragments of a step.
//
// kGlu: W holds the gate and up rows of a gated FFN interleaved (row 2c =
// gate channel c, row 2c+1 = up channel c; M = 2 x channels) and Y receives
// H (N x M/2), h = SiLU(g) * u rounded once to fp16, +0 where |h| < tau.  A
// lane's accumulator holds four consecutive rows of one token, so each
// gate / up pair meets in the same lane's registers.
template <int kWI, int kWJ, int kWM, int kWN, bool kGlu = false>
__global__ __launch_bounds__(64 * kWM * kWN) void dense_dma_kernel(PrefillArgs a) {
  using S = DmaShape<kWI, kWJ, kWM, kWN>;
  constexpr int kAT = S::kAT, kStage = kAT + S::kBTB;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  if (!tile_of(a, tm, tn)) return;
  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int m0 = tm * S::kBR, n0 = tn * S::kBT;
  const int nsteps = (a.K + BK - 1) / BK;
  const uint32_t base = lds_addr(smem);

  // per-lane sources (32-bit byte offsets; the launcher checks W and X fit 4 GiB)
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(a.W);
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.X);
  uint32_t aoff[S::kIA], boff[S::kIB];
  int acol[S::kIA], bcol[S::kIB];
#pragma unroll
  for (int i = 0; i < S::kIA; ++i) {
    const int r = 8 * (wave * S::kIA + i) + (lane >> 3);
    acol[i] = 8 * ((lane & 7) ^ ((r >> 1) & 7));
    aoff[i] = 2u * uint32_t(min(m0 + r, a.M - 1)) * uint32_t(a.ldw);  // rows past M: never stored
  }
#pragma unroll
  for (int i = 0; i < S::kIB; ++i) {
    const int r = 8 * (wave * S::kIB + i) + (lane >> 3);
    bcol[i] = 8 * ((lane & 7) ^ ((r >> 1) & 7));
    boff[i] = 2u * uint32_t(min(n0 + r, a.N - 1)) * uint32_t(a.ldx);  // tokens past N: never stored
  }
  const void* zero = g_pf_zero;
  asm volatile("" : "+s"(zero));  // address kept in registers, not reloaded every step
  // load q of step kq (A rows for q < kIA, else activations) into its stage;
  // past the end: the last step again, into a stage no later step reads (no
  // branch, and the per-step count of loads the waits assume is kept)
  auto issue_one = [&](int kq, int q) {
    uint8_t* sa = smem + (kq % S::kStages) * kStage;
    const int ks = min(kq, nsteps - 1);
    if (q < S::kIA) {
      // columns past K multiply zero activations: read a clamped in-row chunk
      const uint32_t kc = 2u * uint32_t(min(ks * BK + acol[q], a.K - 8));
      lds_dma16(wb + (aoff[q] + kc), sa + (wave * S::kIA + q) * 1024);
    } else {
      const int i = q - S::kIA;
      const int col = ks * BK + bcol[i];  // K % 8 == 0: a chunk is wholly inside or outside
      const void* src = col < a.K ? static_cast<const void*>(xb + (boff[i] + 2u * uint32_t(col))) : zero;
      lds_dma16(src, sa + kAT + (wave * S::kIB + i) * 1024);
    }
  };

  f32x16 acc[kWI][kWJ];
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < kWJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  half8 fa[2][kWI], fb[2][kWJ];
  // fragment q of a slice: A rows for q < kWI, else B tokens
  auto read_frag = [&](int stage, int kk, int slot, int q) {
    const uint32_t aBase = base + stage * kStage, bBase = aBase + kAT;
    const int ch = kk * 2 + (lane >> 5);
    if (q < kWI)
      fa[slot][q] = __builtin_bit_cast(half8, lds_load16(aBase + swz((wm * kWI + q) * 32 + (lane & 31), ch)));
    else
      fb[slot][q - kWI] =
          __builtin_bit_cast(half8, lds_load16(bBase + swz((wn * kWJ + q - kWI) * 32 + (lane & 31), ch)));
  };
  auto product = [&](int sl, int m) {
    const int i = m / kWJ, j = m % kWJ;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[sl][i], fb[sl][j], acc[i][j], 0, 0, 0);
  };
  constexpr int kI = S::kIA + S::kIB;  // loads per wave per step
  constexpr int kG = kWI + kWJ;        // fragment reads per slice
  constexpr int kM = kWI * kWJ;        // products per slice
  constexpr int kH = kM / 2;

  // Steps 0 .. kStages-1 fill every stage; step ks + kStages is requested in
  // step ks once every wave has read its last fragments of step ks.
#pragma unroll
  for (int p = 0; p < S::kStages; ++p)
#pragma unroll
    for (int q = 0; q < kI; ++q) issue_one(p, q);
  wait_vm_lgkm0<(S::kStages - 1) * kI>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kG; ++q) read_frag(0, 0, 0, q);
  __builtin_amdgcn_sched_barrier(0);

  // Each slice: its products in a fixed order, the next slice's fragment
  // reads (and in the last slice the loads of a later step) spread between
  // them; sched_barrier pins that order.
  for (int ks = 0; ks < nsteps; ++ks) {
    const int st = ks % S::kStages, nst = (ks + 1) % S::kStages;
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      const int sl = kk & 1;
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        product(sl, m);
        // all reads in the first half: they land before the next slice starts
#pragma unroll
        for (int q = m * kG / kH; q < (m + 1) * kG / kH && q < kG; ++q) read_frag(st, kk + 1, sl ^ 1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // last slice: one product, then the step's barrier (every fragment of
    // step ks is in registers, this wave's loads of step ks + 1 are in LDS;
    // after it both hold for all waves), then step ks + 1's first fragments
    // and step ks + kStages's loads between the remaining products
    product(1, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<(S::kStages - 2) * kI>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kE = kG + kI;  // reads first, then loads; none after the last two products
#pragma unroll
    for (int m = 1; m < kM; ++m) {
#pragma unroll
      for (int e = (m - 1) * kE / (kM - 2); e < m * kE / (kM - 2) && e < kE; ++e) {
        if (e < kG)
          read_frag(nst, 0, 0, e);  // unused after the last step
        else
          issue_one(ks + S::kStages, e - kG);
      }
      product(1, m);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue: fp16 round-to-nearest-even.  Each wave transposes its
  // 32 kWI x 32 kWJ quadrant through its own LDS region (a row per token,
  // padded by 8 bytes) so that the stores are 16 contiguous bytes per lane;
  // every wave's loads must have landed before any region is written.
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  // output rows per wave quadrant: 32 kWI, or half as many gated channels
  constexpr int kTM = kGlu ? 16 * kWI : 32 * kWI, kTN = 32 * kWJ, kRS = 2 * kTM + 8;
  const uint32_t reg = base + wave * (kTN * kRS);
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < kWJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = j * 32 + (lane & 31), m = i * 32 + q * 8 + (lane >> 5) * 4;
        if constexpr (kGlu) {
          // rows m, m+1 are gate / up of channel m/2, rows m+2, m+3 of m/2+1
          uint16_t h[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float g = acc[i][j][q * 4 + 2 * e], u = acc[i][j][q * 4 + 2 * e + 1];
            _Float16 v = _Float16(g / (1.f + expf(-g)) * u);
            if (!(fabsf(float(v)) >= a.tau)) v = _Float16(0.f);
            h[e] = __builtin_bit_cast(uint16_t, v);
          }
          *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(
              static_cast<uintptr_t>(reg + n * kRS + m)) = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
        } else {
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, _Float16(acc[i][j][q * 4 + e]));
          const u32x2 pk = {uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
          *reinterpret_cast<lds_u32x2*>(static_cast<uintptr_t>(reg + n * kRS + 2 * m)) = pk;
        }
      }
  constexpr int kLPR = kTM / 8;    // lanes per token row
  constexpr int kRPI = 64 / kLPR;  // rows per instruction
  const int Mo = kGlu ? a.M / 2 : a.M;  // rows (or gated channels) of Y
  const int gm = (kGlu ? m0 / 2 : m0) + wm * kTM + (lane % kLPR) * 8;
  const bool vec = (a.ldy % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.Y) & 15) == 0) && gm + 8 <= Mo;
#pragma unroll
  for (int r = 0; r < kTN; r += kRPI) {
    const int nl = r + lane / kLPR;
    const int n = n0 + wn * kTN + nl;
    const u32x4 v = lds_load16(reg + nl * kRS + (lane % kLPR) * 16);
    if (n >= a.N) continue;
    uint16_t* dst = a.Y + int64_t(n) * a.ldy + gm;
    if (vec) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      for (int e = 0; e < 8; ++e)
        if (gm + e < Mo) dst[e] = uint16_t(v[e / 2] >> (16 * (e % 2)));
    }
  }
}

// ------------------------------------------------------------------ sparse, warp-specialized
// 512 threads, eight waves, two per SIMD; the workgroup computes a 128 (rows
// of W) x 256 (tokens) block of Y.  Every wave expands one 16 x 64 weight
// tile per step (slab m0/16 + wave) into the next A stage; on top of that
//   * waves 0-3 (consumers) issue the products: consumer c owns tokens
//     64c .. 64c+63, 4 x 2 v_mfma_f32_32x32x16_f16 accumulators (128 fp32 per
//     lane).  Their expansion is spread one bitmap word per two products, so
//     it issues in the shadow of the matrix pipe;
//   * waves 4-7 (producers) stream the activations: the 256 x 64 tile of
//     step ks+1 is loaded during step ks-1 and stored into the free B stage
//     after the expansion.
// The expansion of a bitmap word is lane-parallel: each lane's rank by
// v_mbcnt, a halfword read at run base + 2 rank, and later a v_cndmask /
// SDWA v_cndmask that zeroes and packs two words' halves into one dword; a
// 16-byte store per 8 words.  Runs are fetched two steps ahead and copied
// into the wave's LDS buffer one step ahead.  One barrier per step:
// afterwards the next stage is complete (both operands) and the current one
// is free.  Both stages use the 16-row XOR swizzle of the dense kernel.
constexpr int WBM = 128, WBN = 256;
constexpr int kWATile = WBM * BK * 2;  // 16 KiB
constexpr int kWBTile = WBN * BK * 2;  // 32 KiB

template <int kRC>
__global__ __launch_bounds__(512, 1) void prefill_ws_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  if (!tile_of(a, tm, tn)) return;  // tiles_m / tiles_n count 128 x 256 blocks
  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = tm * WBM, n0 = tn * WBN;
  const int nsteps = (a.K + BK - 1) / BK;
  constexpr uint32_t tile_run_bytes = uint32_t(kRC) * 512u;
  const uint32_t sA = lds_addr(smem), sB = sA + 2 * kWATile;
  const uint32_t runbuf = sB + 2 * kWBTile + uint32_t(wave) * tile_run_bytes;

  // ---- the wave's weight tile: slab m0/16 + wave (clamped to the last slab:
  // rows past M are never stored), tile column ks (clamped: the last step
  // expands a duplicate into the unused stage).
  const int slab = min(m0 / 16 + wave, a.mt - 1);
  u32x2 runreg[kRC];
  uint32_t wreg = 0, wsave = 0;  // lane l: dword l%32 of the tile's 16 bitmap words
  // tile pointers: lane 0 / 1 hold the run's first / one-past-last index
  auto fetch_tp = [&](int ks) -> uint32_t {
    return a.tile_ptr[uint64_t(slab) * a.kt + min(ks, a.kt - 1) + (lane & 1)];
  };
  auto fetch_runs = [&](int ks, uint32_t tpv) {
    const uint32_t p0 = __builtin_amdgcn_readlane(tpv, 0);
    const uint32_t p1 = __builtin_amdgcn_readlane(tpv, 1);
    const uint32_t last = p1 > p0 + 4 ? p1 - 4 : p0;
#pragma unroll
    for (int cc = 0; cc < kRC; ++cc) {
      const uint32_t off = min(p0 + uint32_t(cc * 256 + lane * 4), last);
      runreg[cc] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.vals + off));
    }
    wreg = reinterpret_cast<const uint32_t*>(a.bits + (uint64_t(slab) * a.kt + min(ks, a.kt - 1)) * 16)[lane & 31];
  };
  auto stage_runs = [&]() {
#pragma unroll
    for (int cc = 0; cc < kRC; ++cc)
      *reinterpret_cast<lds_u32x2*>(static_cast<uintptr_t>(runbuf + cc * 512 + lane * 8)) = runreg[cc];
    wsave = wreg;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  // Word g (0..15) of the staged tile: bitmap word to SGPRs, lane rank, run
  // address, halfword read; `base` walks the run.
  struct Word {
    uint64_t w;
    uint32_t d;
  };
  auto issue_word = [&](int g, uint32_t& base, Word& x) {
    const uint32_t lo = __builtin_amdgcn_readlane(wsave, 2 * g);  // int: zero-extend via u32
    const uint32_t hi = __builtin_amdgcn_readlane(wsave, 2 * g + 1);
    x.w = uint64_t(lo) | (uint64_t(hi) << 32);
    const uint32_t r = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
    uint32_t nb, c, ad;
    asm("s_bcnt1_i32_b64 %1, %2\n\t"
        "s_lshl1_add_u32 %0, %1, %3"
        : "=&s"(nb), "=&s"(c)
        : "s"(x.w), "s"(base)
        : "scc");
    asm("v_lshl_add_u32 %0, %1, 1, %2" : "=v"(ad) : "v"(r), "s"(base));
    x.d = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(ad));
    base = nb;
  };
  // Pair p (words 2p, 2p+1): zero / pack into dword p%4 of unit p/4 (32-column
  // step s = p/4: rows 16 wave + l%16, chunk 4 s + l/16); store after p%4 = 3.
  auto finish_pair = [&](int stage, int p, const Word& x0, const Word& x1, u32x4& out) {
    uint32_t v;
    asm("v_cndmask_b32_e64 %0, 0, %1, %3\n\t"
        "s_mov_b64 vcc, %4\n\t"
        "v_cndmask_b32_sdwa %0, 0, %2, vcc dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:WORD_0"
        : "=&v"(v)
        : "v"(x0.d), "v"(x1.d), "s"(x0.w), "s"(x1.w)
        : "vcc");
    out[p & 3] = v;
    if ((p & 3) == 3)
      lds_store16(sA + stage * kWATile + swz(wave * 16 + (lane & 15), 4 * (p >> 2) + (lane >> 4)), out);
  };
  // Whole-tile expansion with one pair of reads in flight ahead of each finish.
  auto expand_all = [&](int stage) {
    Word x[16];
    u32x4 out;
    uint32_t base = runbuf;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      issue_word(g, base, x[g]);
      if ((g & 1) && g >= 3) finish_pair(stage, (g - 3) >> 1, x[g - 3], x[g - 2], out);
    }
    finish_pair(stage, 7, x[14], x[15], out);
  };

  // ---- producers: activations.  Thread pt moves 16-byte chunk pt%8 of rows
  // 32 r + pt/8 (tokens past N read token N-1; never stored).  32-bit byte
  // offsets into X (the launcher checks that X fits 4 GiB).
  const bool producer = wave >= 4;
  const int pt = tid - 256;
  const int frow = pt >> 3, fch = pt & 7;
  uint32_t xoff[8];
  u32x4 regB[8];
  auto fetch_B = [&](int ks) {
    const uint32_t kc = 2u * uint32_t(min(ks * BK + fch * 8, a.K - 8));  // past K the weights are zero
#pragma unroll
    for (int r = 0; r < 8; ++r)
      regB[r] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.X) + (xoff[r] + kc));
  };
  auto store_B = [&](int stage) {
#pragma unroll
    for (int r = 0; r < 8; ++r) lds_store16(sB + stage * kWBTile + swz(r * 32 + frow, fch), regB[r]);
  };

  // ---- prologue: stage 0 complete in LDS; runs and activations of step 1
  // and tile pointers of step 2 in flight.
  uint32_t tp_next = fetch_tp(2);
  {
    const uint32_t tp0 = fetch_tp(0), tp1 = fetch_tp(1);
    fetch_runs(0, tp0);
    if (producer) {
#pragma unroll
      for (int r = 0; r < 8; ++r) xoff[r] = 2u * uint32_t(min(n0 + r * 32 + frow, a.N - 1)) * uint32_t(a.ldx);
      fetch_B(0);
    }
    stage_runs();
    fetch_runs(1, tp1);
  }
  expand_all(0);
  if (producer) {
    store_B(0);
    fetch_B(min(1, nsteps - 1));
  }
  __syncthreads();

  if (!producer) {
    // ---------------------------------------------------------------- consumer
    const int c = wave;
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    for (int ks = 0; ks < nsteps; ++ks) {
      const int st = ks & 1;
      const uint32_t aBase = sA + st * kWATile, bBase = sB + st * kWBTile;
      stage_runs();  // runs/words of step ks+1 (fetched during step ks-1)
      const uint32_t tp_cur = tp_next;
      tp_next = fetch_tp(ks + 3);
      fetch_runs(ks + 2, tp_cur);
      half8 fa[2][4], fb[2][2];
      auto load_frag = [&](int kk, int slot, int f) {
        const int ch = kk * 2 + (lane >> 5);
        if (f < 4)
          fa[slot][f] = __builtin_bit_cast(half8, lds_load16(aBase + swz(f * 32 + (lane & 31), ch)));
        else
          fb[slot][f - 4] = __builtin_bit_cast(half8, lds_load16(bBase + swz(c * 64 + (f - 4) * 32 + (lane & 31), ch)));
      };
#pragma unroll
      for (int f = 0; f < 6; ++f) load_frag(0, 0, f);
      __builtin_amdgcn_sched_barrier(0);
      // Slot q of slice kk: product (q/2, q%2); the next slice's fragment q
      // (q < 6); word 4 kk + q/2 on even q; on q = 3, 7 the finish of pair
      // 2 (kk-1) + q/4, whose words were issued during the previous slice.
      Word x[16];
      u32x4 out;
      uint32_t base = runbuf;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int sl = kk & 1;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          acc[q >> 1][q & 1] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[sl][q >> 1], fb[sl][q & 1], acc[q >> 1][q & 1], 0, 0, 0);
          if (kk < 3 && q < 6) load_frag(kk + 1, sl ^ 1, q);
          if ((q & 1) == 0) issue_word(4 * kk + (q >> 1), base, x[4 * kk + (q >> 1)]);
          if ((q == 3 || q == 7) && kk > 0) {
            const int p = 2 * (kk - 1) + (q >> 2);
            finish_pair(st ^ 1, p, x[2 * p], x[2 * p + 1], out);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      finish_pair(st ^ 1, 6, x[12], x[13], out);
      finish_pair(st ^ 1, 7, x[14], x[15], out);
      __syncthreads();
    }

    // Epilogue: fp16 round-to-nearest-even, 4 consecutive rows per 8-byte store.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + c * 64 + j * 32 + (lane & 31);
        if (n >= a.N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + i * 32 + q * 8 + (lane >> 5) * 4;
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, _Float16(acc[i][j][q * 4 + e]));
          uint16_t* dst = a.Y + int64_t(n) * a.ldy + m;
          if (m + 3 < a.M && ((reinterpret_cast<uintptr_t>(dst) & 7) == 0)) {
            u32x2 pk = {uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
            *reinterpret_cast<u32x2*>(dst) = pk;
          } else {
            for (int e = 0; e < 4; ++e)
              if (m + e < a.M) dst[e] = h[e];
          }
        }
      }
  } else {
    // ---------------------------------------------------------------- producer
    for (int ks = 0; ks < nsteps; ++ks) {
      const int st = ks & 1;
      stage_runs();  // runs/words of step ks+1 (fetched during step ks-1)
      const uint32_t tp_cur = tp_next;
      tp_next = fetch_tp(ks + 3);
      fetch_runs(ks + 2, tp_cur);
      expand_all(st ^ 1);
      store_B(st ^ 1);  // activations of step ks+1 (clamped past the end)
      fetch_B(min(ks + 2, nsteps - 1));
      __syncthreads();
    }
  }
}

PrefillArgs make_args(int64_t M, int64_t N, int64_t K, const uint16_t* X, int64_t ldx, uint16_t* Y,
                      int64_t ldy) {
  PrefillArgs a{};
  a.X = X;
  a.Y = Y;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int(M);
  a.N = int(N);
  a.K = int(K);
  a.tiles_m = int((M + BM - 1) / BM);
  a.tiles_n = int((N + BN - 1) / BN);
  a.group_m = 8;
  return a;
}

unsigned grid_size(const PrefillArgs& a) {
  const int total = a.tiles_m * a.tiles_n;
  return unsigned((total + 7) / 8 * 8);
}

}  // namespace

bool prefill_supported(int64_t K, int64_t ldx, const void* X) {
  return K >= 8 && (K % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
}

bool prefill_sparse_fits(const Header& h, int64_t N, int64_t ldx) {
  return 2 * ((N - 1) * ldx + h.k) < (int64_t(1) << 32);  // 32-bit activation offsets
}

namespace {
template <int kWI, int kWJ, bool kGlu = false>
hipError_t launch_dense(PrefillArgs a, hipStream_t s) {
  a.tiles_m = int((a.M + 64 * kWI - 1) / (64 * kWI));
  a.tiles_n = int((a.N + 64 * kWJ - 1) / (64 * kWJ));
  // The LDS-direct kernel where W and X fit 32-bit byte offsets; otherwise
  // (or with SWM_DENSE_DMA=0) the register-staged one.
  static const bool dma = [] {
    const char* e = getenv("SWM_DENSE_DMA");
    return !(e && *e == '0');
  }();
  const bool fits = 2 * (int64_t(a.M - 1) * a.ldw + a.K) < (int64_t(1) << 32) &&
                    2 * (int64_t(a.N - 1) * a.ldx + a.K) < (int64_t(1) << 32);
  if (kGlu && !fits) return hipErrorInvalidValue;  // the gated epilogue exists in this kernel only
  if (kGlu || (dma && fits)) {
    // 256 x 256 with eight waves (two per SIMD, 128 x 64 each); the smaller
    // blocks with four
    constexpr int kWN = kWI == 4 && kWJ == 4 ? 4 : 2;
    constexpr int kJ = kWI == 4 && kWJ == 4 ? 2 : kWJ;
    using S = DmaShape<kWI, kJ, 2, kWN>;
    hipLaunchKernelGGL((dense_dma_kernel<kWI, kJ, 2, kWN, kGlu>), dim3(grid_size(a)), dim3(64 * S::kNW), S::kLds,
                       s, a);
    return hipGetLastError();
  }
  const size_t lds = size_t(2) * (64 * kWI + 64 * kWJ) * BK * 2;
  hipLaunchKernelGGL((dense_kernel<kWI, kWJ>), dim3(grid_size(a)), dim3(256), lds, s, a);
  return hipGetLastError();
}
}  // namespace

namespace {
hipError_t launch_dense_any(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx, uint16_t* Y,
                            int64_t ldy, int64_t M, int64_t K, int64_t N, int num_cus, bool glu, float tau,
                            hipStream_t s) {
  PrefillArgs a = make_args(M, N, K, X, ldx, Y, ldy);
  a.W = W;
  a.ldw = ldw;
  a.tau = tau;
  if (glu && M % 2 != 0) return hipErrorInvalidValue;
  if (a.tiles_m == 0 || a.tiles_n == 0) return hipSuccess;
  if (K < 8 || K % 8 != 0) return hipErrorInvalidValue;
  // Block shape 256 x 256, 256 x 128 or 128 x 128: the one with the fewest
  // rounds of blocks over the CUs, each round weighted by its block's
  // measured time relative to 256 x 256 (1, 0.73, 0.54 on up/gate
  // 11008x4096).  A shape whose blocks spill a few past one round loses to a
  // larger one (N = 768: 258 blocks of 256 x 128 took 153 us, 129 of
  // 256 x 256 109 us).  SWM_DENSE_BLOCK = 1 / 2 / 3 forces one.
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  const int64_t mb = (M + 255) / 256, mb128 = (M + 127) / 128;
  const int64_t blocks[3] = {mb * ((N + 255) / 256), mb * ((N + 127) / 128), mb128 * ((N + 127) / 128)};
  const double weight[3] = {1.0, 0.73, 0.54};
  int shape = 1;
  double best = 0.0;
  for (int i = 0; i < 3; ++i) {
    const double cost = double((blocks[i] + cus - 1) / cus) * weight[i];
    if (i == 0 || cost < best) {
      best = cost;
      shape = i + 1;
    }
  }
  if (const char* e = getenv("SWM_DENSE_BLOCK")) {
    if (*e >= '1' && *e <= '3') shape = *e - '0';
  }
  if (glu) {
    if (shape == 1) return launch_dense<4, 4, true>(a, s);
    if (shape == 2) return launch_dense<4, 2, true>(a, s);
    return launch_dense<2, 2, true>(a, s);
  }
  if (shape == 1) return launch_dense<4, 4>(a, s);
  if (shape == 2) return launch_dense<4, 2>(a, s);
  return launch_dense<2, 2>(a, s);
}
}  // namespace

hipError_t launch_prefill_dense(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx,
                                uint16_t* Y, int64_t ldy, int64_t M, int64_t K, int64_t N, int num_cus,
                                hipStream_t s) {
  return launch_dense_any(W, ldw, X, ldx, Y, ldy, M, K, N, num_cus, false, 0.f, s);
}

hipError_t launch_prefill_dense_glu(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx,
                                    uint16_t* H, int64_t ldh, int64_t M2, int64_t K, int64_t N, float tau,
                                    int num_cus, hipStream_t s) {
  return launch_dense_any(W, ldw, X, ldx, H, ldh, M2, K, N, num_cus, true, tau, s);
}

bool prefill_dense_dma_fits(int64_t M, int64_t ldw, int64_t K, int64_t N, int64_t ldx) {
  return 2 * ((M - 1) * ldw + K) < (int64_t(1) << 32) && 2 * ((N - 1) * ldx + K) < (int64_t(1) << 32);
}

size_t prefill_sparse_lds(const Header& h) {
  const size_t chunks = std::max<size_t>((size_t(h.max_tile) + 255) / 256, 1);  // 512-byte chunks per tile run
  return size_t(2) * kWATile + size_t(2) * kWBTile + 8 /*waves*/ * chunks * 512;
}

hipError_t launch_prefill_sparse(const DevFormat& f, const uint16_t* X, int64_t ldx, uint16_t* Y,
                                 int64_t ldy, int64_t N, hipStream_t s) {
  PrefillArgs a = make_args(f.h.m, N, f.h.k, X, ldx, Y, ldy);
  a.tile_ptr = f.tile_ptr;
  a.bits = f.bits;
  a.vals = f.vals;
  a.kt = int(f.h.kt);
  a.mt = int(f.h.mt);
  a.run_chunks = int((f.h.max_tile + 255) / 256);
  if (a.run_chunks < 1) a.run_chunks = 1;
  if (f.h.tm != 16 || f.h.tk != 64 || f.h.max_tile > 1024 || f.h.k < 8 || f.h.k % 8 != 0)
    return hipErrorInvalidValue;
  if (a.tiles_m == 0 || a.tiles_n == 0) return hipSuccess;
  const size_t lds = prefill_sparse_lds(f.h);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (!prefill_sparse_fits(f.h, N, ldx)) return hipErrorInvalidValue;
  a.tiles_m = int((f.h.m + WBM - 1) / WBM);
  a.tiles_n = int((N + WBN - 1) / WBN);
  const dim3 grid{grid_size(a), 1, 1}, block{512, 1, 1};
  switch (a.run_chunks) {
    case 1: hipLaunchKernelGGL((prefill_ws_kernel<1>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_ws_kernel<2>), grid, block, lds, s, a); break;
    case 3: hipLaunchKernelGGL((prefill_ws_kernel<3>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((prefill_ws_kernel<4>), grid, block, lds, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace swm
