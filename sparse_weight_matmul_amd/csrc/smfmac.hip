// Prefill on the sparse matrix cores: W (.) mask split into a 2:4 layer and a
// residual layer, both multiplied by v_smfmac_f32_32x32x32_f16.
//
// Method: "Accelerating GPU inference of LLMs with moderately unstructured
// sparse weight matrices", abstract and Sec. 1 (Challenge 1): at moderate
// sparsity the kept weights are split into a layer the sparse tensor cores
// can run (2 of every 4 consecutive weights along K) and a residual layer
// that keeps the product exact.  On gfx950 the sparse matrix instruction is
// v_smfmac_f32_32x32x32_f16: A is 32 rows x 32 columns of which each row
// keeps at most 2 of every 4 (stored as 16 values and a 2-bit position per
// value), B is dense 32 x 32, and it issues at the rate of the dense
// v_mfma_f32_32x32x16_f16, i.e. twice the dense work per instruction.
//
// Split.  In every group of 4 consecutive columns of a row (aligned to 4),
// the first two kept entries (by column) go to the 2:4 layer and the others
// (at most two) to the residual layer, which is therefore 2:4 conforming as
// well.  Each kept entry lands in exactly one layer, so the two products add
// up to the masked product; both accumulate into the same fp32 registers.  A
// group with fewer than two entries in a layer is filled with +0 at unused
// positions (the two positions of a group are distinct and ascending).
//
// Operand layout (measured on gfx950 with an exact-integer probe): lane l of
// the A operand holds row l%32 and, for q = l/32, the compressed values of
// columns 16q .. 16q+15 of the 32-column slice, 2 per group of 4 in group
// order, with the in-group position of value i in bits 2i+1..2i of the index
// operand; lane l of B holds column (token) l%32 and slice rows
// 8q + (j%8) + 16 (j/8), j = 0..15; the accumulator is laid out as for the
// dense 32x32 instruction.
//
// Layout in the caller's workspace (row-major, Kp = K rounded up to 64):
// values [M][Kp/2] fp16 (group g of a row at 2g, 2g+1) and indices
// [M][Kp/16] uint16 (the 4 groups of a 16-column chunk, 4 bits each); the
// residual layer follows in the same layout when the mask has one.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "kernels.h"

namespace swm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kTK = 64;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr) {
  return *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(addr));
}
template <typename T>
__device__ __forceinline__ T const_load(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(p));
}

// ------------------------------------------------------------------ compaction
struct CompactArgs {
  const uint32_t* tile_ptr;
  const uint64_t* bits;
  const uint16_t* vals;
  uint16_t* v24;   // [M][ldv]
  uint16_t* m24;   // [M][ldm]
  uint16_t* vres;  // residual layer (nullptr: the mask has none)
  uint16_t* mres;
  int64_t ldv, ldm;
  int M, kt;
  int64_t tiles;
};

// One wave per 16 x 64 tile (four per workgroup).  The tile's run and its 16
// bitmap words are read as in the expansion kernel; every kept entry is
// placed in an LDS tile of values and a byte tile of kept flags; then lane l
// takes row l/4 and the 16-column chunk l%4 (four groups) and writes its
// 8 values (16 bytes) and its 16-bit index word of each layer.
__global__ __launch_bounds__(256) void compact24_kernel(CompactArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t run[4][1024];
  // rows padded to 33 and 17 dwords: the 16 rows of a column fall in distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t tv[4][16][66];
  __shared__ __attribute__((aligned(16))) uint8_t tf[4][16][68];
  const int lane = int(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= a.tiles) return;  // uniform per wave; no barrier below
  const int slab = int(t / a.kt), tj = int(t % a.kt);
  const uint32_t p0 = const_load<uint32_t>(a.tile_ptr + t);
  const uint32_t n = const_load<uint32_t>(a.tile_ptr + t + 1) - p0;  // multiple of 8, <= 1024
  const u32x16 wa = const_load<u32x16>(a.bits + t * 16);
  const u32x16 wb = const_load<u32x16>(a.bits + t * 16 + 8);
  u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
  if (uint32_t(lane) * 8u < n) v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vals + p0 + lane * 8));
  if (512u + uint32_t(lane) * 8u < n)
    v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vals + p0 + 512 + lane * 8));
  *reinterpret_cast<u32x4*>(&run[wave][lane * 8]) = v0;
  *reinterpret_cast<u32x4*>(&run[wave][512 + lane * 8]) = v1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t pos = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t lo = (w < 8 ? wa : wb)[2 * (w & 7)], hi = (w < 8 ? wa : wb)[2 * (w & 7) + 1];
    const uint64_t word = uint64_t(lo) | (uint64_t(hi) << 32);
    const bool set = (word >> lane) & 1ull;
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
    const int col = 32 * (w >> 3) + 8 * (lane >> 4) + (w & 7);
    tv[wave][lane & 15][col] = set ? run[wave][min(pos + rank, 1023u)] : uint16_t(0);
    tf[wave][lane & 15][col] = set ? uint8_t(1) : uint8_t(0);
    pos += uint32_t(__builtin_popcountll(word));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int r = lane >> 2, c = lane & 3;
  const int64_t row = int64_t(slab) * 16 + r;
  if (row >= a.M) return;
  uint32_t out24[4], outr[4], idx24 = 0, idxr = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c0 = 16 * c + 4 * g;
    // kept positions of the group in column order: the first two to the 2:4
    // layer, the rest to the residual layer
    int p24[2] = {-1, -1}, pr[2] = {-1, -1};
    int k = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (tf[wave][r][c0 + e]) {
        if (k < 2) p24[k] = e;
        else pr[k - 2] = e;
        ++k;
      }
    }
    // two ascending distinct positions per layer, unused ones filled with +0
    auto place = [&](const int (&p)[2], uint32_t& packed, uint32_t& nib) {
      int lo = p[0], hi = p[1];
      if (lo < 0) {
        lo = 0;
        hi = 1;
      } else if (hi < 0) {
        hi = lo == 3 ? 3 : lo + 1;
        if (lo == 3) lo = 2;
      }
      const uint32_t vlo = (lo == p[0] || lo == p[1]) ? tv[wave][r][c0 + lo] : 0u;
      const uint32_t vhi = (hi == p[0] || hi == p[1]) ? tv[wave][r][c0 + hi] : 0u;
      packed = vlo | (vhi << 16);
      nib = uint32_t(lo) | (uint32_t(hi) << 2);
    };
    uint32_t nb;
    place(p24, out24[g], nb);
    idx24 |= nb << (4 * g);
    place(pr, outr[g], nb);
    idxr |= nb << (4 * g);
  }
  const int64_t vo = row * a.ldv + int64_t(tj) * 32 + c * 8;
  const int64_t mo = row * a.ldm + int64_t(tj) * 4 + c;
  *reinterpret_cast<u32x4*>(a.v24 + vo) = u32x4{out24[0], out24[1], out24[2], out24[3]};
  a.m24[mo] = uint16_t(idx24);
  if (a.vres) {
    *reinterpret_cast<u32x4*>(a.vres + vo) = u32x4{outr[0], outr[1], outr[2], outr[3]};
    a.mres[mo] = uint16_t(idxr);
  }
}

// ------------------------------------------------------------------ SMFMAC GEMM
struct SmfArgs {
  const uint16_t* v24;
  const uint16_t* m24;
  const uint16_t* vres;
  const uint16_t* mres;
  const uint16_t* X;
  uint16_t* Y;
  int64_t ldv, ldm, ldx, ldy;
  int M, N, K, Kp;
  int tiles_m, tiles_n, group_m;
};

__device__ __forceinline__ bool smf_tile_of(const SmfArgs& a, int& tm, int& tn) {
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

// B tile (256 tokens x 64 columns fp16): the dense kernels' swizzle, 8 chunks
// of 16 bytes per row permuted by bits 1..3 of the row.
__device__ __forceinline__ uint32_t swz_b(int row, int chunk) {
  return uint32_t(row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4));
}
// A values tile (256 rows x 32 compressed values = 64 bytes per row): 4 chunks
// per row permuted by bits 2..3 of the row, so 16 consecutive rows reading the
// same chunk hit 16 distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t swz_a(int row, int chunk) {
  return uint32_t(row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4));
}

constexpr int SBM = 256, SBK = 64;
constexpr int kSA = SBM * SBK;       // values bytes per stage (32 halves per row)
constexpr int kSM = SBM * 8;         // index bytes per stage (4 uint16 per row)
// Block of 256 rows x 64 kWJ tokens: waves 2 x kWN, each 4 x kJ accumulators
// of 32 x 32 (kJ = 2 kWJ / kWN).  kWJ = 4 (256 x 256) or 2 (256 x 128, for
// token counts that leave 256 x 256 blocks short of the CUs).  kWN = 2: four
// waves of 128 x 32 kWJ; kWN = 4 (256 x 256 only): eight waves of 128 x 64,
// two per SIMD.
template <bool kRes, int kWJ, int kWN = 2>
struct SmfShape {
  static constexpr int kNW = 2 * kWN;           // waves
  static constexpr int kJ = 2 * kWJ / kWN;      // accumulator columns per wave
  static constexpr int kBN = 64 * kWJ;          // tokens per block
  static constexpr int kSB = kBN * SBK * 2;     // activation bytes per stage
  static constexpr int kIV = kSA / (1024 * kNW);  // value loads per wave per step (per layer)
  static constexpr int kII = kSM / (256 * kNW);   // index loads per wave per step (per layer)
  static constexpr int kIB = kSB / (1024 * kNW);  // activation loads per wave per step
  static_assert(kIV * 1024 * kNW == kSA && kII * 256 * kNW == kSM && kIB * 1024 * kNW == kSB && kJ >= 1,
                "whole loads per wave");
  static constexpr int kStage = kSA + kSM + (kRes ? kSA + kSM : 0) + kSB;
  static constexpr int kStages = 3 * kStage <= 160 * 1024 ? 3 : 2;  // LDS stages
  static constexpr int kOps = (kIV + kII) * (kRes ? 2 : 1) + kIB;  // LDS-direct loads per wave per step
  static constexpr int kEpi = kNW * (32 * kJ) * (2 * 128 + 8);  // epilogue: one transposing region per wave
  static constexpr int kLds = kStages * kStage > kEpi ? kStages * kStage : kEpi;
  static_assert(kLds <= 160 * 1024, "LDS");
};

// Sixteen zero bytes: the source of activation chunks past K.
__device__ __attribute__((aligned(16))) uint16_t g_smf_zero[8];

// Global -> LDS without registers: lane l writes 16 (or 4) bytes at
// lds + 16 l (or 4 l); `lds` must be the same for every lane of the wave.
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// s_waitcnt: at most n vector memory operations of this wave outstanding, and
// every LDS operation complete (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at 7, lgkmcnt 11:8 = 0).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (((n >> 4) & 3) << 14));
}

// Waves in a 2 x kWN layout (SmfShape), each owning 4 x kJ accumulators of
// 32 x 32 (a 128-row x 32 kJ-token part of the output block); 64-column K
// steps in two 32-column slices.  The tiles go from global memory straight
// into LDS (global_load_lds_dwordx4 / _dword: lane l of an instruction writes
// 16 or 4 bytes at LDS base + 16l or 4l, so each lane loads the chunk that
// the swizzled layout places there) and need no staging registers.  The
// tiles of step ks + kStages - 1 are requested right after the barrier that
// opens step ks, so each load has kStages - 1 steps of products to arrive;
// the wait before that barrier is explicit: at most the later steps' loads
// may still be in flight.  kRes: the residual layer is staged and multiplied
// too, into the same accumulators.
template <bool kRes, int kWJ, int kWN = 2>
__global__ __launch_bounds__(128 * kWN) void smf_kernel(SmfArgs a) {
  using S = SmfShape<kRes, kWJ, kWN>;
  constexpr int kJ = S::kJ, kIV = S::kIV, kII = S::kII;
  constexpr int kStage = S::kStage;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  if (!smf_tile_of(a, tm, tn)) return;
  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int m0 = tm * SBM, n0 = tn * S::kBN;
  // stage layout: values | indices | [residual values | residual indices] | activations
  auto oV = [&](int st) { return uint32_t(st * kStage); };
  auto oI = [&](int st) { return uint32_t(st * kStage + kSA); };
  auto oVr = [&](int st) { return uint32_t(st * kStage + kSA + kSM); };
  auto oIr = [&](int st) { return uint32_t(st * kStage + 2 * kSA + kSM); };
  auto oB = [&](int st) { return uint32_t(st * kStage + kSA + kSM + (kRes ? kSA + kSM : 0)); };
  const uint32_t base = lds_addr(smem);
  const int nsteps = a.Kp / SBK;

  // Per-lane sources of the LDS-direct loads (32-bit byte offsets; the
  // launcher checks that every operand fits 4 GiB).
  //  values: instruction i of wave w fills LDS bytes (kIV w + i) KiB + 16
  //    lane: row r = 16 (kIV w + i) + lane/4, stored chunk lane%4 = logical
  //    chunk (lane%4) ^ ((r >> 2) & 3);
  //  indices: instruction i fills (kII w + i) * 256 + 4 lane: row
  //    32 (kII w + i) + lane/2, dword lane%2 of the row's 8 bytes;
  //  activations: instruction i fills (8w + i) KiB + 16 lane: token
  //    r = 8 (8w + i) + lane/8, stored chunk lane%8 = logical chunk
  //    (lane%8) ^ ((r >> 1) & 7).
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.X);
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v24);
  const uint8_t* vrb = reinterpret_cast<const uint8_t*>(a.vres);
  const uint8_t* mb = reinterpret_cast<const uint8_t*>(a.m24);
  const uint8_t* mrb = reinterpret_cast<const uint8_t*>(a.mres);
  uint32_t voff[kIV], ioff[kII], xoff[S::kIB];
  int xcol[S::kIB];
#pragma unroll
  for (int i = 0; i < kIV; ++i) {
    const int r = 16 * (kIV * wave + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    voff[i] = 2u * uint32_t(min(m0 + r, a.M - 1)) * uint32_t(a.ldv) + 16u * uint32_t(c);
  }
#pragma unroll
  for (int i = 0; i < kII; ++i) {
    const int r = 32 * (kII * wave + i) + (lane >> 1);
    ioff[i] = 2u * uint32_t(min(m0 + r, a.M - 1)) * uint32_t(a.ldm) + 4u * uint32_t(lane & 1);
  }
#pragma unroll
  for (int i = 0; i < S::kIB; ++i) {
    const int r = 8 * (S::kIB * wave + i) + (lane >> 3);
    xcol[i] = 8 * ((lane & 7) ^ ((r >> 1) & 7));
    xoff[i] = 2u * uint32_t(min(n0 + r, a.N - 1)) * uint32_t(a.ldx) + 2u * uint32_t(xcol[i]);
  }
  // load o of step kq: values, indices, [residual values, residual
  // indices,] activations last.  Past the end: a reload of the last step
  // into the stage of step kq, which no later step reads.
  auto issue_op = [&](int kq, int o) {
    const int st = kq % S::kStages;
    const int ks = min(kq, nsteps - 1);
    const uint32_t vk = 64u * uint32_t(ks), mk = 8u * uint32_t(ks);
    constexpr int kL = kIV + kII;            // loads of one layer
    constexpr int kB0 = kRes ? 2 * kL : kL;  // first activation load
    if (o < kIV) {
      lds_dma16(vb + (voff[o] + vk), smem + oV(st) + (kIV * wave + o) * 1024);
    } else if (o < kL) {
      lds_dma4(mb + (ioff[o - kIV] + mk), smem + oI(st) + (kII * wave + o - kIV) * 256);
    } else if (kRes && o < kL + kIV) {
      lds_dma16(vrb + (voff[o - kL] + vk), smem + oVr(st) + (kIV * wave + o - kL) * 1024);
    } else if (kRes && o < 2 * kL) {
      lds_dma4(mrb + (ioff[o - kL - kIV] + mk), smem + oIr(st) + (kII * wave + o - kL - kIV) * 256);
    } else {
      const int i = o - kB0;
      const bool in = ks * SBK + xcol[i] < a.K;  // K % 8 == 0: a chunk is wholly inside or outside
      const void* src = in ? static_cast<const void*>(xb + (xoff[i] + 128u * uint32_t(ks)))
                           : static_cast<const void*>(g_smf_zero);
      lds_dma16(src, smem + oB(st) + (S::kIB * wave + i) * 1024);
    }
  };
  auto issue = [&](int kq) {
#pragma unroll
    for (int o = 0; o < S::kOps; ++o) issue_op(kq, o);
  };

  f32x16 acc[4][kJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int q = lane >> 5, lr = lane & 31;
  // Fragments by slice (slot s = slice s of a step): compressed A values of
  // both layers, B as two 16-byte halves, and one 8-byte index read per row
  // holding both slices' index words.
  half8 fa[2][4], far_[2][4];
  half16 fb[2][kJ];
  u32x2 iv[4], ivr[4];
  auto read_a = [&](int st, int s, int i) {
    const int row = (wm * 4 + i) * 32 + lr;
    fa[s][i] = __builtin_bit_cast(half8, lds_load16(base + oV(st) + swz_a(row, 2 * s + q)));
    if constexpr (kRes) far_[s][i] = __builtin_bit_cast(half8, lds_load16(base + oVr(st) + swz_a(row, 2 * s + q)));
  };
  auto read_b = [&](int st, int s, int j) {
    // tokens (wn*4 + j)*32 + lr, slice rows 8q .. +7 and 16 + 8q .. +7
    const int tok = (wn * kJ + j) * 32 + lr;
    const u32x4 lo = lds_load16(base + oB(st) + swz_b(tok, 4 * s + q));
    const u32x4 hi = lds_load16(base + oB(st) + swz_b(tok, 4 * s + 2 + q));
    fb[s][j] = __builtin_bit_cast(half16, u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  auto read_i = [&](int st, int i) {
    const int row = (wm * 4 + i) * 32 + lr;
    iv[i] = *reinterpret_cast<const lds_u32x2*>(static_cast<uintptr_t>(base + oI(st) + row * 8));
    if constexpr (kRes) ivr[i] = *reinterpret_cast<const lds_u32x2*>(static_cast<uintptr_t>(base + oIr(st) + row * 8));
  };
  // read unit u of a slice: A rows i = u (u < 4), else B tokens j = u - 4
  auto read_unit = [&](int st, int s, int u) {
    if (u < 4) read_a(st, s, u);
    else read_b(st, s, u - 4);
  };
  // index word of slice s for lane half q: uint16 number 2s + q of the row
  auto idx = [&](const u32x2& v, int s) { return int((v[s] >> (16 * q)) & 0xFFFFu); };
  int x1[4], x1r[4];  // slice 1's index words, kept while the next step's are read
  auto product = [&](int s, int m, const int* xi, const int* xr) {
    const int i = m / kJ, j = m % kJ;
    acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(fa[s][i], fb[s][j], acc[i][j], xi[i], 0, 0);
    if constexpr (kRes)
      acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(far_[s][i], fb[s][j], acc[i][j], xr[i], 0, 0);
  };
  constexpr int kRead = 4 + kJ;            // read units per slice (4 A, kJ B)
  constexpr int kM = 4 * kJ;               // products per slice
  constexpr int kNext = 4 + kRead;         // step ks + 1: 4 index units, then slice 0's read units

  // Steps 0 .. kStages-1 fill every stage; step ks + kStages is requested in
  // step ks once every wave holds its last fragments of step ks.
#pragma unroll
  for (int p = 0; p < S::kStages; ++p) issue(p);
  wait_vm_lgkm0<(S::kStages - 1) * S::kOps>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) read_i(0, i);
#pragma unroll
  for (int u = 0; u < kRead; ++u) read_unit(0, 0, u);
  __builtin_amdgcn_sched_barrier(0);

  // Per step: slice 0's products with slice 1's reads in their first half;
  // slice 1's first product, the step's barrier (slice 1's fragments are in
  // registers, this wave's loads of step ks + 1 are in LDS; after it both
  // hold for every wave), then step ks + 1's index and slice-0 reads and the
  // loads of step ks + kStages (into the stage just released) between the
  // remaining products.  sched_barrier pins the order.
  for (int ks = 0; ks < nsteps; ++ks) {
    const int st = ks % S::kStages, nst = (ks + 1) % S::kStages;
    int x0[4], x0r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x0[i] = idx(iv[i], 0);
      x1[i] = idx(iv[i], 1);
      if constexpr (kRes) {
        x0r[i] = idx(ivr[i], 0);
        x1r[i] = idx(ivr[i], 1);
      }
    }
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      product(0, m, x0, x0r);
      // all reads in the first half: they land before slice 1 starts
#pragma unroll
      for (int u = m * kRead / (kM / 2); u < (m + 1) * kRead / (kM / 2) && u < kRead; ++u) read_unit(st, 1, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    product(1, 0, x1, x1r);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lgkm0<(S::kStages - 2) * S::kOps>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // reads first, then the loads; none after the last two products
    constexpr int kE = kNext + S::kOps;
#pragma unroll
    for (int m = 1; m < kM; ++m) {
#pragma unroll
      for (int e = (m - 1) * kE / (kM - 2); e < m * kE / (kM - 2) && e < kE; ++e) {
        if (e < 4)
          read_i(nst, e);  // unused after the last step
        else if (e < kNext)
          read_unit(nst, 0, e - 4);
        else
          issue_op(ks + S::kStages, e - kNext);
      }
      product(1, m, x1, x1r);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Epilogue: fp16 round-to-nearest-even.  Each wave transposes its 128 x
  // 32 kJ part through its own LDS region (a row per token, padded by 8 bytes)
  // so that the stores are 16 contiguous bytes per lane; every wave's loads
  // must have landed before any region is written.
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  constexpr int kRS = 2 * 128 + 8, kTN = 32 * kJ;
  const uint32_t reg = base + wave * (kTN * kRS);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int n = j * 32 + (lane & 31), m = i * 32 + qq * 8 + (lane >> 5) * 4;
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = __builtin_bit_cast(uint16_t, _Float16(acc[i][j][qq * 4 + e]));
        *reinterpret_cast<lds_u32x2*>(static_cast<uintptr_t>(reg + n * kRS + 2 * m)) =
            u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
      }
  const int gm = m0 + wm * 128 + (lane & 15) * 8;
  const bool vec = (a.ldy % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.Y) & 15) == 0) && gm + 8 <= a.M;
#pragma unroll
  for (int r = 0; r < kTN; r += 4) {
    const int nl = r + (lane >> 4);
    const int n = n0 + wn * kTN + nl;
    const u32x4 v = lds_load16(reg + nl * kRS + (lane & 15) * 16);
    if (n >= a.N) continue;
    uint16_t* dst = a.Y + int64_t(n) * a.ldy + gm;
    if (vec) {
      *reinterpret_cast<u32x4*>(dst) = v;
    } else {
      for (int e = 0; e < 8; ++e)
        if (gm + e < a.M) dst[e] = uint16_t(v[e / 2] >> (16 * (e % 2)));
    }
  }
}

}  // namespace

Sparse24Layout sparse24_layout(const Header& h, bool residual) {
  Sparse24Layout L;
  L.kp = (h.k + 63) / 64 * 64;
  L.ldv = L.kp / 2;
  L.ldm = L.kp / 16;
  const size_t vb = (size_t(h.m) * L.ldv * 2 + 255) / 256 * 256;
  const size_t mb = (size_t(h.m) * L.ldm * 2 + 255) / 256 * 256;
  L.off_m24 = vb;
  L.off_vres = residual ? vb + mb : 0;
  L.off_mres = residual ? 2 * vb + mb : 0;
  L.bytes = residual ? 2 * (vb + mb) : vb + mb;
  return L;
}

hipError_t launch_compact24(const DevFormat& f, const Sparse24Layout& L, bool residual, void* ws, hipStream_t s) {
  if (f.h.tm != 16 || f.h.tk != uint32_t(kTK)) return hipErrorInvalidValue;
  CompactArgs a;
  a.tile_ptr = f.tile_ptr;
  a.bits = f.bits;
  a.vals = f.vals;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.v24 = reinterpret_cast<uint16_t*>(w);
  a.m24 = reinterpret_cast<uint16_t*>(w + L.off_m24);
  a.vres = residual ? reinterpret_cast<uint16_t*>(w + L.off_vres) : nullptr;
  a.mres = residual ? reinterpret_cast<uint16_t*>(w + L.off_mres) : nullptr;
  a.ldv = L.ldv;
  a.ldm = L.ldm;
  a.M = int(f.h.m);
  a.kt = int(f.h.kt);
  a.tiles = int64_t(f.h.mt) * f.h.kt;
  if (a.tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(compact24_kernel, dim3(unsigned((a.tiles + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

bool smf_fits(const Header& h, int64_t N, int64_t ldx) {
  const int64_t kp = (h.k + 63) / 64 * 64;
  return 2 * ((N - 1) * ldx + h.k) < (int64_t(1) << 32) && h.m * kp < (int64_t(1) << 32);
}

hipError_t launch_smf(const Header& h, const Sparse24Layout& L, bool residual, const void* ws, const uint16_t* X,
                      int64_t ldx, uint16_t* Y, int64_t ldy, int64_t N, int num_cus, hipStream_t s) {
  if (h.k < 8 || h.k % 8 != 0 || N < 1 || !smf_fits(h, N, ldx)) return hipErrorInvalidValue;
  SmfArgs a;
  const uint8_t* w = static_cast<const uint8_t*>(ws);
  a.v24 = reinterpret_cast<const uint16_t*>(w);
  a.m24 = reinterpret_cast<const uint16_t*>(w + L.off_m24);
  a.vres = residual ? reinterpret_cast<const uint16_t*>(w + L.off_vres) : nullptr;
  a.mres = residual ? reinterpret_cast<const uint16_t*>(w + L.off_mres) : nullptr;
  a.X = X;
  a.Y = Y;
  a.ldv = L.ldv;
  a.ldm = L.ldm;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int(h.m);
  a.N = int(N);
  a.K = int(h.k);
  a.Kp = int(L.kp);
  a.tiles_m = int((h.m + SBM - 1) / SBM);
  a.group_m = 8;
  if (a.tiles_m == 0) return hipSuccess;
  // 256 x 256 blocks when they give every CU one (or more than a round),
  // else 256 x 128 (twice the blocks)
  const int64_t big = int64_t(a.tiles_m) * ((N + 255) / 256);
  const bool wide = big >= num_cus;
  a.tiles_n = int(wide ? (N + 255) / 256 : (N + 127) / 128);
  const unsigned grid = unsigned((a.tiles_m * a.tiles_n + 7) / 8 * 8);
  constexpr size_t kL04 = SmfShape<false, 4>::kLds, kL02 = SmfShape<false, 2>::kLds;
  constexpr size_t kL14 = SmfShape<true, 4>::kLds, kL12 = SmfShape<true, 2>::kLds;
  constexpr size_t kL04w = SmfShape<false, 4, 4>::kLds, kL02w = SmfShape<false, 2, 4>::kLds;
  // Blocks of a 2:4 mask with eight waves (two per SIMD) unless
  // SWM_SMF_WAVES=4 (read once).  Two A/B runs, us, q_proj 2:4: N = 4096
  // (256 x 256 blocks) 109.8 / 111.0 with four waves against 92.9 / 92.9
  // with eight; N = 1024 / 2048 (256 x 128 blocks) 57.5 / 68.7 against
  // 54.8 / 65.4.  With a residual layer the 256 x 256 eight-wave instance
  // would spill its A fragments, so that route keeps four waves.
  static const bool eight = [] {
    const char* e = getenv("SWM_SMF_WAVES");
    return !(e && atoi(e) == 4);
  }();
  if (residual) {
    if (wide)
      hipLaunchKernelGGL((smf_kernel<true, 4>), dim3(grid), dim3(256), kL14, s, a);
    else
      hipLaunchKernelGGL((smf_kernel<true, 2>), dim3(grid), dim3(256), kL12, s, a);
  } else {
    if (wide && eight)
      hipLaunchKernelGGL((smf_kernel<false, 4, 4>), dim3(grid), dim3(512), kL04w, s, a);
    else if (wide)
      hipLaunchKernelGGL((smf_kernel<false, 4>), dim3(grid), dim3(256), kL04, s, a);
    else if (eight)
      hipLaunchKernelGGL((smf_kernel<false, 2, 4>), dim3(grid), dim3(512), kL02w, s, a);
    else
      hipLaunchKernelGGL((smf_kernel<false, 2>), dim3(grid), dim3(256), kL02, s, a);
  }
  return hipGetLastError();
}

}  // namespace swm
