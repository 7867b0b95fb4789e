// Prefill-regime kernels (large N): Y = W X on the matrix cores, with W
// either dense (the in-house baseline) or expanded on chip from the SWM-TCB v1
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
// gfx950 design: one 256-thread workgroup computes a 256 (rows of W) x 256
// (tokens) block of Y over K in steps of 64.  Four waves in a 2 x 2 layout each
// own a 128 x 128 sub-block = 4 x 4 v_mfma_f32_32x32x16_f16 accumulators (256
// fp32 per lane, in AGPRs).  A and B tiles (256 x 64 fp16 each) are double
// buffered in LDS with an XOR swizzle of the 16-byte chunks (row r, chunk c at
// chunk c ^ (r & 7)) so that the 16-byte fragment reads of eight consecutive
// rows hit distinct banks without padding.  Next step's tiles are fetched into
// VGPRs while the current step's 64 products issue.  In the sparse variant each
// wave expands one 64 x 64 weight tile per step (the decode kernel's bitmap
// rank scheme, then one 16-byte LDS store per 8 columns), interleaved with
// the products of the current step.  The workgroup-to-tile map is XCD aware:
// consecutive workgroup ids go to different XCDs, so ids are regrouped to give
// each XCD a contiguous band of output tiles that share weight rows in its L2.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace swm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) _Float16 lds_f16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kTileBytes = BM * BK * 2;  // 32 KiB per operand stage

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void lds_store16(uint32_t addr, u32x4 v) {
  *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(addr)) = v;
}
__device__ __forceinline__ u32x4 lds_load16(uint32_t addr) {
  return *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ _Float16 lds_half(uint32_t addr) {
  return *reinterpret_cast<const lds_f16*>(static_cast<uintptr_t>(addr));
}
// Byte offset of (row, 16-byte chunk) in a swizzled 256 x 64 fp16 tile.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return uint32_t(row * 128 + ((chunk ^ (row & 7)) << 4));
}

__device__ __forceinline__ uint32_t run_addr(uint64_t word, uint32_t run_base, uint32_t zero_addr) {
  const uint32_t rank =
      __builtin_amdgcn_mbcnt_hi(uint32_t(word >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(word), 0u));
  uint32_t a;
  asm("v_lshl_add_u32 %0, %1, 1, %2\n\t"
      "v_cndmask_b32_e64 %0, %3, %0, %4"
      : "=&v"(a)
      : "v"(rank), "s"(run_base), "v"(zero_addr), "s"(word));
  return a;
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
  int tiles_m, tiles_n, kt;
  int group_m;     // output-tile rows per L2 group
  int run_chunks;  // 512-byte run chunks per tile (1..4), sparse variant
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

template <bool kSparse>
__global__ __launch_bounds__(256, 1) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  int tm, tn;
  if (!tile_of(a, tm, tn)) return;
  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = tm * BM, n0 = tn * BN;

  // LDS: A stages [2][32 KiB] | B stages [2][32 KiB] | zero (16 B) | run buffers
  const uint32_t sA = lds_addr(smem), sB = sA + 2 * kTileBytes;
  const uint32_t zero_addr = sB + 2 * kTileBytes;
  const uint32_t runbuf = zero_addr + 16 + uint32_t(wave) * 4u * uint32_t(a.run_chunks) * 512u;
  if (kSparse && tid < 4) reinterpret_cast<uint32_t*>(smem + 4 * kTileBytes)[tid] = 0u;

  // Global fetch map: thread -> (row r*32 + tid/8, chunk tid%8), r = 0..7.
  const int frow = tid >> 3, fch = tid & 7;
  const int nsteps = (a.K + BK - 1) / BK;

  u32x4 regA[8], regB[8];
  u32x2 runreg[16];  // sparse: 4 tiles x up to 4 chunks of 8 bytes per lane
  auto fetch_B = [&](int ks) {
    const int k = ks * BK + fch * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int n = n0 + r * 32 + frow;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (n < a.N && k < a.K) v = *reinterpret_cast<const u32x4*>(a.X + int64_t(n) * a.ldx + k);
      regB[r] = v;
    }
  };
  auto store_B = [&](int stage) {
#pragma unroll
    for (int r = 0; r < 8; ++r) lds_store16(sB + stage * kTileBytes + swz(r * 32 + frow, fch), regB[r]);
  };
  auto fetch_A_dense = [&](int ks) {
    const int k = ks * BK + fch * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int m = m0 + r * 32 + frow;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < a.M && k < a.K) v = *reinterpret_cast<const u32x4*>(a.W + int64_t(m) * a.ldw + k);
      regA[r] = v;
    }
  };
  auto store_A_dense = [&](int stage) {
#pragma unroll
    for (int r = 0; r < 8; ++r) lds_store16(sA + stage * kTileBytes + swz(r * 32 + frow, fch), regA[r]);
  };
  // Sparse: at step ks this wave expands the four 16x64 tiles (slabs
  // m0/16 + 4*wave + tt, tile column ks), tt = 0..3, into A-stage rows
  // 64*wave + 16*tt .. +15.  Their runs are staged in this wave's LDS run
  // buffer in 512-byte chunks (8 bytes per lane), run_chunks per tile.
  const int slab0 = m0 / 16 + 4 * wave;
  const uint32_t tile_run_bytes = uint32_t(a.run_chunks) * 512u;
  auto fetch_A_run = [&](int ks) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if ((slab0 + tt) * 16 >= a.M) continue;
      const uint64_t t = uint64_t(slab0 + tt) * a.kt + ks;
      const uint32_t p0 = a.tile_ptr[t], p1 = a.tile_ptr[t + 1];
      const uint32_t last = p1 > p0 + 4 ? p1 - 4 : p0;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < a.run_chunks) {
          const uint32_t off = min(p0 + uint32_t(c * 256 + lane * 4), last);
          runreg[tt * 4 + c] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.vals + off));
        }
    }
  };
  auto stage_A_run = [&]() {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if ((slab0 + tt) * 16 >= a.M) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c < a.run_chunks)
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
              static_cast<uintptr_t>(runbuf + tt * tile_run_bytes + c * 512 + lane * 8)) = runreg[tt * 4 + c];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  // Expand step s (32 columns) of tile tt: eight words -> this lane's row
  // l%16, columns 32s + 8(l/16) .. +7 -> one 16-byte store.  `base` walks the
  // tile's run in LDS (bytes).
  auto expand_unit = [&](int ks, int stage, int tt, int s, uint32_t& base) {
    const int row = wave * 64 + tt * 16 + (lane & 15);
    u32x4 out = {0u, 0u, 0u, 0u};
    if ((slab0 + tt) * 16 < a.M) {
      const uint64_t t = uint64_t(slab0 + tt) * a.kt + ks;
      const uint64_t* tb = a.bits + t * 16 + 8 * s;
      half8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint64_t w = tb[e];
        const uint32_t ad = run_addr(w, base, zero_addr);
        base += 2u * uint32_t(__builtin_popcountll(w));
        h[e] = lds_half(ad);
      }
      out = __builtin_bit_cast(u32x4, h);
    }
    lds_store16(sA + stage * kTileBytes + swz(row, 4 * s + (lane >> 4)), out);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Prologue: stage 0.  Sparse runs are two steps deep: the run of step k+1
  // is already in VGPRs when step k starts, the run of step k+2 is fetched
  // during step k.
  fetch_B(0);
  if constexpr (kSparse) {
    __syncthreads();  // zero word visible
    fetch_A_run(0);
    stage_A_run();
    for (int tt = 0; tt < 4; ++tt) {
      uint32_t base = runbuf + uint32_t(tt) * tile_run_bytes;
      for (int s2 = 0; s2 < 2; ++s2) expand_unit(0, 0, tt, s2, base);
    }
    if (nsteps > 1) fetch_A_run(1);
  } else {
    fetch_A_dense(0);
    store_A_dense(0);
  }
  store_B(0);
  __syncthreads();

  for (int ks = 0; ks < nsteps; ++ks) {
    const int st = ks & 1;
    const bool more = ks + 1 < nsteps;
    if constexpr (kSparse) {
      if (more) stage_A_run();
      if (ks + 2 < nsteps) fetch_A_run(ks + 2);
    }
    if (more) {
      fetch_B(ks + 1);
      if constexpr (!kSparse) fetch_A_dense(ks + 1);
    }
    const uint32_t aBase = sA + st * kTileBytes, bBase = sB + st * kTileBytes;
    uint32_t base = runbuf;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      half8 fa[4], fb[4];
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = __builtin_bit_cast(half8, lds_load16(aBase + swz(wm * 128 + i * 32 + (lane & 31), ch)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = __builtin_bit_cast(half8, lds_load16(bBase + swz(wn * 128 + j * 32 + (lane & 31), ch)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        if constexpr (kSparse) {
          // eight expansion units per step (tile tt = unit/2, step s = unit%2),
          // one after every second product
          if (more && (i & 1)) {
            const int unit = kk * 2 + (i >> 1), tt = unit >> 1, s2 = unit & 1;
            if (s2 == 0) base = runbuf + uint32_t(tt) * tile_run_bytes;
            expand_unit(ks + 1, st ^ 1, tt, s2, base);
          }
        }
      }
    }
    if (more) {
      if constexpr (!kSparse) store_A_dense(st ^ 1);
      store_B(st ^ 1);
    }
    __syncthreads();
  }

  // Epilogue: fp16 round-to-nearest-even, 4 consecutive rows per 8-byte store.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 128 + j * 32 + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * 128 + i * 32 + q * 8 + (lane >> 5) * 4;
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
  return (K % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
}

size_t prefill_sparse_lds(const Header& h) {
  const size_t chunks = (size_t(h.max_tile) + 255) / 256;  // 512-byte chunks per tile run
  return size_t(4) * kTileBytes + 16 + 4 /*waves*/ * 4 /*tiles*/ * (chunks ? chunks : 1) * 512;
}

hipError_t launch_prefill_dense(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx,
                                uint16_t* Y, int64_t ldy, int64_t M, int64_t K, int64_t N,
                                hipStream_t s) {
  PrefillArgs a = make_args(M, N, K, X, ldx, Y, ldy);
  a.W = W;
  a.ldw = ldw;
  if (a.tiles_m == 0 || a.tiles_n == 0) return hipSuccess;
  const size_t lds = size_t(4) * kTileBytes;
  hipLaunchKernelGGL((prefill_kernel<false>), dim3(grid_size(a)), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_sparse(const DevFormat& f, const uint16_t* X, int64_t ldx, uint16_t* Y,
                                 int64_t ldy, int64_t N, hipStream_t s) {
  PrefillArgs a = make_args(f.h.m, N, f.h.k, X, ldx, Y, ldy);
  a.tile_ptr = f.tile_ptr;
  a.bits = f.bits;
  a.vals = f.vals;
  a.kt = int(f.h.kt);
  a.run_chunks = int((f.h.max_tile + 255) / 256);
  if (a.run_chunks < 1) a.run_chunks = 1;
  if (f.h.tm != 16 || f.h.tk != 64 || f.h.max_tile > 1024) return hipErrorInvalidValue;
  if (a.tiles_m == 0 || a.tiles_n == 0) return hipSuccess;
  const size_t lds = prefill_sparse_lds(f.h);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<true>), dim3(grid_size(a)), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace swm
