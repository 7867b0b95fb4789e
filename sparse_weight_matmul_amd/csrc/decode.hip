// Decode-regime kernels (N <= 16 tokens): sparse SpMM / spMspV over the
// SWM-TCB v1 format, the dense small-N baseline, and format expansion.
//
// Method: "Unified Static-Dynamic Pruning for Efficient LLM Inference" (SPDP),
// abstract -- a decode kernel streams the tiled column-bitmap weights, decodes
// the bitmaps on chip and skips input channels whose activation is zero.
// Decode is bandwidth bound because every token re-reads all weights ("Reduced
// Matrix Multiplication" blog page, Sec. 3.1), and bitmap decoding on the
// vector units must keep up with HBM ("Accelerating GPU inference of LLMs with
// moderately unstructured sparse weight matrices", Sec. 1, Challenge 3).
//
// gfx950 mapping of one 64 x 64 tile (TM = 64 rows, TK = 64 columns):
//  * one wave owns the tile; lane l owns row l;
//  * the tile's packed run (column-major) is streamed HBM -> VGPR (dwordx4,
//    1 KiB per wave instruction, prefetched one tile ahead) -> LDS;
//  * per column c the 64-bit bitmap word is wave-uniform (scalar load); the
//    run offset of column c is a scalar popcount prefix, the lane's rank is
//    v_mbcnt over the word, and lanes whose bit is clear read a zero halfword;
//  * eight decoded columns give lane l the fp16 values W[l][c..c+7], which is
//    the A operand of v_mfma_f32_32x32x16_f16 if the two 32-row halves of the
//    tile are treated as the two k-halves of the instruction; the B operand is
//    then block-diagonal (tokens 0..15 for rows 0..31 in lanes 0..15, for rows
//    32..63 in lanes 48..63, zeros elsewhere), so one instruction yields the
//    full 64 rows x 16 tokens partial product with fp32 accumulation;
//  * split-K over workgroups; each workgroup reduces its waves in LDS in fixed
//    order, writes one fp32 partial, and the last workgroup of a row block
//    (arrival counter) sums the partials in split order and stores fp16 Y.
//    The result is bitwise reproducible run to run.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace swm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) _Float16 lds_f16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kTM = 64;
constexpr int kMaxChunks = 8;  // a 64x64 tile run is at most 4096 values = 8 KiB = 8 x 1 KiB

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// LDS byte address of the lane's value in a column run: run_base + 2*rank if
// the lane's bit is set in `word`, else `zero_addr`.
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

__device__ __forceinline__ _Float16 lds_half(uint32_t addr) {
  return *reinterpret_cast<const lds_f16*>(static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ half8 zero_h8() {
  half8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = _Float16(0);
  return z;
}

// Eight fp16 activations x[col .. col+7] of one token row (zero outside [0, K)).
template <bool kVec>
__device__ __forceinline__ half8 load_x8(const uint16_t* row, int64_t col, int64_t K) {
  if constexpr (kVec) {
    if (col < K) return __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(row + col));
    return zero_h8();
  } else {
    half8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = (col + e < K) ? __builtin_bit_cast(_Float16, row[col + e]) : _Float16(0);
    return v;
  }
}

struct DecodeArgs {
  const uint32_t* tile_ptr;
  const uint64_t* bits;
  const uint16_t* vals;
  const uint16_t* zeros;
  const uint16_t* X;
  uint16_t* Y;
  float* partials;
  uint32_t* counters;
  int64_t ldx, ldy;
  int M, K, N, kt;
  int tpw, splits, buf_vals;
};

// Shared tail of the split-K decode kernels: reduce the waves' 64x16 fp32
// accumulators in LDS, then either store fp16 Y (one split) or publish a
// partial and let the last workgroup of the row block finish.
// `red` must hold nwaves*16*64 floats; `flag` one word.
__device__ __forceinline__ void reduce_and_store(float* red, uint32_t* flag, int nwaves, int wave,
                                                 int lane, const float (&accv)[16], int rowblk,
                                                 int split, int splits, int M, int N, uint16_t* Y,
                                                 int64_t ldy, float* partials, uint32_t* counters,
                                                 bool mfma32_layout) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    int row, tok;
    if (mfma32_layout) {  // v_mfma_f32_32x32x16 with the block-diagonal B operand
      row = ((lane & 31) >> 4) * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      tok = lane & 15;
    } else {  // four 16x16x32 row groups, group = v / 4
      row = (v >> 2) * 16 + (lane >> 4) * 4 + (v & 3);
      tok = lane & 15;
    }
    red[(wave * 16 + tok) * 64 + row] = accv[v];
  }
  __syncthreads();
  const int m0 = rowblk * kTM;
  const int nout = N * 64;
  for (int e = threadIdx.x; e < nout; e += blockDim.x) {
    const int tok = e >> 6, row = e & 63;
    float sum = 0.f;
    for (int w = 0; w < nwaves; ++w) sum += red[(w * 16 + tok) * 64 + row];
    if (splits == 1) {
      if (m0 + row < M) Y[int64_t(tok) * ldy + m0 + row] = __builtin_bit_cast(uint16_t, _Float16(sum));
    } else {
      partials[((size_t(rowblk) * splits + split) * 16 + tok) * 64 + row] = sum;
    }
  }
  if (splits == 1) return;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&counters[rowblk], 1u);
    *flag = (old == uint32_t(splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (*flag == 0u) return;
  __threadfence();
  for (int e = threadIdx.x; e < nout; e += blockDim.x) {
    const int tok = e >> 6, row = e & 63;
    const float* p = partials + (size_t(rowblk) * splits * 16 + tok) * 64 + row;
    float sum = 0.f;
    for (int q = 0; q < splits; ++q) sum += __builtin_nontemporal_load(p + size_t(q) * 16 * 64);
    if (m0 + row < M) Y[int64_t(tok) * ldy + m0 + row] = __builtin_bit_cast(uint16_t, _Float16(sum));
  }
  if (threadIdx.x == 0) counters[rowblk] = 0u;  // ready for the next stream-ordered call
}

// One workgroup = `nwaves` waves on the same 64-row block; wave w decodes the
// `tpw` consecutive 64x64 tiles starting at tile column (split*nwaves + w)*tpw.
// kSkip: input channels whose activation is zero in every token are not
// decoded (their run is still streamed in this kernel).
template <bool kSkip, bool kVec>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int rowblk = int(blockIdx.x) / a.splits;
  const int split = int(blockIdx.x) - rowblk * a.splits;

  // LDS: [0,16) zeros | flag (16 B) | nwaves run buffers; the reduction area
  // reuses the run buffers after a barrier.
  if (threadIdx.x < 8) reinterpret_cast<uint32_t*>(smem)[threadIdx.x] = 0u;
  __syncthreads();
  const uint32_t zero_addr = lds_addr(smem);
  uint8_t* bufp = smem + 32 + size_t(wave) * a.buf_vals * 2;
  const uint32_t buf = lds_addr(bufp);

  const int j0 = (split * nwaves + wave) * a.tpw;
  const int j1 = min(j0 + a.tpw, a.kt);

  // Block-diagonal B operand: lanes 0..15 and 48..63 carry token (lane & 15).
  const int q = lane >> 5, jj = lane & 31, tok = lane & 15;
  const bool xlane = ((jj >> 4) == q) && (tok < a.N);
  const uint16_t* xrow = xlane ? a.X + int64_t(tok) * a.ldx : a.zeros;

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;

  if (j0 < j1) {
    const uint64_t tbase = uint64_t(rowblk) * a.kt;
    u32x4 pre[kMaxChunks];
    {
      const uint32_t p0 = a.tile_ptr[tbase + j0], p1 = a.tile_ptr[tbase + j0 + 1];
      const int nch = int((p1 - p0 + 511) >> 9);
      const u32x4* src = reinterpret_cast<const u32x4*>(a.vals + p0) + lane;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < nch) pre[c] = __builtin_nontemporal_load(src + c * 64);
    }
    for (int j = j0; j < j1; ++j) {
      const uint64_t t = tbase + j;
      const uint32_t p0 = a.tile_ptr[t], p1 = a.tile_ptr[t + 1];
      const int nch = int((p1 - p0 + 511) >> 9);
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < nch) *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(buf + c * 1024 + lane * 16)) = pre[c];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (j + 1 < j1) {
        const uint32_t n0 = p1, n1 = a.tile_ptr[t + 2];
        const int nn = int((n1 - n0 + 511) >> 9);
        const u32x4* src = reinterpret_cast<const u32x4*>(a.vals + n0) + lane;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)
          if (c < nn) pre[c] = __builtin_nontemporal_load(src + c * 64);
      }
      const int64_t col0 = int64_t(j) * 64;
      half8 bop[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) bop[g] = load_x8<kVec>(xrow, col0 + 8 * g, a.K);

      uint64_t active = ~0ull;
      if constexpr (kSkip) {
        bool nz = false;
        const int64_t col = col0 + lane;
        if (col < a.K)
          for (int n = 0; n < a.N; ++n) nz |= (a.X[int64_t(n) * a.ldx + col] & 0x7FFFu) != 0;
        active = __ballot(nz);
      }

      const uint64_t* tb = a.bits + t * 64;
      uint32_t base = buf;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (col0 + 8 * g >= a.K) break;  // whole group beyond K (K % 8 == 0 on the vector path)
        half8 aop;
        if constexpr (kSkip) {
          if (((active >> (8 * g)) & 0xFFull) == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) base += 2u * uint32_t(__builtin_popcountll(tb[8 * g + e]));
            continue;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint64_t w = tb[8 * g + e];
          const uint32_t ad = run_addr(w, base, zero_addr);
          base += 2u * uint32_t(__builtin_popcountll(w));
          aop[e] = lds_half(ad);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop[g], acc, 0, 0, 0);
      }
    }
  }

  __syncthreads();  // all run buffers are free: reuse them as the reduction area
  float accv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) accv[v] = acc[v];
  reduce_and_store(reinterpret_cast<float*>(smem + 32), reinterpret_cast<uint32_t*>(smem + 16),
                   nwaves, wave, lane, accv, rowblk, split, a.splits, a.M, a.N, a.Y, a.ldy,
                   a.partials, a.counters, true);
}

// ------------------------------------------------------------------ dense, N <= 16
struct DenseArgs {
  const uint16_t* W;
  const uint16_t* X;
  const uint16_t* zeros;
  uint16_t* Y;
  float* partials;
  uint32_t* counters;
  int64_t ldw, ldx, ldy, M, K;
  int N, kchunk, splits;
};

// One workgroup = nwaves waves on one 64-row block, wave w covers columns
// [(split*nwaves + w)*kchunk, +kchunk).  Per 32 columns: four
// v_mfma_f32_16x16x32_f16 (16 rows each); lane l loads W[row][k0 + 8(l/16) ..+7]
// and X[l%16][k0 + 8(l/16) ..+7], 16 B each.  Next step's loads are issued
// before the current step's products.
template <bool kVec>
__global__ __launch_bounds__(256) void dense_small_kernel(DenseArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int rowblk = int(blockIdx.x) / a.splits;
  const int split = int(blockIdx.x) - rowblk * a.splits;
  const int64_t m0 = int64_t(rowblk) * kTM;
  const int64_t kb = int64_t(split * nwaves + wave) * a.kchunk;
  const int64_t ke = min(kb + a.kchunk, a.K);
  const int koff = 8 * (lane >> 4);
  const int tok = lane & 15;
  const uint16_t* xrow = (tok < a.N) ? a.X + int64_t(tok) * a.ldx : a.zeros;

  f32x4 acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[r][v] = 0.f;

  const uint16_t* wrow[4];
  bool rok[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = m0 + r * 16 + (lane & 15);
    rok[r] = row < a.M;
    wrow[r] = rok[r] ? a.W + row * a.ldw : a.zeros;
  }

  auto loadA = [&](int64_t k0, half8 (&A)[4], half8& B) {
    const int64_t k = k0 + koff;
#pragma unroll
    for (int r = 0; r < 4; ++r) A[r] = load_x8<kVec>(wrow[r], k, ke);
    B = load_x8<kVec>(xrow, k, ke);
  };
  if (kb < ke) {
    half8 A0[4], B0, A1[4], B1;
    loadA(kb, A0, B0);
    int64_t k0 = kb;
    for (; k0 + 32 < ke; k0 += 64) {
      loadA(k0 + 32, A1, B1);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[r], B0, acc[r], 0, 0, 0);
      if (k0 + 64 < ke) loadA(k0 + 64, A0, B0);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1[r], B1, acc[r], 0, 0, 0);
    }
    if (k0 < ke) {
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[r], B0, acc[r], 0, 0, 0);
    }
  }
  float accv[16];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) accv[r * 4 + v] = acc[r][v];
  reduce_and_store(reinterpret_cast<float*>(smem + 32), reinterpret_cast<uint32_t*>(smem + 16),
                   nwaves, wave, lane, accv, rowblk, split, a.splits, int(a.M), a.N, a.Y, a.ldy,
                   a.partials, a.counters, false);
}

// ------------------------------------------------------------------ decompress
// One wave per 64x64 tile: decode each column into an LDS tile [64 rows][64+8
// cols] (padded row stride), then write the rows of W out with 16-byte stores.
struct DecompArgs {
  const uint32_t* tile_ptr;
  const uint64_t* bits;
  const uint16_t* vals;
  uint16_t* W;
  int64_t ldw;
  int M, K, kt;
  int64_t tiles;
  int vec;
};

__global__ __launch_bounds__(256) void decompress_kernel(DecompArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[4][64][72];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= a.tiles) return;
  const int rowblk = int(t / a.kt), tj = int(t % a.kt);
  const uint64_t* tb = a.bits + t * 64;
  uint32_t pos = a.tile_ptr[t];
  for (int c = 0; c < 64; ++c) {
    const uint64_t w = tb[c];
    const bool set = (w >> lane) & 1ull;
    const uint32_t rank =
        __builtin_amdgcn_mbcnt_hi(uint32_t(w >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(w), 0u));
    tile[wave][lane][c] = set ? a.vals[pos + rank] : uint16_t(0);
    pos += uint32_t(__builtin_popcountll(w));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // lane -> (row = lane/8 + 8*it, 8-column chunk = lane%8)
  for (int it = 0; it < 8; ++it) {
    const int r = it * 8 + (lane >> 3), ch = lane & 7;
    const int64_t row = int64_t(rowblk) * 64 + r, col = int64_t(tj) * 64 + ch * 8;
    if (row >= a.M) continue;
    if (a.vec && col + 8 <= a.K) {
      *reinterpret_cast<u32x4*>(a.W + row * a.ldw + col) = *reinterpret_cast<const u32x4*>(&tile[wave][r][ch * 8]);
    } else {
      for (int e = 0; e < 8; ++e)
        if (col + e < a.K) a.W[row * a.ldw + col + e] = tile[wave][r][ch * 8 + e];
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ host launchers
DecodePlan plan_decode(const Header& h, int n, int num_cus) {
  (void)n;
  DecodePlan p;
  p.waves = 4;
  const int64_t tiles = int64_t(h.mt) * h.kt;
  // Aim at roughly eight resident waves per CU for the whole call.
  int64_t tpw = tiles / (int64_t(num_cus) * 8);
  if (tpw < 1) tpw = 1;
  if (tpw > 16) tpw = 16;
  p.tiles_per_wave = int(tpw);
  p.splits = int((h.kt + p.waves * p.tiles_per_wave - 1) / (p.waves * p.tiles_per_wave));
  if (p.splits < 1) p.splits = 1;
  return p;
}

size_t decode_partial_floats(const Header& h, const DecodePlan& p) {
  return p.splits > 1 ? size_t(h.mt) * p.splits * 16 * 64 : 0;
}

hipError_t launch_decode(const DevFormat& f, const DecodePlan& p, const uint16_t* X, int64_t ldx,
                         uint16_t* Y, int64_t ldy, int n, bool skip, hipStream_t s) {
  DecodeArgs a;
  a.tile_ptr = f.tile_ptr;
  a.bits = f.bits;
  a.vals = f.vals;
  a.zeros = f.zeros;
  a.X = X;
  a.Y = Y;
  a.partials = f.partials;
  a.counters = f.counters;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int(f.h.m);
  a.K = int(f.h.k);
  a.N = n;
  a.kt = int(f.h.kt);
  a.tpw = p.tiles_per_wave;
  a.splits = p.splits;
  // Runs are copied to LDS in 1 KiB (512-value) chunks: round the per-wave buffer up.
  a.buf_vals = int((f.h.max_tile + 511) / 512 * 512);
  if (f.h.max_tile > 64u * 64u) return hipErrorInvalidValue;  // a 64x64 tile holds at most 4096 values
  size_t run_bytes = size_t(p.waves) * a.buf_vals * 2;
  size_t red_bytes = size_t(p.waves) * 16 * 64 * 4;
  size_t lds = 32 + (run_bytes > red_bytes ? run_bytes : red_bytes);
  const bool vec = (f.h.k % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  if (f.h.mt == 0) return hipSuccess;
  dim3 grid(unsigned(int64_t(f.h.mt) * p.splits)), block(unsigned(p.waves * 64));
  if (skip) {
    if (vec) hipLaunchKernelGGL((decode_kernel<true, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((decode_kernel<true, false>), grid, block, lds, s, a);
  } else {
    if (vec) hipLaunchKernelGGL((decode_kernel<false, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((decode_kernel<false, false>), grid, block, lds, s, a);
  }
  return hipGetLastError();
}

DensePlan plan_dense_small(int64_t M, int64_t K, int n, int num_cus) {
  (void)n;
  DensePlan p;
  p.waves = 4;
  const int64_t mt = (M + 63) / 64;
  // about eight resident waves per CU
  const int64_t want_waves = int64_t(num_cus) * 8;
  int64_t chunks = (want_waves + mt - 1) / mt;  // K chunks per row block
  int64_t kchunk = (K + chunks - 1) / chunks;
  kchunk = (kchunk + 63) / 64 * 64;
  if (kchunk < 256) kchunk = 256;
  p.kchunk = int(kchunk);
  p.splits = int((K + p.waves * kchunk - 1) / (p.waves * kchunk));
  if (p.splits < 1) p.splits = 1;
  return p;
}

size_t dense_partial_floats(int64_t M, const DensePlan& p) {
  return p.splits > 1 ? size_t((M + 63) / 64) * p.splits * 16 * 64 : 0;
}

hipError_t launch_dense_small(const DensePlan& p, const uint16_t* W, int64_t ldw, const uint16_t* X,
                              int64_t ldx, uint16_t* Y, int64_t ldy, int64_t M, int64_t K, int n,
                              float* partials, uint32_t* counters, const uint16_t* zeros,
                              hipStream_t s) {
  DenseArgs a;
  a.W = W;
  a.X = X;
  a.zeros = zeros;
  a.Y = Y;
  a.partials = partials;
  a.counters = counters;
  a.ldw = ldw;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = M;
  a.K = K;
  a.N = n;
  a.kchunk = p.kchunk;
  a.splits = p.splits;
  const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && (ldw % 8 == 0) &&
                   ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  const int64_t mt = (M + 63) / 64;
  if (mt == 0) return hipSuccess;
  dim3 grid(unsigned(mt * p.splits)), block(unsigned(p.waves * 64));
  size_t lds = 32 + size_t(p.waves) * 16 * 64 * 4;
  if (vec) hipLaunchKernelGGL((dense_small_kernel<true>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((dense_small_kernel<false>), grid, block, lds, s, a);
  return hipGetLastError();
}

hipError_t launch_decompress(const DevFormat& f, uint16_t* W, int64_t ldw, hipStream_t s) {
  DecompArgs a;
  a.tile_ptr = f.tile_ptr;
  a.bits = f.bits;
  a.vals = f.vals;
  a.W = W;
  a.ldw = ldw;
  a.M = int(f.h.m);
  a.K = int(f.h.k);
  a.kt = int(f.h.kt);
  a.tiles = int64_t(f.h.mt) * f.h.kt;
  a.vec = (ldw % 8 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  if (a.tiles == 0) return hipSuccess;
  dim3 grid(unsigned((a.tiles + 3) / 4)), block(256);
  hipLaunchKernelGGL(decompress_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace swm
