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

#include <cstdlib>

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

// How a split-K partial reaches the output.
//  kRedFence : fp32 partial stores, device-scope fence, arrival counter; the
//              last workgroup of a row block sums the partials (fences write
//              back and invalidate the L2 of every XCD that executes them).
//  kRedAtomic: partial stores and loads are device-coherent relaxed atomics
//              (they bypass the non-coherent L2); the writer waits for its
//              stores to complete before it bumps the arrival counter.
//  kRedKernel: partials only; a second kernel sums them in split order.
enum RedMode { kRedFence = 0, kRedAtomic = 1, kRedKernel = 2 };

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
  int red;  // RedMode
};

// Shared tail of the split-K decode kernels: reduce the waves' 64x16 fp32
// accumulators in LDS (fixed wave order), then either store fp16 Y (one
// split) or publish a partial that is summed in fixed split order.
// `red` must hold nwaves*16*64 floats; `flag` one word.
__device__ __forceinline__ void reduce_and_store(int kRed, float* red, uint32_t* flag, int nwaves, int wave,
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
  float* mypart = partials + (size_t(rowblk) * splits + split) * 16 * 64;
  for (int e = threadIdx.x; e < nout; e += blockDim.x) {
    const int tok = e >> 6, row = e & 63;
    float sum = 0.f;
    for (int w = 0; w < nwaves; ++w) sum += red[(w * 16 + tok) * 64 + row];
    if (splits == 1) {
      if (m0 + row < M) Y[int64_t(tok) * ldy + m0 + row] = __builtin_bit_cast(uint16_t, _Float16(sum));
    } else if (kRed == kRedAtomic) {
      __hip_atomic_store(mypart + e, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      mypart[e] = sum;
    }
  }
  if (splits == 1 || kRed == kRedKernel) return;
  if (kRed == kRedFence) {
    __threadfence();
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are done
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&counters[rowblk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = (old == uint32_t(splits - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (*flag == 0u) return;
  if (kRed == kRedFence) __threadfence();
  const float* base = partials + size_t(rowblk) * splits * 16 * 64;
  for (int e = threadIdx.x; e < nout; e += blockDim.x) {
    const int tok = e >> 6, row = e & 63;
    float sum = 0.f;
    for (int q = 0; q < splits; ++q) {
      const float* p = base + size_t(q) * 16 * 64 + e;
      sum += (kRed == kRedAtomic) ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : __builtin_nontemporal_load(p);
    }
    if (m0 + row < M) Y[int64_t(tok) * ldy + m0 + row] = __builtin_bit_cast(uint16_t, _Float16(sum));
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[rowblk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum split-K partials in split order and store fp16 Y (kRedKernel).
// One thread per (row, token) output; partial layout [rowblk][split][16][64].
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ partials,
                                                              uint16_t* __restrict__ Y, int64_t ldy,
                                                              int M, int N, int splits) {
  const int rowblk = blockIdx.x;
  const float* base = partials + size_t(rowblk) * splits * 16 * 64;
  for (int e = threadIdx.x; e < N * 64; e += blockDim.x) {
    const int tok = e >> 6, row = e & 63;
    float sum = 0.f;
    for (int q = 0; q < splits; ++q) sum += base[size_t(q) * 16 * 64 + e];
    const int m = rowblk * kTM + row;
    if (m < M) Y[int64_t(tok) * ldy + m] = __builtin_bit_cast(uint16_t, _Float16(sum));
  }
}

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint64_t word_of(const u32x16& w, int e) {
  return uint64_t(w[2 * e]) | (uint64_t(w[2 * e + 1]) << 32);
}

// One workgroup = `nwaves` waves on the same 64-row block; wave w decodes the
// `tpw` consecutive 64x64 tiles starting at tile column (split*nwaves + w)*tpw.
//
// Per tile every global access has a fixed count so the compiler can keep
// loads in flight across tiles: the run is fetched as kR 1 KiB chunks one tile
// ahead (addresses clamped into the run, so chunks past its end re-read
// cached bytes instead of branching), the next tile's bitmap words are touched
// with a vector load to bring them into L2, bitmap words reach SGPRs one
// 8-column group ahead (s_load_dwordx16), and B operands two groups ahead.
// kSkip: input channels whose activation is zero in every token are not
// decoded (their run is still streamed).
template <int kR, bool kSkip, bool kVec>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int rowblk = int(blockIdx.x) / a.splits;
  const int split = int(blockIdx.x) - rowblk * a.splits;

  // LDS: [0,16) zeros | flag | nwaves run buffers (kR KiB each); the
  // reduction area reuses the run buffers after a barrier.
  if (threadIdx.x < 8) reinterpret_cast<uint32_t*>(smem)[threadIdx.x] = 0u;
  __syncthreads();
  const uint32_t zero_addr = lds_addr(smem);
  const uint32_t buf = lds_addr(smem + 32 + size_t(wave) * kR * 1024);

  const int j0 = (split * nwaves + wave) * a.tpw;
  const int j1 = min(j0 + a.tpw, a.kt);

  // Block-diagonal B operand: lanes 0..15 and 48..63 carry token (lane & 15).
  const int q = lane >> 5, jj = lane & 31, tok = lane & 15;
  const bool xlane = ((jj >> 4) == q) && (tok < a.N);
  const uint16_t* xrow = xlane ? a.X + int64_t(tok) * a.ldx : a.zeros;
  const int64_t kmax8 = a.K >= 8 ? a.K - 8 : 0;  // clamp for groups past K (their A is zero)

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  uint32_t keep = 0;  // consumes the L2 prefetch so it is not removed

  if (j0 < j1) {
    const uint64_t tbase = uint64_t(rowblk) * a.kt;
    auto load_run = [&](int j, u32x4 (&pre)[kR]) {
      const uint32_t p0 = a.tile_ptr[tbase + j], p1 = a.tile_ptr[tbase + j + 1];
      const uint32_t last = p1 > p0 + 8 ? p1 - 8 : p0;  // last 8-value slot of the run
#pragma unroll
      for (int c = 0; c < kR; ++c) {
        const uint32_t off = min(p0 + uint32_t(c * 512 + lane * 8), last);
        pre[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vals + off));
      }
    };
    auto load_b = [&](int j, int g) -> half8 {
      int64_t col = int64_t(j) * 64 + 8 * g;
      if constexpr (kVec) {
        col = col < a.K ? col : kmax8;
        return __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(xrow + col));
      } else {
        return load_x8<false>(xrow, col, a.K);
      }
    };
    auto load_words = [&](int j, int g) -> u32x16 {
      return *reinterpret_cast<const u32x16*>(a.bits + (tbase + j) * 64 + 8 * g);
    };

    u32x4 pre[kR];
    load_run(j0, pre);
    half8 bop[8];
    bop[0] = load_b(j0, 0);
    bop[1] = load_b(j0, 1);
    u32x16 wslot[2];
    wslot[0] = load_words(j0, 0);

    for (int j = j0; j < j1; ++j) {
      const int jn = min(j + 1, j1 - 1);
      const uint64_t t = tbase + j;
      // Stage this tile's run, then fetch the next tile's run behind it.
#pragma unroll
      for (int c = 0; c < kR; ++c)
        *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(buf + c * 1024 + lane * 16)) = pre[c];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      load_run(jn, pre);
      {
        const u32x2 w = *reinterpret_cast<const u32x2*>(a.bits + (tbase + jn) * 64 + lane);
        keep ^= w[0] ^ w[1];
      }
      uint64_t active = ~0ull;
      if constexpr (kSkip) {
        bool nz = false;
        const int64_t col = int64_t(j) * 64 + lane;
        if (col < a.K)
          for (int n = 0; n < a.N; ++n) nz |= (a.X[int64_t(n) * a.ldx + col] & 0x7FFFu) != 0;
        active = __ballot(nz);
      }
      (void)t;
      uint32_t base = buf;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        // This group's words (scalar popcounts force their wait first), then
        // the lookahead: words one group ahead, B operands two groups ahead.
        const u32x16 wv = wslot[g & 1];
        uint32_t pc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pc[e] = 2u * uint32_t(__builtin_popcountll(word_of(wv, e)));
        __builtin_amdgcn_sched_barrier(0);
        wslot[(g + 1) & 1] = (g < 7) ? load_words(j, g + 1) : load_words(jn, 0);
        bop[(g + 2) & 7] = (g < 6) ? load_b(j, g + 2) : load_b(jn, g - 6);
        __builtin_amdgcn_sched_barrier(0);  // keep both loads ahead of this group's decode
        if constexpr (kSkip) {
          if (((active >> (8 * g)) & 0xFFull) == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) base += pc[e];
            continue;
          }
        }
        half8 aop;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t ad = run_addr(word_of(wv, e), base, zero_addr);
          base += pc[e];
          aop[e] = lds_half(ad);
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop[g], acc, 0, 0, 0);
      }
    }
  }
  if (keep == 0x9E3779B9u && a.N < 0) a.Y[0] = 0;  // never true: keeps the prefetch alive

  __syncthreads();  // all run buffers are free: reuse them as the reduction area
  float accv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) accv[v] = acc[v];
  reduce_and_store(a.red, reinterpret_cast<float*>(smem + 32), reinterpret_cast<uint32_t*>(smem + 16),
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
  int red;  // RedMode
};

// One workgroup = nwaves waves on one 64-row block, wave w covers columns
// [(split*nwaves + w)*kchunk, +kchunk) (kchunk a multiple of 128).  Per 32
// columns: four v_mfma_f32_16x16x32_f16 (16 rows each); lane l loads
// W[row][k0 + 8(l/16) .. +7] and X[l%16][k0 + 8(l/16) .. +7], 16 B each.
// Loads run three 32-column steps ahead through a four-slot register ring.
// Addresses past the chunk or past K point at the zero row instead.
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
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = m0 + r * 16 + (lane & 15);
    wrow[r] = row < a.M ? a.W + row * a.ldw : a.zeros;
  }

  if (kb < ke) {
    if constexpr (kVec) {
      const int nsteps = int((ke - kb + 31) / 32);
      half8 A[4][4], B[4];
      auto issue = [&](int s, int slot) {
        const int64_t k = kb + int64_t(s) * 32 + koff;
        const bool ok = k < ke;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          A[slot][r] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>((ok ? wrow[r] : a.zeros) + (ok ? k : 0)));
        B[slot] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>((ok ? xrow : a.zeros) + (ok ? k : 0)));
      };
      issue(0, 0);
      issue(1, 1);
      issue(2, 2);
      for (int s0 = 0; s0 < nsteps; s0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          issue(s0 + u + 3, (u + 3) & 3);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u][r], B[u], acc[r], 0, 0, 0);
        }
      }
    } else {
      for (int64_t k0 = kb; k0 < ke; k0 += 32) {
        const int64_t k = k0 + koff;
        half8 A0[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) A0[r] = load_x8<false>(wrow[r], k, ke);
        const half8 B0 = load_x8<false>(xrow, k, ke);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0[r], B0, acc[r], 0, 0, 0);
      }
    }
  }
  float accv[16];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) accv[r * 4 + v] = acc[r][v];
  reduce_and_store(a.red, reinterpret_cast<float*>(smem + 32), reinterpret_cast<uint32_t*>(smem + 16),
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

namespace {

template <int kR>
void launch_decode_r(bool skip, bool vec, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                     const DecodeArgs& a) {
  if (skip) {
    if (vec) hipLaunchKernelGGL((decode_kernel<kR, true, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((decode_kernel<8, true, false>), grid, block, lds, s, a);
  } else {
    if (vec) hipLaunchKernelGGL((decode_kernel<kR, false, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((decode_kernel<8, false, false>), grid, block, lds, s, a);
  }
}

}  // namespace

int reduce_mode_default() {
  static int mode = -1;
  if (mode < 0) {
    const char* e = getenv("SWM_SPLITK_REDUCE");
    mode = kRedKernel;
    if (e && e[0] == 'f') mode = kRedFence;
    if (e && e[0] == 'a') mode = kRedAtomic;
    if (e && e[0] == 'k') mode = kRedKernel;
  }
  return mode;
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
  a.red = reduce_mode_default();
  if (f.h.max_tile > 64u * 64u) return hipErrorInvalidValue;  // a 64x64 tile holds at most 4096 values
  // Runs are staged to LDS as kR 1 KiB (512-value) chunks per wave.
  const int need = int((f.h.max_tile + 511) / 512);
  const bool vec = (f.h.k % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  int kR = 8;
  if (vec) {
    const int opts[] = {2, 3, 4, 5, 6, 8};
    for (int o : opts)
      if (o >= need) { kR = o; break; }
  }
  a.buf_vals = kR * 512;
  const size_t run_bytes = size_t(p.waves) * kR * 1024;
  const size_t red_bytes = size_t(p.waves) * 16 * 64 * 4;
  const size_t lds = 32 + (run_bytes > red_bytes ? run_bytes : red_bytes);
  if (f.h.mt == 0) return hipSuccess;
  dim3 grid(unsigned(int64_t(f.h.mt) * p.splits)), block(unsigned(p.waves * 64));
  switch (kR) {
    case 2: launch_decode_r<2>(skip, vec, grid, block, lds, s, a); break;
    case 3: launch_decode_r<3>(skip, vec, grid, block, lds, s, a); break;
    case 4: launch_decode_r<4>(skip, vec, grid, block, lds, s, a); break;
    case 5: launch_decode_r<5>(skip, vec, grid, block, lds, s, a); break;
    case 6: launch_decode_r<6>(skip, vec, grid, block, lds, s, a); break;
    default: launch_decode_r<8>(skip, vec, grid, block, lds, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1 && a.red == kRedKernel) {
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(unsigned(f.h.mt)), dim3(256), 0, s, a.partials, Y, ldy,
                       a.M, n, p.splits);
    e = hipGetLastError();
  }
  return e;
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
  kchunk = (kchunk + 127) / 128 * 128;
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
  a.red = reduce_mode_default();
  const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && (ldw % 8 == 0) &&
                   ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  const int64_t mt = (M + 63) / 64;
  if (mt == 0) return hipSuccess;
  dim3 grid(unsigned(mt * p.splits)), block(unsigned(p.waves * 64));
  size_t lds = 32 + size_t(p.waves) * 16 * 64 * 4;
  if (vec) hipLaunchKernelGGL((dense_small_kernel<true>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((dense_small_kernel<false>), grid, block, lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1 && a.red == kRedKernel) {
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(unsigned(mt)), dim3(256), 0, s, partials, Y, ldy,
                       int(M), n, p.splits);
    e = hipGetLastError();
  }
  return e;
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
