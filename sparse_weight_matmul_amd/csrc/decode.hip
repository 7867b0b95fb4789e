// Decode-regime kernels (N <= 32 tokens): sparse SpMM / spMspV over the
// SWM-TCB v2 format, the dense small-N baseline, format expansion and an HBM
// streaming calibration kernel.
//
// Method: "Unified Static-Dynamic Pruning for Efficient LLM Inference" (SPDP),
// abstract -- a decode kernel streams the tiled column-bitmap weights, decodes
// the bitmaps on chip and skips input channels whose activation is zero.
// Decode is bandwidth bound because every token re-reads all weights ("Reduced
// Matrix Multiplication" blog page, Sec. 3.1), and bitmap decoding on the
// vector units must keep up with HBM ("Accelerating GPU inference of LLMs with
// moderately unstructured sparse weight matrices", Sec. 1, Challenge 3).
//
// gfx950 mapping.  A workgroup owns one 16-row slab of W over the whole K, so
// M = 4096 already gives 256 workgroups and no cross-workgroup reduction is
// needed; its waves split K and are summed in LDS in a fixed order (bitwise
// reproducible results).  Per 32-column step a wave decodes eight 64-bit
// bitmap words; lane l of word e stands for row l%16 and column 8(l/16)+e,
// which is where v_mfma_f32_16x16x32_f16 expects A[l%16][8(l/16)+e], so the
// decoded halves go straight into the A operand and the activations of 16
// tokens into B.  Decoding one word: its column-run offset is a scalar
// popcount prefix, the lane's rank inside the word is v_mbcnt, and lanes whose
// bit is clear read a zero halfword (v_cndmask on the SGPR-pair word).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace swm {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) _Float16 lds_f16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kSlab = 16;  // rows per tile / workgroup
constexpr int kTK = 64;    // columns per tile (two 32-column steps, 16 words)

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// LDS byte address of the lane's value in a word's run: run_base + 2*rank if
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

// A operand of one 32-column step from its eight bitmap words: element e of
// lane l is the lane's value in word e, or +0 where its bit is clear.  Per
// pair of words: each lane reads the halfword at its rank in either run (lanes
// whose bit is clear read a neighbour), then one v_cndmask zeroes the low half
// and a v_cndmask with SDWA (destination = upper word, lower word preserved)
// zeroes and packs the high half in one instruction.  `base` is the LDS byte
// address of word 0's run and advances past the step's eight runs.
__device__ __forceinline__ half8 decode_step(const u32x16& w, uint32_t& base) {
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  u32x4 out;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint64_t w0 = uint64_t(w[4 * p]) | (uint64_t(w[4 * p + 1]) << 32);
    const uint64_t w1 = uint64_t(w[4 * p + 2]) | (uint64_t(w[4 * p + 3]) << 32);
    const uint32_t r0 = __builtin_amdgcn_mbcnt_hi(uint32_t(w0 >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(w0), 0u));
    const uint32_t r1 = __builtin_amdgcn_mbcnt_hi(uint32_t(w1 >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(w1), 0u));
    // Run bases in bytes, one s_bcnt1 + s_lshl1_add per word, and the lane
    // address in one v_lshl_add (written out so that they are not
    // re-associated into a separate add per lane).
    uint32_t b1, b2, c0, c1, a0, a1;
    asm("s_bcnt1_i32_b64 %2, %4\n\t"
        "s_lshl1_add_u32 %0, %2, %6\n\t"
        "s_bcnt1_i32_b64 %3, %5\n\t"
        "s_lshl1_add_u32 %1, %3, %0"
        : "=&s"(b1), "=&s"(b2), "=&s"(c0), "=&s"(c1)
        : "s"(w0), "s"(w1), "s"(base)
        : "scc");
    asm("v_lshl_add_u32 %0, %1, 1, %2" : "=v"(a0) : "v"(r0), "s"(base));
    asm("v_lshl_add_u32 %0, %1, 1, %2" : "=v"(a1) : "v"(r1), "s"(b1));
    const uint32_t d0 = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(a0));
    const uint32_t d1 = *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(a1));
    base = b2;
    uint32_t v;
    asm("v_cndmask_b32_e64 %0, 0, %1, %3\n\t"
        "s_mov_b64 vcc, %4\n\t"
        "v_cndmask_b32_sdwa %0, 0, %2, vcc dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:WORD_0"
        : "=&v"(v)
        : "v"(d0), "v"(d1), "s"(w0), "s"(w1)
        : "vcc");
    out[p] = v;
  }
  return __builtin_bit_cast(half8, out);
}

__device__ __forceinline__ _Float16 lds_half(uint32_t addr) {
  return *reinterpret_cast<const lds_f16*>(static_cast<uintptr_t>(addr));
}

// Global -> LDS without registers: lane l writes 16 bytes at lds + 16 l.
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}
// The same with the non-temporal hint (streamed once, not kept in L2).
__device__ __forceinline__ void lds_dma16_nt(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 2);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Wave-uniform reads of the format's read-only arrays through the constant
// address space: always scalar loads, whatever other memory operations the
// kernel performs before them.
template <typename T>
__device__ __forceinline__ T const_load(const void* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ uint64_t word_of(const u32x16& w, int e) {
  return uint64_t(w[2 * e]) | (uint64_t(w[2 * e + 1]) << 32);
}

// Eight fp16 values row[col .. col+7] (zero outside [0, K)), element by element.
__device__ __forceinline__ half8 load8_checked(const uint16_t* row, int64_t col, int64_t K) {
  half8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (col + e < K) ? __builtin_bit_cast(_Float16, row[col + e]) : _Float16(0);
  return v;
}

// Sum the waves' 16x16 (rows x tokens) fp32 accumulators in LDS in fixed wave
// order and store fp16 Y.  `red` holds nwaves*256 floats.  The accumulator
// layout is that of v_mfma_f32_16x16x32: lane l, element v = row 4(l/16)+v,
// token l%16.
__device__ __forceinline__ void slab_reduce_store(float* red, int nwaves, int wave, int lane,
                                                  const f32x4& acc, int slab, int M, int N,
                                                  uint16_t* Y, int64_t ldy) {
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (lane & 15) * 16 + (lane >> 4) * 4 + v] = acc[v];
  __syncthreads();
  const int m0 = slab * kSlab;
  for (int e = threadIdx.x; e < N * kSlab; e += blockDim.x) {
    const int tok = e >> 4, row = e & 15;
    // all (at most 16) partials are read at once, then added in wave order
    float v[16];
#pragma unroll
    for (int w = 0; w < 16; ++w) v[w] = red[min(w, nwaves - 1) * 256 + e];
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) sum += w < nwaves ? v[w] : 0.f;
    if (m0 + row < M) Y[int64_t(tok) * ldy + m0 + row] = __builtin_bit_cast(uint16_t, _Float16(sum));
  }
}

// Gated epilogue: the partials of waves [0, wpm) sum to g and those of waves
// [wpm, 2 wpm) to u, each in fixed wave order; the stored value is
// h = SiLU(g) * u = g / (1 + e^-g) * u in fp32, rounded once to fp16, and +0
// where |h| (as rounded) is below tau.
__device__ __forceinline__ void slab_reduce_glu_store(float* red, int wpm, int wave, int lane, const f32x4& acc,
                                                      int slab, int M, int N, uint16_t* Y, int64_t ldy,
                                                      float tau) {
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave * 256 + (lane & 15) * 16 + (lane >> 4) * 4 + v] = acc[v];
  __syncthreads();
  const int m0 = slab * kSlab;
  for (int e = threadIdx.x; e < N * kSlab; e += blockDim.x) {
    const int tok = e >> 4, row = e & 15;
    float vg[8], vu[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      vg[w] = red[min(w, wpm - 1) * 256 + e];
      vu[w] = red[(wpm + min(w, wpm - 1)) * 256 + e];
    }
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      g += w < wpm ? vg[w] : 0.f;
      u += w < wpm ? vu[w] : 0.f;
    }
    _Float16 h = _Float16(g / (1.f + expf(-g)) * u);
    if (!(fabsf(float(h)) >= tau)) h = _Float16(0.f);
    if (m0 + row < M) Y[int64_t(tok) * ldy + m0 + row] = __builtin_bit_cast(uint16_t, h);
  }
}

struct DecodeArgs {
  const uint32_t* tile_ptr;
  const uint64_t* bits;
  const uint16_t* vals;
  const uint16_t* zeros;
  const uint16_t* X;
  uint16_t* Y;
  int64_t ldx, ldy;
  int M, K, N, kt;
  int tpw;  // tiles per wave
};

// Arguments of the gated instances of the straight-line kernel: waves
// [0, wpm) decode the first format (gate), waves [wpm, 2 wpm) the second (up,
// same M and K), and the epilogue stores SiLU(g) * u with |.| < tau dropped.
// A separate type keeps the ungated instances' arguments as they are.
struct GluArgs : DecodeArgs {
  const uint32_t* tile_ptr2;
  const uint64_t* bits2;
  const uint16_t* vals2;
  int wpm;
  float tau;
};
template <bool kGlu>
struct SeqArgs {
  using type = DecodeArgs;
};
template <>
struct SeqArgs<true> {
  using type = GluArgs;
};

constexpr int kSegTiles = 4;  // tiles per streamed segment

// One workgroup per 16-row slab; wave w decodes tiles [w*tpw, w*tpw + tpw),
// which are one contiguous stream in memory.  The stream is fetched in
// segments of kSegTiles tiles, each as kC fixed 1 KiB loads (addresses clamped
// into the segment, so loads past its end re-read cached bytes instead of
// branching; kC covers the largest segment of the matrix).  Segments go
// through a two-deep register ring: segment g+2 is requested while segment g
// is decoded from LDS.  Bitmap words are touched by a vector load two segments
// ahead (into L2) and read by s_load_dwordx16 one step ahead; B operands
// (activations, L2 resident) run two steps ahead.  kSkip: words whose four
// columns carry a zero activation in every token are not decoded (their run
// is still streamed).  kH = 2 serves 17 <= N <= 32 tokens: each decoded A
// operand feeds two MFMAs, one per group of 16 tokens, so the weight stream is
// read once for all of them.
template <int kC, bool kSkip, bool kVec, int kH = 1>
__global__ __launch_bounds__(1024) void decode_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int slab = int(blockIdx.x);

  // LDS: [0,16) zeros | nwaves segment buffers (kC KiB each); the reduction
  // area reuses the segment buffers after a barrier.
  if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(smem)[threadIdx.x] = 0u;
  __syncthreads();
  const uint32_t zero_addr = lds_addr(smem);
  const uint32_t buf = lds_addr(smem + 16 + size_t(wave) * kC * 1024);

  const int j0 = wave * a.tpw;
  const int j1 = min(j0 + a.tpw, a.kt);

  // B operand: lane l carries token 16h + l%16 (token group h < kH), columns
  // 8(l/16) .. +7 of the step.
  const int tok = lane & 15, kq = 8 * (lane >> 4);
  const uint16_t* xrow[kH];
#pragma unroll
  for (int h = 0; h < kH; ++h) xrow[h] = (16 * h + tok < a.N) ? a.X + int64_t(16 * h + tok) * a.ldx : a.zeros;
  const int64_t kmax8 = a.K >= 8 ? a.K - 8 : 0;  // clamp for steps past K (their A is zero)

  f32x4 acc[kH];
#pragma unroll
  for (int h = 0; h < kH; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t keep = 0;  // consumes the L2 prefetches so they are kept

  if (j0 < j1) {
    const uint64_t tbase = uint64_t(slab) * a.kt;
    const int jlast = j1 - 1;
    const int nseg = (j1 - j0 + kSegTiles - 1) / kSegTiles;
    auto seg_first = [&](int g) { return j0 + kSegTiles * min(g, nseg - 1); };
    // A segment in flight: its kC 1 KiB loads and its kSegTiles+1 tile
    // pointers (wave-uniform).  Segments past the wave's last one load one
    // cached 16-byte slot instead of repeating the last segment.
    struct Seg {
      u32x4 r[kC];
      uint32_t tp[kSegTiles + 1];
    };
    auto load_seg = [&](int g, Seg& sg) {
      const int ja = seg_first(g), jb = min(ja + kSegTiles, j1);
#pragma unroll
      for (int i = 0; i <= kSegTiles; ++i) sg.tp[i] = const_load<uint32_t>(a.tile_ptr + tbase + min(ja + i, jb));
      const uint32_t p0 = sg.tp[0], p1 = sg.tp[kSegTiles];
      const bool real = g < nseg;
      const uint32_t last = (real && p1 > p0 + 8) ? p1 - 8 : p0;  // last 8-value slot
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const uint32_t off = min(p0 + uint32_t(c * 512 + lane * 8), last);
        sg.r[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.vals + off));
      }
    };
    auto touch_seg_words = [&](int g) {
      const int ja = seg_first(g), jb = min(ja + kSegTiles, j1);
      const int w = min(lane, 16 * (jb - ja) - 1);
      const u32x2 v = *(reinterpret_cast<const u32x2*>(a.bits + (tbase + ja) * 16) + w);
      keep ^= v[0] ^ v[1];
    };
    auto load_words = [&](int j, int s) -> u32x16 {
      return const_load<u32x16>(a.bits + (tbase + j) * 16 + 8 * s);
    };
    auto load_b = [&](int j, int s, int h) -> half8 {
      int64_t col = int64_t(j) * kTK + 32 * s + kq;
      if constexpr (kVec) {
        col = col < a.K ? col : kmax8;
        return __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(xrow[h] + col));
      } else {
        return load8_checked(xrow[h], col, a.K);
      }
    };

    Seg segA, segB;
    touch_seg_words(0);
    touch_seg_words(1);
    load_seg(0, segA);
    load_seg(1, segB);
    half8 bop[kH][4];
#pragma unroll
    for (int h = 0; h < kH; ++h) {
      bop[h][0] = load_b(j0, 0, h);
      bop[h][1] = load_b(j0, 1, h);
    }
    u32x16 wslot[2];
    wslot[0] = load_words(j0, 0);

    // Decode tile j whose run starts at LDS byte address `run`.  `par` is the
    // tile's parity inside its segment and selects the static B ring slots.
    auto do_tile = [&](int j, uint32_t run, int par) {
      const int jn = min(j + 1, jlast);
      uint64_t active = ~0ull;
      if constexpr (kSkip) {
        bool nz = false;
        const int64_t col = int64_t(j) * kTK + lane;
        if (col < a.K)
          for (int n = 0; n < a.N; ++n) nz |= (a.X[int64_t(n) * a.ldx + col] & 0x7FFFu) != 0;
        active = __ballot(nz);
      }
      uint32_t base = run;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // This step's words (their scalar popcounts force the wait first),
        // then the lookahead: words one step ahead, B two steps ahead.
        const u32x16 wv = wslot[s];
        uint32_t pc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pc[e] = 2u * uint32_t(__builtin_popcountll(word_of(wv, e)));
        __builtin_amdgcn_sched_barrier(0);
        wslot[s ^ 1] = (s == 0) ? load_words(j, 1) : load_words(jn, 0);
#pragma unroll
        for (int h = 0; h < kH; ++h) bop[h][(2 * par + s + 2) & 3] = load_b(jn, s, h);
        __builtin_amdgcn_sched_barrier(0);
        half8 aop;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (kSkip) {
            // word e of step s covers columns 32s + 8q + e, q = 0..3
            if (((active >> (32 * s + e)) & 0x01010101ull) == 0) {
              aop[e] = _Float16(0);
              base += pc[e];
              continue;
            }
          }
          const uint32_t ad = run_addr(word_of(wv, e), base, zero_addr);
          base += pc[e];
          aop[e] = lds_half(ad);
        }
#pragma unroll
        for (int h = 0; h < kH; ++h)
          acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[h][(2 * par + s) & 3], acc[h], 0, 0, 0);
      }
    };

    // Stage segment g (in `sg`) into LDS, request segment g+2 into `sg`, then
    // decode the segment's tiles.
    auto do_seg = [&](int g, Seg& sg) {
#pragma unroll
      for (int c = 0; c < kC; ++c)
        *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(buf + c * 1024 + lane * 16)) = sg.r[c];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const int ja = j0 + kSegTiles * g;
      uint32_t run[kSegTiles];
#pragma unroll
      for (int tt = 0; tt < kSegTiles; ++tt) run[tt] = buf + 2u * (sg.tp[tt] - sg.tp[0]);
      load_seg(g + 2, sg);
      touch_seg_words(g + 2);
#pragma unroll
      for (int tt = 0; tt < kSegTiles; ++tt) {
        const int j = ja + tt;
        if (j >= j1) break;
        do_tile(j, run[tt], tt & 1);
      }
    };

    for (int g = 0; g < nseg; g += 2) {
      do_seg(g, segA);
      if (g + 1 < nseg) do_seg(g + 1, segB);
    }
  }
  if (keep == 0x9E3779B9u && a.N < 0) a.Y[0] = 0;  // never true: keeps the prefetch loads

  __syncthreads();  // all segment buffers are free: reuse them as the reduction area
  slab_reduce_store(reinterpret_cast<float*>(smem + 16), nwaves, wave, lane, acc[0], slab, a.M, min(a.N, 16),
                    a.Y, a.ldy);
  if constexpr (kH == 2) {
    __syncthreads();  // every thread is done reading the first group's partials
    slab_reduce_store(reinterpret_cast<float*>(smem + 16), nwaves, wave, lane, acc[1], slab, a.M, a.N - 16,
                      a.Y + 16 * a.ldy, a.ldy);
  }
}

// ------------------------------------------------------------------ sparse, straight-line schedule
// Same work split as decode_kernel (one workgroup per slab, wave w owns tiles
// [w*tpw, w*tpw + tpw) with tpw <= 2*NS; in gated mode the second half of the
// waves does the same over the second format), but the whole wave program is
// unrolled so that every vector load is issued unconditionally in a fixed
// order, and each wait covers exactly the data it needs (vector loads return
// in issue order):
//   * the wave's tile pointers and the first bitmap step are requested first
//     (scalar), then the bitmap words of the range are touched into L2 so
//     that the per-step scalar loads hit there;
//   * per segment of two tiles, the activations of its 128 columns for the N
//     tokens are loaded first, then its value chunks (kC 1 KiB loads, with
//     the non-temporal hint), both straight into the wave's LDS
//     (global_load_lds_dwordx4: four token rows of 256 contiguous bytes, or
//     1 KiB of the run stream, per load; no staging registers and no LDS
//     stores).  Against loads into registers stored to LDS, measured in
//     alternating runs on one box: activations 1.7% / 3.3% faster at N = 16
//     on q_proj / down, values a further 3.9% / 9.5% at N = 16 and 1.9-3.3%
//     at N = 1;
//   * one segment is requested ahead: segment g+1 is issued when segment g
//     has been decoded.  With every wave's whole range in flight at once, the
//     memory system served the waves of a SIMD in launch order and the last
//     one decoded its entire range after the stream had ended; one segment
//     ahead interleaves the waves' requests, so each wave has at most one
//     segment left when the last bytes arrive (measured 5-9% faster on the
//     q_proj, down and up shapes);
//   * a segment's decode starts once its loads have landed (vmcnt(0)), and
//     the next segment is requested only after every LDS read of the
//     current one has returned (lgkmcnt(0)), so one LDS region per wave
//     serves all segments; the B operands are read with ds_read_b128 from
//     the staged rows (chunk k of row t at position k ^ t, so the 16 rows of
//     one read meet no bank twice);
//   * the gated instances (kGlu) keep the earlier form: activations and value
//     chunks through registers into a padded row layout, and an opening
//     zero slot and workgroup barrier (with the direct loads and no barrier
//     their launch measured 22% slower, 26.9 against 32.8 us at n = 1 on the
//     gate/up shape, both builds alternating on one box; neither change
//     alone recovered it);
//   * kDB (16 token rows only): the activations are loaded straight in the B
//     operand layout instead, one 1 KiB load per 32-column step (lane l:
//     token l%16, columns 8(l/16) .. +7), and used from registers; the wave
//     needs no LDS for them, so more workgroups fit a CU, at the price of
//     loads that touch 16 token rows each.  Its value chunks go through
//     registers (loaded straight into LDS they measured 1.3% slower: the
//     wait for the LDS reads before each request is then pure cost).
// LDS bytes reserved per staged token row (the rows are 256 bytes; the
// reserve, from an earlier padded layout, keeps the work splits below as
// measured).
constexpr int kXRow = 272;
// LDS bytes per wave for a segment's staged activations (kxi 1 KiB loads;
// none when the B operands are loaded straight into registers).
constexpr int seq_x_bytes(int kxi, bool direct) { return direct ? 0 : 4 * kxi * kXRow; }

template <int NS, int kC, int kXI, bool kGlu = false, bool kDB = false>
__global__ __launch_bounds__(1024) void decode_seq_kernel(typename SeqArgs<kGlu>::type a) {
  static_assert(!kDB || kXI == 4, "B operands straight from memory only with 16 staged token rows");
  constexpr int kT = 2 * NS;      // tile slots per wave
  constexpr int kSteps = 2 * kT;  // 32-column steps
  constexpr int kTouch = (kT * 128 + 1023) / 1024;
  constexpr int kXRows = 4 * kXI;  // token rows of the activation buffer
  constexpr uint32_t kWaveLds = kC * 1024 + (kDB ? 0 : kXRows * kXRow);
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int slab = int(blockIdx.x);

  // LDS: [0,16) unused | per wave: kC KiB of value chunks, then (unless kDB)
  // the segment's activations [kXRows][256 bytes, swizzled]; the reduction area reuses it
  // after a barrier.  No barrier at the start: each wave issues its first
  // loads as soon as it runs (lanes whose bit is clear read a neighbouring
  // value, not a zero slot; 1-2% faster than zeroing a slot and waiting for
  // the whole workgroup first).
  if constexpr (kGlu) {
    // the gated instances keep the zero slot and the opening barrier: their
    // two wave halves measured 22% slower without them and with LDS-direct
    // staging (alternating runs of both builds on one box)
    if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(smem)[threadIdx.x] = 0u;
    __syncthreads();
  }
  const uint32_t buf = lds_addr(smem + 16 + size_t(wave) * kWaveLds);
  const uint32_t xbuf = buf + kC * 1024;

  // The format this wave decodes (wave-uniform; the second one only in the
  // gated instances).
  const uint32_t* tile_ptr = a.tile_ptr;
  const uint64_t* bits = a.bits;
  const uint16_t* vals = a.vals;
  int fwave = wave;
  if constexpr (kGlu) {
    if (wave >= a.wpm) {
      tile_ptr = a.tile_ptr2;
      bits = a.bits2;
      vals = a.vals2;
      fwave = wave - a.wpm;
    }
  }
  const int j0 = fwave * a.tpw;
  const int nt = min(a.tpw, a.kt - j0);  // tiles of this wave (<= kT)

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint32_t keep = 0;
  if (nt > 0) {
    const uint64_t tb = uint64_t(slab) * a.kt + j0;  // first tile of the range
    const int kmax8 = a.K - 8;                        // K >= 8 and K % 8 == 0 on this path

    uint32_t tp[kT + 1];
#pragma unroll
    for (int i = 0; i <= kT; ++i) tp[i] = const_load<uint32_t>(tile_ptr + tb + min(i, nt));
    u32x16 wv[kSteps];
    auto load_w = [&](int t) {
      const int jt = min(t >> 1, nt - 1);
      wv[t] = const_load<u32x16>(bits + (tb + jt) * 16 + 8 * (t & 1));
    };
    load_w(0);
    __builtin_amdgcn_sched_barrier(0);

    u32x4 th[kTouch];
    {
      const uint32_t wbytes = uint32_t(nt) * 128u;
      const uint8_t* wb = reinterpret_cast<const uint8_t*>(bits + tb * 16);
#pragma unroll
      for (int i = 0; i < kTouch; ++i)
        th[i] = *reinterpret_cast<const u32x4*>(wb + min(uint32_t(i * 1024 + lane * 16), wbytes - 16u));
    }

    // Activation pieces: piece p = 64 i + lane is token p/16 (rows past N
    // repeat token N-1), columns 8 (p%16) .. +7 of the segment; with kDB,
    // load i is step i's B operand (token lane%16, rows past N repeating
    // token N-1, columns 32 i + 8 (lane/16) .. +7).  Byte offsets fit 32 bits
    // (16 tokens of at most 2^27 halves).
    // direct: activations and value chunks go straight into LDS; otherwise
    // (the B-operand instances, and gated ones unless switched) through
    // registers
    constexpr bool direct = !kDB && !kGlu;
    uint32_t xrow_off[kXI], xcol[kXI], xl[kXI];
#pragma unroll
    for (int i = 0; i < kXI; ++i) {
      const int pce = i * 64 + lane;
      xl[i] = xbuf + uint32_t(pce >> 4) * kXRow + 16u * uint32_t(pce & 15);
      if constexpr (kDB) {
        xrow_off[i] = 2u * uint32_t(min(lane & 15, a.N - 1)) * uint32_t(a.ldx);
        xcol[i] = 32u * uint32_t(i) + 8u * uint32_t(lane >> 4);
      } else if (!direct) {
        xrow_off[i] = 2u * uint32_t(min(pce >> 4, a.N - 1)) * uint32_t(a.ldx);
        xcol[i] = 8u * uint32_t(pce & 15);
      } else {
        // LDS-direct staging: load i fills rows 4i .. 4i+3 of 256 bytes
        // (lane l at row 4i + l/16, position l%16; rows past N repeat token
        // N-1); the lane fetches chunk (l%16) ^ row, so chunk k of row t sits
        // at position k ^ t and the B reads of one instruction (16 rows, one
        // chunk) meet no LDS bank twice
        xrow_off[i] = 2u * uint32_t(min(pce >> 4, a.N - 1)) * uint32_t(a.ldx);
        xcol[i] = 8u * uint32_t((pce & 15) ^ ((pce >> 4) & 15));
      }
    }
    // B operand: lane l carries token l%16 (rows past kXRows repeat a valid
    // row; their accumulator columns are never stored), columns 8(l/16) .. +7
    // of the step: chunk 4q + l/16 of the segment for step q = 2 tt + s
    const uint32_t xrow = uint32_t(min(lane & 15, kXRows - 1));
    const uint32_t xb = xbuf + xrow * kXRow + 16u * uint32_t(lane >> 4);  // register-staged layout
    uint32_t xsw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xsw[q] = xbuf + xrow * 256u + 16u * ((uint32_t(4 * q) + uint32_t(lane >> 4)) ^ xrow);

    u32x4 xr[NS][(kDB || kGlu) ? kXI : 1];  // activations in registers (kDB, gated)
    u32x4 r[NS][(kDB || kGlu) ? kC : 1];  // value chunks in registers
    // Segment g: its activations, then its value chunks.  For g = 0 the first
    // step's bitmap is folded into the first tile pointer with a mask that is
    // always zero (N >= 1), so the wait for the pointers also covers that
    // scalar load, which would otherwise sink behind the first staging
    // branches and be waited for there.
    auto issue_seg = [&](int g) {
      const int c0 = (j0 + 2 * g) * kTK;
      if (direct) {
        // the previous segment's B and value reads must have returned before
        // its rows and chunks are overwritten
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kXI; ++i) {
          const uint32_t col = uint32_t(min(c0 + int(xcol[i]), kmax8));
          const uint32_t off = xrow_off[i] + 2u * col;  // one 32-bit offset from the uniform base
          lds_dma16(reinterpret_cast<const uint8_t*>(a.X) + off, smem + (xbuf - lds_addr(smem)) + i * 1024);
        }
      } else if constexpr (kDB || kGlu) {
#pragma unroll
        for (int i = 0; i < kXI; ++i) {
          const uint32_t col = uint32_t(min(c0 + int(xcol[i]), kmax8));
          xr[g][i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.X) + xrow_off[i] +
                                                     2u * col);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (g == 0) tp[0] += wv[0][0] & uint32_t(a.N >> 31);
      const uint32_t p0 = tp[2 * g], p1 = tp[2 * g + 2];
      const uint32_t last = p1 > p0 + 8 ? p1 - 8 : p0;  // last 8-value slot of the segment
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const uint32_t off = min(p0 + uint32_t(c * 512 + lane * 8), last);
        if constexpr (kDB || kGlu) {
          if (!direct)
            r[g][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vals + off));
          else
            lds_dma16_nt(vals + off, smem + (buf - lds_addr(smem)) + c * 1024);
        } else {
          lds_dma16_nt(vals + off, smem + (buf - lds_addr(smem)) + c * 1024);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    issue_seg(0);

#pragma unroll
    for (int g = 0; g < NS; ++g) {
      const uint32_t p0 = tp[2 * g];
      if (2 * g < nt) {
        // The segment's activations and all its value chunks (chunks past the
        // segment hold clamped duplicates and are never read).
        if constexpr (kDB || kGlu) {
          if (!direct) {
            if constexpr (!kDB) {
#pragma unroll
              for (int i = 0; i < kXI; ++i)
                *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(xl[i])) = xr[g][i];
            }
#pragma unroll
            for (int c = 0; c < kC; ++c)
              *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(buf + c * 1024 + lane * 16)) = r[g][c];
          }
        }
        if (direct) {
          // the segment's LDS-direct rows and chunks have landed
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
          __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int jt = 2 * g + tt;
        if (jt == 0 || jt < nt) {  // tile slot 0 always exists (nt >= 1)
          if (jt == 0) {
#pragma unroll
            for (int i = 0; i < kTouch; ++i) keep ^= th[i][0] ^ th[i][1] ^ th[i][2] ^ th[i][3];
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          uint32_t base = buf + 2u * (tp[jt] - p0);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int t = 2 * jt + s;
            const u32x16 w = wv[t];
            // wait for this step's words, then request the next step's
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t wk = w[0];
            asm volatile("" ::"s"(wk));
            if (t + 1 < kSteps) load_w(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            half8 bop;
            if constexpr (kDB)
              bop = __builtin_bit_cast(half8, xr[g][2 * tt + s]);
            else if (direct)
              bop = __builtin_bit_cast(half8,
                                       *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(xsw[2 * tt + s])));
            else
              bop = __builtin_bit_cast(
                  half8, *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(xb + tt * 128 + s * 64)));
            const half8 aop = decode_step(w, base);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc, 0, 0, 0);
          }
        }
      }
      if (g + 1 < NS) issue_seg(g + 1);
    }
  }
  if (keep == 0x9E3779B9u && a.N < 0) a.Y[0] = 0;  // never true: keeps the L2 touch loads
  // LDS-direct rows requested for segments past a short range are never
  // read; they must have landed before the area is reused
  if constexpr (!kDB && !kGlu) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  __syncthreads();  // all wave buffers are free: reuse them as the reduction area
  if constexpr (kGlu)
    slab_reduce_glu_store(reinterpret_cast<float*>(smem + 16), a.wpm, wave, lane, acc, slab, a.M, a.N, a.Y, a.ldy,
                          a.tau);
  else
    slab_reduce_store(reinterpret_cast<float*>(smem + 16), nwaves, wave, lane, acc, slab, a.M, a.N, a.Y, a.ldy);
}

// ------------------------------------------------------------------ dense, N <= 16
struct DenseArgs {
  const uint16_t* W;
  const uint16_t* X;
  uint16_t* Y;
  int64_t ldw, ldx, ldy;
  int M, K, N;
  int kc;  // columns per wave, a multiple of 256
};

// Sixteen zero bytes in the code object's own data (zero-initialised when the
// module loads, never written): the source of the dense kernel's loads past
// the end of a wave's columns.
__device__ __attribute__((aligned(16))) uint16_t g_zero_chunk[8];

// Same slab decomposition as the sparse kernel: one workgroup per 16-row slab,
// wave w covers columns [w*kc, w*kc + kc).  Per 32 columns one
// v_mfma_f32_16x16x32_f16 with A = W[16 rows][32 columns] (lane l loads row
// l%16, columns 8(l/16) .. +7: 16 B) and B = X[16 tokens][32 columns].  Loads
// run seven steps ahead through an eight-slot register ring; loads past the
// wave's columns read g_zero_chunk.  Rows past M read row M-1 and tokens past
// N read token N-1: their accumulator entries are never stored.
//
// kXI > 0 (5-16 tokens): the activations are staged through LDS as in the
// sparse kernel instead of loaded in the B operand layout, whose loads touch
// 16 token rows of 64 bytes each: per 128-column segment kXI loads of 4 token
// rows x 256 contiguous bytes (whole cache lines), two segments ahead, stored
// into the wave's LDS rows and read back as B operands with ds_read_b128.
constexpr int kDXRow = 272;  // LDS bytes per staged token row (256 + pad)

template <bool kVec, int kXI = 0>
__global__ __launch_bounds__(1024) void dense_small_kernel(DenseArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int nwaves = int(blockDim.x >> 6);
  const int slab = int(blockIdx.x);
  const int64_t kb = int64_t(wave) * a.kc;
  const int64_t ke = min(kb + a.kc, int64_t(a.K));
  const int kq = 8 * (lane >> 4);
  const int tok = lane & 15;
  const int64_t row = min(int64_t(slab) * kSlab + (lane & 15), int64_t(a.M) - 1);
  const uint16_t* wrow = a.W + row * a.ldw;
  const uint16_t* xrow = a.X + int64_t(min(tok, a.N - 1)) * a.ldx;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (kb < ke) {
    if constexpr (kVec && kXI > 0) {
      constexpr int kXRows = 4 * kXI;
      const int nsteps = int((ke - kb + 31) / 32);  // a multiple of 8 but for the last wave
      const uint32_t xs = lds_addr(smem) + uint32_t(wave) * (kXRows * kDXRow);
      // staged piece p = 64 i + lane: token p/16 (rows past N repeat token
      // N-1), 16-byte chunk p%16 of the segment's 256 bytes
      const uint16_t* xsrc[kXI];
      uint32_t xdst[kXI];
      int xch[kXI];
#pragma unroll
      for (int i = 0; i < kXI; ++i) {
        const int pce = 64 * i + lane;
        xsrc[i] = a.X + int64_t(min(pce >> 4, a.N - 1)) * a.ldx;
        xch[i] = 8 * (pce & 15);
        xdst[i] = xs + uint32_t(pce >> 4) * kDXRow + 16u * uint32_t(pce & 15);
      }
      // B operand: token lane%16 (rows past kXRows repeat a staged row; their
      // accumulator columns are never stored), columns 8(lane/16) .. +7
      const uint32_t xb = xs + uint32_t(min(lane & 15, kXRows - 1)) * kDXRow + 16u * uint32_t(lane >> 4);
      half8 A[8];
      u32x4 xr[2][kXI];
      auto issueA = [&](int st, int slot) {
        const int64_t k = kb + int64_t(st) * 32 + kq;
        A[slot] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(k < ke ? wrow + k : g_zero_chunk));
      };
      auto issueX = [&](int g, int slot) {
#pragma unroll
        for (int i = 0; i < kXI; ++i) {
          const int64_t k = kb + int64_t(g) * 128 + xch[i];
          xr[slot][i] = *reinterpret_cast<const u32x4*>(k < ke ? xsrc[i] + k : g_zero_chunk);
        }
      };
      issueX(0, 0);
      issueX(1, 1);
#pragma unroll
      for (int u = 0; u < 7; ++u) issueA(u, u);
      for (int s0 = 0; s0 < nsteps; s0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if ((u & 3) == 0) {
            // segment (s0 + u) / 4 into the wave's LDS rows (its previous
            // segment's B reads were issued before these writes), then the
            // segment two ahead into the freed registers
            const int slot = u >> 2;
#pragma unroll
            for (int i = 0; i < kXI; ++i)
              *reinterpret_cast<lds_u32x4*>(static_cast<uintptr_t>(xdst[i])) = xr[slot][i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            issueX((s0 + u) / 4 + 2, slot);
          }
          issueA(s0 + u + 7, (u + 7) & 7);
          const half8 B = __builtin_bit_cast(
              half8, *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(xb + 64u * uint32_t(u & 3))));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u], B, acc, 0, 0, 0);
        }
      }
    } else if constexpr (kVec) {
      const int nsteps = int((ke - kb + 31) / 32);
      half8 A[8], B[8];
      auto issue = [&](int s, int slot) {
        const int64_t k = kb + int64_t(s) * 32 + kq;
        const bool ok = k < ke;
        A[slot] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(ok ? wrow + k : g_zero_chunk));
        B[slot] = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(ok ? xrow + k : g_zero_chunk));
      };
#pragma unroll
      for (int u = 0; u < 7; ++u) issue(u, u);
      for (int s0 = 0; s0 < nsteps; s0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          issue(s0 + u + 7, (u + 7) & 7);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[u], B[u], acc, 0, 0, 0);
        }
      }
    } else {
      for (int64_t k0 = kb; k0 < ke; k0 += 32) {
        const int64_t k = k0 + kq;
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(load8_checked(wrow, k, ke), load8_checked(xrow, k, ke),
                                                     acc, 0, 0, 0);
      }
    }
  }
  if constexpr (kXI > 0) __syncthreads();  // every wave is done with its staged rows
  slab_reduce_store(reinterpret_cast<float*>(smem), nwaves, wave, lane, acc, slab, a.M, a.N, a.Y, a.ldy);
}

// ------------------------------------------------------------------ HBM stream calibration
// Reads `n16` 16-byte words; each wave walks a contiguous slice with kU
// dwordx4 loads in flight per lane and folds them into one word per wave.
// Measures the read bandwidth reachable for a given byte count and launch.
template <int kU>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ out) {
  const size_t waves = size_t(gridDim.x) * (blockDim.x >> 6);
  const size_t wave = size_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const size_t per = (n16 + waves - 1) / waves;
  const size_t b = wave * per, e = min(b + per, n16);
  uint32_t acc = 0;
  size_t i = b;
  for (; i + size_t(kU) * 64 <= e; i += size_t(kU) * 64) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 64 + lane);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < e; i += 64)
    if (i + lane < e) {
      const u32x4 v = src[i + lane];
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  acc ^= __shfl_xor(acc, 32);
  acc ^= __shfl_xor(acc, 16);
  acc ^= __shfl_xor(acc, 8);
  acc ^= __shfl_xor(acc, 4);
  acc ^= __shfl_xor(acc, 2);
  acc ^= __shfl_xor(acc, 1);
  if (lane == 0) out[wave] = acc;
}

// ------------------------------------------------------------------ decompress
// One wave per 16x64 tile.  The tile's value run (at most 1024 halves, two
// coalesced 1 KiB loads) and its 16 bitmap words (two scalar 64-byte loads)
// are requested together, so a tile waits for one memory round trip; the run
// is staged in LDS, each word is decoded against it into an LDS tile
// [16][64+8] (padded rows), and the rows of W are written with 16-byte stores.
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
  __shared__ __attribute__((aligned(16))) uint16_t run[4][1024];
  // A wave's 16 x 64 tile as 16 rows of 32 dwords (two fp16 each); dword d
  // of row r is stored at d ^ swz(r), swz flipping bits 0, 1 and 4 by the row,
  // so that neither the paired-column stores (16 rows x 4 column groups per
  // instruction) nor the 16-byte row reads meet in an LDS bank.
  __shared__ __attribute__((aligned(16))) uint32_t tile[4][16][32];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= a.tiles) return;
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
  auto swz = [](int r) { return uint32_t(((r >> 1) & 3) | (((r >> 3) & 1) << 4)); };
  const int row = lane & 15;
  const uint32_t h = swz(row);
  uint32_t pos = 0;
#pragma unroll
  for (int w = 0; w < 16; w += 2) {
    // words w and w + 1 hold this lane's columns col and col + 1 (col even)
    uint32_t v2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint64_t word = word_of((w + e) < 8 ? wa : wb, (w + e) & 7);
      const bool set = (word >> lane) & 1ull;
      const uint32_t rank =
          __builtin_amdgcn_mbcnt_hi(uint32_t(word >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(word), 0u));
      v2[e] = set ? uint32_t(run[wave][min(pos + rank, 1023u)]) : 0u;
      pos += uint32_t(__builtin_popcountll(word));
    }
    const int col = 32 * (w >> 3) + 8 * (lane >> 4) + (w & 7);
    tile[wave][row][uint32_t(col >> 1) ^ h] = v2[0] | (v2[1] << 16);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // lane -> (row = lane/8 + 8*it, 8-column chunk = lane%8)
  for (int it = 0; it < 2; ++it) {
    const int r = it * 8 + (lane >> 3), ch = lane & 7;
    const uint32_t hr = swz(r);
    // the chunk's four dwords: physical chunk ch ^ (bit 4 of swz) / 4, dword j at j ^ (swz & 3)
    const u32x4 raw = *reinterpret_cast<const u32x4*>(&tile[wave][r][uint32_t(4 * ch) ^ (hr & 16u)]);
    const u32x4 s1 = (hr & 1u) ? u32x4{raw[1], raw[0], raw[3], raw[2]} : raw;
    const u32x4 c = (hr & 2u) ? u32x4{s1[2], s1[3], s1[0], s1[1]} : s1;
    const int64_t grow = int64_t(slab) * kSlab + r, gcol = int64_t(tj) * kTK + ch * 8;
    if (grow >= a.M) continue;
    if (a.vec && gcol + 8 <= a.K) {
      *reinterpret_cast<u32x4*>(a.W + grow * a.ldw + gcol) = c;
    } else {
      for (int e = 0; e < 8; ++e)
        if (gcol + e < a.K) a.W[grow * a.ldw + gcol + e] = uint16_t(c[e / 2] >> (16 * (e % 2)));
    }
  }
}

template <int NS, int kXI, bool kGlu, bool kDB = false>
void launch_seq_x(int kc, dim3 grid, dim3 block, size_t lds, hipStream_t s, const typename SeqArgs<kGlu>::type& a) {
  switch (kc) {
    case 1: hipLaunchKernelGGL((decode_seq_kernel<NS, 1, kXI, kGlu, kDB>), grid, block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((decode_seq_kernel<NS, 2, kXI, kGlu, kDB>), grid, block, lds, s, a); break;
    case 3: hipLaunchKernelGGL((decode_seq_kernel<NS, 3, kXI, kGlu, kDB>), grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL((decode_seq_kernel<NS, 4, kXI, kGlu, kDB>), grid, block, lds, s, a); break;
  }
}

template <int NS, bool kGlu = false>
void launch_seq_ns(int kc, int kxi, bool direct, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                   const typename SeqArgs<kGlu>::type& a) {
  if (kxi == 1) launch_seq_x<NS, 1, kGlu>(kc, grid, block, lds, s, a);
  else if (kxi == 2) launch_seq_x<NS, 2, kGlu>(kc, grid, block, lds, s, a);
  else if (direct) launch_seq_x<NS, 4, kGlu, true>(kc, grid, block, lds, s, a);
  else launch_seq_x<NS, 4, kGlu>(kc, grid, block, lds, s, a);
}

// Smallest instantiated segment count covering `segs` two-tile segments (0: none).
int seq_instance(int segs) {
  static const int kInst[] = {1, 2, 3, 4, 6, 8};
  for (int v : kInst)
    if (segs <= v) return v;
  return 0;
}

template <int kC>
void launch_decode_c(bool skip, dim3 grid, dim3 block, size_t lds, hipStream_t s, const DecodeArgs& a) {
  if (a.N > 16) hipLaunchKernelGGL((decode_kernel<kC, false, true, 2>), grid, block, lds, s, a);
  else if (skip) hipLaunchKernelGGL((decode_kernel<kC, true, true>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((decode_kernel<kC, false, true>), grid, block, lds, s, a);
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return (e && atoi(e) > 0) ? atoi(e) : dflt;
}

}  // namespace

// ------------------------------------------------------------------ host launchers
// Largest two-tile segment of ranges of `tpw` tiles, in 1 KiB loads.
static int seq_chunks_for(const Header& h, const uint32_t* tp, int64_t tpw) {
  uint64_t max2 = 0;
  for (uint64_t i = 0; i < h.mt; ++i)
    for (int64_t ja = 0; ja < int64_t(h.kt); ja += tpw)
      for (int64_t js = ja; js < std::min<int64_t>(ja + tpw, h.kt); js += 2) {
        const int64_t je = std::min<int64_t>({js + 2, ja + tpw, int64_t(h.kt)});
        const uint64_t b = 2ull * (tp[i * h.kt + je] - tp[i * h.kt + js]);
        if (b > max2) max2 = b;
      }
  const int c = int((max2 + 1023) / 1024);
  return c < 1 ? 1 : c;
}

DecodePlan plan_decode(const Header& h, const uint32_t* tp, int num_cus, int waves_per_cu, bool straight_line,
                       int kxi) {
  DecodePlan p;
  const int64_t tiles = int64_t(h.mt) * h.kt;
  const int64_t min_tpw = (int64_t(h.kt) + 15) / 16;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  int64_t tpw = 0;
  if (straight_line && kxi > 0 && min_tpw <= 16) {
    // Straight-line kernel: the split with the most waves resident per CU.
    // A workgroup (one slab) of w waves holds w * (value chunks + kxi * 4
    // staged activation rows) of LDS; a CU runs as many workgroups as its
    // 160 KiB of LDS, its 32 wave slots and the slab count allow.  Ranges
    // are whole two-tile segments (an even tile count, or the least count
    // that covers a slab row with 16 waves); ties go to fewer tiles per
    // wave.  Measured on the layer shapes at N = 8 / 16 (one box, us): q/k/v
    // stacked 12288x4096 N = 8: 22.9 / 18.4 / 16.7 / 18.6 / 19.7 at 4 / 6 /
    // 8 / 11 / 16 tiles per wave (this rule: 8); gate/up stacked 22016x4096
    // N = 16: 41.4 / 35.1 / 37.2 / 38.7 / 36.8 (this rule: 6; the earlier
    // rule, about 32 waves per CU, took 11).  An odd count that leaves the
    // slab's last wave one tile measured slower (7 at N = 8 on gate/up:
    // 33.9 us against 30.3 for 6).
    auto best_split = [&](bool direct, int64_t& score) {
      int64_t best_t = 0;
      score = -1;
      for (int64_t t = min_tpw; t <= 16; t = (t + 2) & ~int64_t(1)) {
        const int64_t w = (int64_t(h.kt) + t - 1) / t;
        if (w > 16 || seq_instance(int((t + 1) / 2)) == 0) continue;
        const int chunks = seq_chunks_for(h, tp, t);
        if (chunks > 4) continue;
        const int64_t lds = 16 + w * (int64_t(chunks) * 1024 + seq_x_bytes(kxi, direct));
        if (lds > 160 * 1024) continue;
        const int64_t per_cu =
            std::min<int64_t>({int64_t(160 * 1024) / lds, 32 / w, (int64_t(h.mt) + cus - 1) / cus});
        if (per_cu * w > score) {
          score = per_cu * w;
          best_t = t;
        }
      }
      return best_t;
    };
    // With 16 token rows the B operands can instead be loaded straight into
    // registers (no activation staging in LDS).  Those loads touch 16 rows
    // per instruction instead of 4, which costs 11-15% on shapes whose
    // workgroups fill the CUs either way (q_proj, down at N = 16); taken only
    // where the freed LDS gives at least 1.25x the resident waves (up
    // 11008x4096 N = 12 / 16: 17.36 / 18.08 us against 18.13 / 18.88;
    // gate/up stacked 22016x4096: 30.36 / 32.42 against 32.93 / 34.58).
    int64_t score = 0, score_d = 0;
    tpw = best_split(false, score);
    if (kxi == 4) {
      const int64_t td = best_split(true, score_d);
      if (td > 0 && 4 * score_d >= 5 * score) {
        tpw = td;
        p.direct_b = true;
      }
    }
  }
  if (tpw == 0) {
    // About `waves_per_cu` waves per CU (SWM_DECODE_WAVES_PER_CU overrides).
    // When that leaves more tiles per wave than the straight-line kernel
    // holds, it runs with its largest instance (16 tiles per wave) if a slab
    // row fits 16 such waves and the split is for token counts it serves (on
    // the 65536x16384 shape: 339 / 363 us at N = 1 / 16 against 368 / 373 us
    // for one round of 16 waves per CU of the looped kernel, and 414 us at
    // N = 16 for 128 tiles per wave); else the looped kernel runs one round
    // of 16 waves per CU (at N = 32 on that shape: 581 us, against 666 us
    // with 16 tiles per wave).
    auto split = [&](int64_t wpc) {
      const int64_t t = (tiles + cus * wpc - 1) / (cus * wpc);
      return t < min_tpw ? min_tpw : t;
    };
    tpw = split(env_int("SWM_DECODE_WAVES_PER_CU", waves_per_cu));
    if (seq_instance(int((tpw + 1) / 2)) == 0) tpw = straight_line && min_tpw <= 16 ? 16 : split(16);
  }
  if (tpw < 1) tpw = 1;
  tpw = env_int("SWM_DECODE_TPW", int(tpw));  // tuning override
  if (tpw < min_tpw) tpw = min_tpw;
  p.tiles_per_wave = int(tpw);
  p.waves = int((int64_t(h.kt) + tpw - 1) / tpw);
  if (p.waves < 1) p.waves = 1;
  p.seg_tiles = kSegTiles;
  // Largest segment (kSegTiles consecutive tiles of one wave) in 1 KiB loads.
  uint64_t max_bytes = 0;
  for (uint64_t i = 0; i < h.mt; ++i)
    for (int64_t ja = 0; ja < int64_t(h.kt); ja += tpw)
      for (int64_t js = ja; js < std::min<int64_t>(ja + tpw, h.kt); js += kSegTiles) {
        const int64_t je = std::min<int64_t>({js + kSegTiles, ja + tpw, int64_t(h.kt)});
        const uint64_t b = 2ull * (tp[i * h.kt + je] - tp[i * h.kt + js]);
        if (b > max_bytes) max_bytes = b;
      }
  p.seg_chunks = int((max_bytes + 1023) / 1024);
  if (p.seg_chunks < 1) p.seg_chunks = 1;
  // Straight-line schedule: two-tile segments aligned to each wave's range.
  p.seq_segs = seq_instance(int((tpw + 1) / 2));
  p.seq_chunks = seq_chunks_for(h, tp, tpw);
  if (p.seq_chunks > 4) p.seq_segs = 0;  // cannot happen: two tiles hold at most 4 KiB
  // ablation: the looped kernel everywhere (SWM_DECODE_PATH=loop, or SWM_DECODE_LOOP set)
  const char* path = getenv("SWM_DECODE_PATH");
  if (getenv("SWM_DECODE_LOOP") || (path && !strcmp(path, "loop"))) p.seq_segs = 0;
  return p;
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
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int(f.h.m);
  a.K = int(f.h.k);
  a.N = n;
  a.kt = int(f.h.kt);
  a.tpw = p.tiles_per_wave;
  if (f.h.tm != uint32_t(kSlab) || f.h.tk != uint32_t(kTK)) return hipErrorInvalidValue;
  if (p.seg_chunks > 8) return hipErrorInvalidValue;  // 4 tiles hold at most 8 KiB
  const bool vec = (f.h.k % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  const int kC = vec ? p.seg_chunks : 8;
  const size_t run_bytes = size_t(p.waves) * kC * 1024;
  const size_t red_bytes = size_t(p.waves) * 256 * 4;
  const size_t lds = 16 + (run_bytes > red_bytes ? run_bytes : red_bytes);
  if (f.h.mt == 0) return hipSuccess;
  const dim3 grid{unsigned(f.h.mt), 1, 1}, block{unsigned(p.waves * 64), 1, 1};
  // The straight-line kernel addresses X with 32-bit byte offsets.
  const bool x32 = 2 * ((int64_t(n) - 1) * ldx + f.h.k) < (int64_t(1) << 32);
  // Activation skipping is not applied on this path: with 16-row tiles a
  // bitmap word spans four columns (all inactive for only ~0.7^4 = 24% of
  // words at 70% zero activations) and a column run is at most 32 bytes, so
  // neither the decode nor the fetch of inactive columns can be dropped
  // profitably; the product is computed in full (same result).
  if (vec && p.seq_segs > 0 && a.K >= 8 && x32 && n <= 16) {
    const int kxi = n <= 4 ? 1 : n <= 8 ? 2 : 4;
    const bool direct = p.direct_b && kxi == 4;
    const size_t per_wave = size_t(p.seq_chunks) * 1024 + size_t(seq_x_bytes(kxi, direct));
    const size_t seq_lds = 16 + size_t(p.waves) * per_wave;
    switch (p.seq_segs) {
      case 1: launch_seq_ns<1>(p.seq_chunks, kxi, direct, grid, block, seq_lds, s, a); break;
      case 2: launch_seq_ns<2>(p.seq_chunks, kxi, direct, grid, block, seq_lds, s, a); break;
      case 3: launch_seq_ns<3>(p.seq_chunks, kxi, direct, grid, block, seq_lds, s, a); break;
      case 4: launch_seq_ns<4>(p.seq_chunks, kxi, direct, grid, block, seq_lds, s, a); break;
      case 6: launch_seq_ns<6>(p.seq_chunks, kxi, direct, grid, block, seq_lds, s, a); break;
      default: launch_seq_ns<8>(p.seq_chunks, kxi, direct, grid, block, seq_lds, s, a); break;
    }
    return hipGetLastError();
  }
  if (!vec) {
    if (n > 16) {
      // unaligned activations: two passes of 16 and n - 16 tokens (a
      // two-group instance of the unaligned kernel would spill registers)
      DecodeArgs a2 = a;
      a2.N = 16;
      hipLaunchKernelGGL((decode_kernel<8, false, false>), grid, block, lds, s, a2);
      a2.X = a.X + 16 * a.ldx;
      a2.Y = a.Y + 16 * a.ldy;
      a2.N = n - 16;
      hipLaunchKernelGGL((decode_kernel<8, false, false>), grid, block, lds, s, a2);
    } else if (skip) hipLaunchKernelGGL((decode_kernel<8, true, false>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((decode_kernel<8, false, false>), grid, block, lds, s, a);
    return hipGetLastError();
  }
  switch (kC) {
    case 1: launch_decode_c<1>(skip, grid, block, lds, s, a); break;
    case 2: launch_decode_c<2>(skip, grid, block, lds, s, a); break;
    case 3: launch_decode_c<3>(skip, grid, block, lds, s, a); break;
    case 4: launch_decode_c<4>(skip, grid, block, lds, s, a); break;
    case 5: launch_decode_c<5>(skip, grid, block, lds, s, a); break;
    case 6: launch_decode_c<6>(skip, grid, block, lds, s, a); break;
    case 7: launch_decode_c<7>(skip, grid, block, lds, s, a); break;
    default: launch_decode_c<8>(skip, grid, block, lds, s, a); break;
  }
  return hipGetLastError();
}

DensePlan plan_dense_small(int64_t M, int64_t K, int n, int num_cus) {
  (void)n;
  DensePlan p;
  // One workgroup per 16-row slab; split K over up to 16 waves so that the
  // call is about one round of `wpc` waves per CU.
  const int64_t slabs = (M + 15) / 16;
  const int64_t wpc = env_int("SWM_DENSE_WAVES_PER_CU", 16);
  int64_t waves = (int64_t(num_cus) * wpc + slabs - 1) / (slabs > 0 ? slabs : 1);
  if (waves > 16) waves = 16;
  if (waves < 1) waves = 1;
  int64_t kc = (K + waves - 1) / waves;
  kc = (kc + 255) / 256 * 256;  // whole 8-step blocks of the load ring
  if (kc < 256) kc = 256;
  p.kchunk = int(kc);
  p.waves = int((K + kc - 1) / kc);
  if (p.waves < 1) p.waves = 1;
  return p;
}

hipError_t launch_dense_small(const DensePlan& p, const uint16_t* W, int64_t ldw, const uint16_t* X,
                              int64_t ldx, uint16_t* Y, int64_t ldy, int64_t M, int64_t K, int n, hipStream_t s) {
  DenseArgs a;
  a.W = W;
  a.X = X;
  a.Y = Y;
  a.ldw = ldw;
  a.ldx = ldx;
  a.ldy = ldy;
  a.M = int(M);
  a.K = int(K);
  a.N = n;
  a.kc = p.kchunk;
  const bool vec = (K % 8 == 0) && (ldx % 8 == 0) && (ldw % 8 == 0) &&
                   ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  const int64_t slabs = (M + 15) / 16;
  if (slabs == 0) return hipSuccess;
  if (n < 1 || n > 16) return hipErrorInvalidValue;
  const dim3 grid{unsigned(slabs), 1, 1}, block{unsigned(p.waves * 64), 1, 1};
  const size_t red = size_t(p.waves) * 256 * 4;
  // 5-16 tokens: activations staged through LDS (4 or 8 KiB-ish per wave)
  const int kxi = n <= 4 ? 0 : n <= 8 ? 2 : 4;
  const size_t stage = size_t(p.waves) * size_t(4 * kxi) * kDXRow;
  const size_t lds = std::max(red, stage);
  if (vec && kxi == 4) hipLaunchKernelGGL((dense_small_kernel<true, 4>), grid, block, lds, s, a);
  else if (vec && kxi == 2) hipLaunchKernelGGL((dense_small_kernel<true, 2>), grid, block, lds, s, a);
  else if (vec) hipLaunchKernelGGL((dense_small_kernel<true>), grid, block, red, s, a);
  else hipLaunchKernelGGL((dense_small_kernel<false>), grid, block, red, s, a);
  return hipGetLastError();
}

DecodePlan plan_decode_glu(const Header& g, const Header& u, int num_cus, int n) {
  // Both formats' tiles in one launch, at most 8 waves per format (16 per
  // workgroup) and at most 16 tiles per wave (the largest straight-line
  // instance).  As for the ungated kernel, the split (an even tile count,
  // or the least that fits 8 waves per format) with the most waves resident
  // per CU, counting the LDS a workgroup needs for its staged activation
  // rows (4, 8 or 16 tokens), the 32 wave slots and the slab count.  On
  // gate/up 11008x4096 that is 8 tiles per wave up to 4 tokens (26.3 us at
  // N = 1 against 28.1 at 16) and 14 from 5 tokens (two A/B runs on one
  // box: 34.8 / 33.7 / 36.8 us at N = 6 / 8 / 16 against 37.1 / 35.5 / 37.9
  // for the earlier split of 8 tiles per wave up to 8 tokens, where a
  // workgroup's staged rows left room for one workgroup per CU, and 16
  // above).
  DecodePlan p;
  const int64_t kt = g.kt;
  const int64_t min_tpw = (kt + 7) / 8;
  const int kxi = n <= 4 ? 1 : n <= 8 ? 2 : 4;
  // Two tiles hold at most 2 * max_tile values: a bound on every segment.
  const uint64_t max2 = 4ull * std::max(g.max_tile, u.max_tile);
  p.seq_chunks = int(std::max<uint64_t>((max2 + 1023) / 1024, 1));
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  auto best_split = [&](bool direct, int64_t& score) {
    int64_t best_t = 0;
    score = -1;
    for (int64_t t = min_tpw; t <= 16; t = (t + 2) & ~int64_t(1)) {
      const int64_t w = 2 * ((kt + t - 1) / t);
      const int64_t lds = 16 + w * (int64_t(p.seq_chunks) * 1024 + seq_x_bytes(kxi, direct));
      if (w > 16 || lds > 160 * 1024) continue;
      const int64_t per_cu =
          std::min<int64_t>({int64_t(160 * 1024) / lds, 32 / w, (int64_t(g.mt) + cus - 1) / cus});
      if (per_cu * w > score) {
        score = per_cu * w;
        best_t = t;
      }
    }
    return best_t;
  };
  // B operands straight into registers where that gives 1.25x the resident
  // waves (as for the ungated kernel)
  int64_t score = 0, score_d = 0;
  int64_t tpw = best_split(false, score);
  if (kxi == 4) {
    const int64_t td = best_split(true, score_d);
    if (td > 0 && 4 * score_d >= 5 * score) {
      tpw = td;
      p.direct_b = true;
    }
  }
  static const int env_tpw = env_int("SWM_GLU_TPW", 0);
  if (env_tpw > 0) tpw = env_tpw;
  if (tpw < min_tpw || tpw > 16 || kt < 1 || p.seq_chunks > 4) {
    p.seq_segs = 0;  // no instance covers this shape
    return p;
  }
  p.tiles_per_wave = int(tpw);
  p.waves = 2 * int((kt + tpw - 1) / tpw);
  // gated instances exist for 1, 2, 4 and 8 two-tile segments per wave
  const int segs = int((tpw + 1) / 2);
  p.seq_segs = segs <= 1 ? 1 : segs <= 2 ? 2 : segs <= 4 ? 4 : 8;
  return p;
}

hipError_t launch_decode_glu(const DevFormat& g, const DevFormat& u, const DecodePlan& p, const uint16_t* X,
                             int64_t ldx, uint16_t* H, int64_t ldh, int n, float tau, hipStream_t s) {
  GluArgs a;
  a.tile_ptr = g.tile_ptr;
  a.bits = g.bits;
  a.vals = g.vals;
  a.zeros = g.zeros;
  a.X = X;
  a.Y = H;
  a.ldx = ldx;
  a.ldy = ldh;
  a.M = int(g.h.m);
  a.K = int(g.h.k);
  a.N = n;
  a.kt = int(g.h.kt);
  a.tpw = p.tiles_per_wave;
  a.tile_ptr2 = u.tile_ptr;
  a.bits2 = u.bits;
  a.vals2 = u.vals;
  a.wpm = p.waves / 2;
  a.tau = tau;
  // The caller has checked these; they are what the straight-line kernel assumes.
  if (g.h.tm != uint32_t(kSlab) || g.h.tk != uint32_t(kTK) || u.h.tm != g.h.tm || u.h.tk != g.h.tk ||
      u.h.m != g.h.m || u.h.k != g.h.k)
    return hipErrorInvalidValue;
  if (p.seq_segs == 0 || p.waves < 2 || p.waves > 16 || p.waves % 2 || n < 1 || n > 16 || a.K < 8 || a.K % 8 ||
      ldx % 8 || (reinterpret_cast<uintptr_t>(X) & 15) || 2 * ((int64_t(n) - 1) * ldx + g.h.k) >= (int64_t(1) << 32))
    return hipErrorInvalidValue;
  if (g.h.mt == 0) return hipSuccess;
  const dim3 grid{unsigned(g.h.mt), 1, 1}, block{unsigned(p.waves * 64), 1, 1};
  const int kxi = n <= 4 ? 1 : n <= 8 ? 2 : 4;
  const bool direct = p.direct_b && kxi == 4;
  const size_t per_wave = size_t(p.seq_chunks) * 1024 + size_t(seq_x_bytes(kxi, direct));
  const size_t lds = 16 + size_t(p.waves) * per_wave;
  switch (p.seq_segs) {
    case 1: launch_seq_ns<1, true>(p.seq_chunks, kxi, direct, grid, block, lds, s, a); break;
    case 2: launch_seq_ns<2, true>(p.seq_chunks, kxi, direct, grid, block, lds, s, a); break;
    case 4: launch_seq_ns<4, true>(p.seq_chunks, kxi, direct, grid, block, lds, s, a); break;
    default: launch_seq_ns<8, true>(p.seq_chunks, kxi, direct, grid, block, lds, s, a); break;
  }
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
  if (f.h.tm != uint32_t(kSlab) || f.h.tk != uint32_t(kTK)) return hipErrorInvalidValue;
  if (a.tiles == 0) return hipSuccess;
  dim3 grid(unsigned((a.tiles + 3) / 4)), block(256);
  hipLaunchKernelGGL(decompress_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream(const void* src, size_t bytes, int unroll, int blocks, uint32_t* out,
                         hipStream_t s) {
  const size_t n16 = bytes / 16;
  const dim3 grid{unsigned(blocks), 1, 1}, block{256, 1, 1};
  const u32x4* p = static_cast<const u32x4*>(src);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_kernel<1>, grid, block, 0, s, p, n16, out); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, grid, block, 0, s, p, n16, out); break;
    case 4: hipLaunchKernelGGL(stream_kernel<4>, grid, block, 0, s, p, n16, out); break;
    case 8: hipLaunchKernelGGL(stream_kernel<8>, grid, block, 0, s, p, n16, out); break;
    default: hipLaunchKernelGGL(stream_kernel<16>, grid, block, 0, s, p, n16, out); break;
  }
  return hipGetLastError();
}

}  // namespace swm
