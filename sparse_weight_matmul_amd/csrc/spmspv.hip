// Activation-skipping decode (spMspV) over the SWM-CR v2 column-run encoding.
//
// Method: "Unified Static-Dynamic Pruning for Efficient LLM Inference" (SPDP),
// abstract -- at decode time the input-adaptive (dynamic) sparsity of the
// activations is exploited by a sparse-matrix x sparse-vector kernel that
// skips zero activations at run time.  "Reduced Matrix Multiplication" (blog
// page, Sec. 4.2) states the identity it rests on: input channels whose
// activation is zero contribute nothing, so the product over the kept
// channels equals the full product.
//
// gfx950 design.  A workgroup (16 waves, one per CU) owns a 256-row block b
// and a range of cps <= 1024 input columns (split s); the grid is S x Mb
// workgroups, about one per CU.  The encoding stores the blocks of a column
// four at a time (one 128-byte line of bitmap words, adjacent runs), and the
// four workgroups of one (split, group of four blocks) are placed on the same
// XCD, so the lines they share are fetched into that XCD's L2 once.
//  1. Active columns: each thread tests one column (any of the n <= 4 tokens
//     nonzero); a wave ballot and v_mbcnt give each active column its slot in
//     a list ordered by (wave, lane), so the list is a deterministic function
//     of x.  The list, the columns' activations (as fp32) and their run
//     bounds go to LDS.  The run pointers of the whole range are read in this
//     pass (8 bytes per column), so the runs need no extra round trip later;
//     inactive columns' runs and bitmaps are never read.
//  2. Wave w takes list entries w, w + 16, ..., in batches of 16; the next
//     batch's loads are issued before the current batch is decoded.  One
//     vector load brings a batch's 4 x 16 bitmap words (lane 4i + q = word q
//     of slot i) and, in the same round trip, all 16 runs are requested (8
//     bytes per lane, clamped into the run).  Runs are copied to the wave's
//     four LDS slots, four at a time.  Decode per 64-row word q: v_readlane
//     moves the word to SGPRs, v_mbcnt gives the lane's rank, a halfword read
//     at run base + 2 rank the value, and v_fma_mix_f32 (fp16 operand, fp32
//     accumulate) runs with exec narrowed to the word, so lanes whose bit is
//     clear are untouched.  Lane l holds rows 64q + l, q = 0..3, for every
//     token.
//  3. The 16 waves' sums are added in LDS in wave order and stored as the
//     workgroup's partial (256 rows x n, fp32).  A second launch adds the S
//     partials of each row in split order (one round of loads at S <= 16)
//     and stores fp16 Y.  Both ways of doing that inside the first launch
//     were measured slower on this chip: the last-arriving workgroup needs
//     an agent-scope release per workgroup, which writes back the XCD's L2
//     each time (several times the whole product), or partials tagged per
//     call and read back with relaxed device-scope atomics (1.1 us slower
//     than the second launch for down_proj, n = 1).  Every sum runs in a
//     fixed order, so results are bitwise reproducible, and the calls keep
//     no state on the device between launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kernels.h"

namespace swm {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kCrWaves = 16;  // waves per workgroup
constexpr int kCrBatch = 16;  // list entries per wave batch
constexpr int kCrSlots = 4;   // LDS run slots per wave

// One batch in registers: the slots' bitmap words and one 8-byte piece of
// each slot's run per lane.
struct CrBatchRegs {
  uint32_t bits_lo, bits_hi;
  u32x2 run[kCrBatch];
};

struct CrArgs {
  const uint32_t* ptr;   // entries + 1
  const uint64_t* bits;  // entries * 4
  const uint16_t* vals;  // padded runs (+ 8 bytes of slack)
  const uint16_t* x;     // token-major n x K
  uint16_t* y;           // token-major n x M
  float* partials;       // [mb][S][4][256]
  int64_t ldx, ldy;
  float tau;             // |x| < tau counts as zero
  int M, K, n, mb, S, cps;
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// acc[t] += f16(d) * x[t] for t < kN, in the lanes whose bit of w is set.  exec
// is narrowed to w for the FMAs (lanes with a clear bit keep acc), and
// v_fma_mix_f32 takes the fp16 operand directly (its conversion to fp32 is
// exact), so the word costs no select and no conversion.  The caller runs
// with every lane of the wave active.
template <int kN>
__device__ __forceinline__ void fma_masked(float (&acc)[4], _Float16 d, const float (&x)[kN], uint64_t w) {
  uint64_t sv;
  if constexpr (kN == 1) {
    asm("s_and_saveexec_b64 %[sv], %[w]\n\t"
        "v_fma_mix_f32 %[a0], %[d], %[x0], %[a0] op_sel_hi:[1,0,0]\n\t"
        "s_mov_b64 exec, %[sv]"
        : [a0] "+v"(acc[0]), [sv] "=&s"(sv)
        : [d] "v"(d), [x0] "v"(x[0]), [w] "s"(w)
        : "scc");
  } else if constexpr (kN == 2) {
    asm("s_and_saveexec_b64 %[sv], %[w]\n\t"
        "v_fma_mix_f32 %[a0], %[d], %[x0], %[a0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %[a1], %[d], %[x1], %[a1] op_sel_hi:[1,0,0]\n\t"
        "s_mov_b64 exec, %[sv]"
        : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [sv] "=&s"(sv)
        : [d] "v"(d), [x0] "v"(x[0]), [x1] "v"(x[1]), [w] "s"(w)
        : "scc");
  } else if constexpr (kN == 3) {
    asm("s_and_saveexec_b64 %[sv], %[w]\n\t"
        "v_fma_mix_f32 %[a0], %[d], %[x0], %[a0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %[a1], %[d], %[x1], %[a1] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %[a2], %[d], %[x2], %[a2] op_sel_hi:[1,0,0]\n\t"
        "s_mov_b64 exec, %[sv]"
        : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [sv] "=&s"(sv)
        : [d] "v"(d), [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [w] "s"(w)
        : "scc");
  } else {
    asm("s_and_saveexec_b64 %[sv], %[w]\n\t"
        "v_fma_mix_f32 %[a0], %[d], %[x0], %[a0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %[a1], %[d], %[x1], %[a1] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %[a2], %[d], %[x2], %[a2] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %[a3], %[d], %[x3], %[a3] op_sel_hi:[1,0,0]\n\t"
        "s_mov_b64 exec, %[sv]"
        : [a0] "+v"(acc[0]), [a1] "+v"(acc[1]), [a2] "+v"(acc[2]), [a3] "+v"(acc[3]), [sv] "=&s"(sv)
        : [d] "v"(d), [x0] "v"(x[0]), [x1] "v"(x[1]), [x2] "v"(x[2]), [x3] "v"(x[3]), [w] "s"(w)
        : "scc");
  }
}

template <int kN>
__global__ __launch_bounds__(1024) void spmspv_cr_kernel(CrArgs a) {
  __shared__ uint16_t s_col[kCrMaxCols];
  __shared__ u32x2 s_p[kCrMaxCols];          // run [start, end) of each listed column
  __shared__ float s_x[kCrMaxCols][4];       // activations of each listed column, as fp32
  __shared__ uint32_t s_cnt[kCrWaves];
  // kCrSlots run slots of 512 B per wave, reused in turn (a wave's LDS
  // accesses complete in order); 16 B of slack: a lane whose bit is clear may
  // read the halfword just past the last slot (its value is not used).  The
  // wave sums of step 3 reuse this area.
  constexpr int kRunWords = kCrWaves * kCrSlots * 128;
  constexpr int kRedWords = kCrWaves * kN * 256;
  __shared__ __attribute__((aligned(16))) uint32_t s_run[(kRunWords > kRedWords ? kRunWords : kRedWords) + 4];
  const int tid = int(threadIdx.x);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroup -> (split s, block b = 4g + j).  Workgroups are handed to the
  // eight XCDs in turn, so ids x, x + 8, x + 16, x + 24 of each run of 32
  // share an XCD: they take the four blocks of one (split, group) item.  The
  // placement only affects speed; any mapping gives the same result.
  const int id = int(blockIdx.x);
  const int item = (id >> 5) * 8 + (id & 7), j = (id >> 3) & 3;
  const int gn = (a.mb + 3) >> 2;
  const int g = item % gn, s = item / gn, b = 4 * g + j;
  if (s >= a.S || b >= a.mb) return;  // uniform, before any barrier
  const int k0 = s * a.cps;
  const int kend = min(k0 + a.cps, a.K);
  // entry of column k0 + t in block b: ebase + 4 t
  const uint64_t ebase = (uint64_t(g) * uint64_t(a.K) + uint64_t(k0)) * 4 + uint64_t(j);

  // ---- 1. active columns of [k0, kend), in (wave, lane) order, with their
  // activations and run bounds (the pointers are read for every column of
  // the range, so the runs can be requested together with the bitmaps)
  {
    const int k = k0 + tid;
    bool on = false;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    u32x2 p = {0u, 0u};
    if (k < kend) {
#pragma unroll
      for (int t = 0; t < kN; ++t) {
        // a token's activation counts when it is nonzero and not below tau
        // (the fp16 value is exact in fp32; tau = 0 keeps every nonzero, and
        // a NaN is never below tau, so it is kept and propagates)
        const uint16_t h = a.x[int64_t(t) * a.ldx + k];
        const float xv = float(__builtin_bit_cast(_Float16, h));
        const bool keep = (h & 0x7FFFu) != 0 && !(__builtin_fabsf(xv) < a.tau);
        v[t] = keep ? xv : 0.f;
        on |= keep;
      }
      p[0] = a.ptr[ebase + 4 * uint64_t(tid)];
      p[1] = a.ptr[ebase + 4 * uint64_t(tid) + 1];
    }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    if (lane == 0) s_cnt[wave] = uint32_t(__builtin_popcountll(bal));
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int i = 0; i < kCrWaves; ++i)
      if (i < wave) base += int(s_cnt[i]);
    if (on) {
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(uint32_t(bal >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0u));
      const int pos = base + int(rank);
      s_col[pos] = uint16_t(tid);
      *reinterpret_cast<f32x4*>(s_x[pos]) = v;
      s_p[pos] = p;
    }
  }
  int L = 0;
#pragma unroll
  for (int i = 0; i < kCrWaves; ++i) L += int(s_cnt[i]);
  __syncthreads();

  // ---- 2. this wave's entries j = wave + 16 e, e = 0 .. nw-1, in batches of
  // kCrBatch; batch g + 1 is fetched before batch g is decoded, so only the
  // first batch's round trip is exposed.
  float acc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[q][t] = 0.f;
  const int nw = __builtin_amdgcn_readfirstlane(L > wave ? (L - wave + kCrWaves - 1) / kCrWaves : 0);
  const uint32_t slots = lds_addr(s_run) + uint32_t(wave) * (kCrSlots * 512);
  // Fetch of batch g: bitmap words (lane 4i + q: word q of slot i) and the 16
  // runs, 8 bytes per lane clamped into the run (runs are padded to 4 values;
  // an empty run reads the 8 bytes at its start, which the allocation's slack
  // covers).  Slots past the wave's last
  // entry repeat that entry, so the loads of a batch past the end hit in
  // cache and need no branch.
  auto fetch = [&](int g, CrBatchRegs& B) {
    const int e0 = g * kCrBatch;
    const u32x2 pb = s_p[wave + kCrWaves * min(e0 + (lane & 15), nw - 1)];
    const uint32_t cb = s_col[wave + kCrWaves * min(e0 + (lane >> 2), nw - 1)];
    const uint64_t bv = a.bits[(ebase + 4 * uint64_t(cb)) * 4 + uint64_t(lane & 3)];
    B.bits_lo = uint32_t(bv);
    B.bits_hi = uint32_t(bv >> 32);
#pragma unroll
    for (int i = 0; i < kCrBatch; ++i) {
      const uint32_t p0 = __builtin_amdgcn_readlane(pb[0], i);
      const uint32_t p1 = __builtin_amdgcn_readlane(pb[1], i);
      const uint32_t last = p1 > p0 ? p1 - 4u : p0;
      const uint32_t off = min(p0 + 4u * uint32_t(lane), last);
      B.run[i] = *reinterpret_cast<const u32x2*>(a.vals + off);
    }
  };
  // Decode of batch g, in groups of kCrSlots slots (entry 16 g + i for slot
  // i; a group is skipped when its first entry does not exist, later slots
  // past the end decode with zero activations).  The group's runs go to the
  // wave's LDS slots; per slot and 64-row word q, v_readlane moves the word to
  // SGPRs, v_mbcnt ranks the lane among the set bits, a halfword read fetches
  // the value (all 16 reads of a group are in flight together) and the FMAs
  // run with exec narrowed to the word.
  auto decode = [&](int g, const CrBatchRegs& B) {
#pragma unroll
    for (int i0 = 0; i0 < kCrBatch; i0 += kCrSlots) {
      if (g * kCrBatch + i0 >= nw) break;  // uniform
#pragma unroll
      for (int u = 0; u < kCrSlots; ++u)
        *reinterpret_cast<lds_u32x2*>(static_cast<uintptr_t>(slots + uint32_t(u) * 512u + 8u * uint32_t(lane))) =
            B.run[i0 + u];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      uint64_t w[kCrSlots][4];
      _Float16 d[kCrSlots][4];  // high halves of the registers are not used
      float xs[kCrSlots][kN];
#pragma unroll
      for (int u = 0; u < kCrSlots; ++u) {
        const int e = g * kCrBatch + i0 + u;
        const int j = wave + kCrWaves * min(e, nw - 1);
#pragma unroll
        for (int t = 0; t < kN; ++t) xs[u][t] = e < nw ? s_x[j][t] : 0.f;
        // byte address of word q's first value (uniform: scalar arithmetic)
        uint32_t base = slots + uint32_t(u) * 512u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = __builtin_amdgcn_readlane(B.bits_lo, 4 * (i0 + u) + q);
          const uint32_t hi = __builtin_amdgcn_readlane(B.bits_hi, 4 * (i0 + u) + q);
          w[u][q] = uint64_t(lo) | (uint64_t(hi) << 32);
          const uint32_t rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
          d[u][q] = __builtin_bit_cast(_Float16, *reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(base + 2u * rank)));
          base += 2u * uint32_t(__builtin_popcountll(w[u][q]));
          asm("" : "+s"(base));  // keeps base scalar: one v_lshl_add per word
        }
      }
#pragma unroll
      for (int u = 0; u < kCrSlots; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) fma_masked<kN>(acc[q], d[u][q], xs[u], w[u][q]);
    }
  };
  if (nw > 0) {
    const int G = (nw + kCrBatch - 1) / kCrBatch;
    CrBatchRegs A, B;
    fetch(0, A);
    for (int g = 0;; g += 2) {
      fetch(g + 1, B);
      decode(g, A);
      if (g + 1 >= G) break;
      fetch(g + 2, A);
      decode(g + 1, B);
      if (g + 2 >= G) break;
    }
  }

  // ---- 3. workgroup partial (wave sums in wave order)
  __syncthreads();  // every wave is done with its run slots
  float* red = reinterpret_cast<float*>(s_run);  // [wave][token][256 rows]
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int t = 0; t < kN; ++t) red[(wave * kN + t) * 256 + q * 64 + lane] = acc[q][t];
  __syncthreads();
  const int t = tid >> 8, r = tid & 255;  // thread tid < 256 kN: token t, row r of the block
  if (t < kN) {
    float v = red[t * 256 + r];
#pragma unroll
    for (int w = 1; w < kCrWaves; ++w) v += red[(w * kN + t) * 256 + r];
    a.partials[((size_t(b) * a.S + s) * 4 + t) * 256 + r] = v;
  }
}

// Sum of the S partials of one row block and token (workgroup (b, t), one
// row per thread), in split order with up to 16 loads in flight, rounded once
// to fp16.
__global__ __launch_bounds__(256) void spmspv_cr_reduce(CrArgs a) {
  const int b = int(blockIdx.x), t = int(blockIdx.y), r = int(threadIdx.x);
  const float* pp = a.partials + (size_t(b) * a.S * 4 + t) * 256 + r;
  float sum = 0.f;
  for (int s0 = 0; s0 < a.S; s0 += 16) {
    float u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = s0 + i < a.S ? pp[size_t(s0 + i) * 4 * 256] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += u[i];
  }
  const int m = b * 256 + r;
  if (m < a.M) a.y[int64_t(t) * a.ldy + m] = __builtin_bit_cast(uint16_t, _Float16(sum));
}

// Partial sums of swm_spmspv_noalloc: a fixed device array in this code
// object (each GPU that loads the library holds its own copy until the
// process ends).  Host code never passes the array's name to a kernel: in
// host code that name is a host-side stand-in, not a device address.  The
// device address comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kScratchFloats = size_t(1) << 20;  // 4 MiB
static __device__ __attribute__((aligned(256))) float scratch[kScratchFloats];

}  // namespace

hipError_t spmspv_scratch(float** out, size_t* floats) {
  static std::mutex mu;
  static std::vector<float*> ptrs;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  if (dev >= int(ptrs.size())) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = static_cast<float*>(p);
  }
  *out = ptrs[dev];
  *floats = kScratchFloats;
  return hipSuccess;
}

size_t colruns_partial_floats(const ColRunsPlan& p) { return size_t(p.mb) * size_t(p.splits) * 4 * 256; }

ColRunsPlan plan_colruns(int64_t M, int64_t K) {
  // about one workgroup per CU (256), at most kCrMaxCols columns each
  ColRunsPlan p;
  p.mb = int((M + 255) / 256);
  const int64_t want = std::max<int64_t>((256 + p.mb - 1) / p.mb, (K + kCrMaxCols - 1) / kCrMaxCols);
  int64_t cps = (K + want - 1) / want;
  if (cps < 1) cps = 1;
  p.cps = int(cps);
  p.splits = int((K + cps - 1) / cps);
  return p;
}

hipError_t launch_spmspv_cr(const DevColRuns& c, const uint16_t* x, int64_t ldx, uint16_t* y, int64_t ldy,
                            int n, float tau, hipStream_t s) {
  if (n < 1 || n > 4 || c.plan.cps > kCrMaxCols) return hipErrorInvalidValue;
  CrArgs a;
  a.ptr = c.ptr;
  a.bits = c.bits;
  a.vals = c.vals;
  a.x = x;
  a.y = y;
  a.partials = c.partials;
  a.ldx = ldx;
  a.ldy = ldy;
  a.tau = tau;
  a.M = int(c.m);
  a.K = int(c.k);
  a.n = n;
  a.mb = c.plan.mb;
  a.S = c.plan.splits;
  a.cps = c.plan.cps;
  if (a.mb == 0 || a.S == 0) return hipSuccess;
  const unsigned items = unsigned((a.mb + 3) / 4) * unsigned(a.S);  // (split, group) pairs
  const dim3 grid(32u * ((items + 7u) / 8u)), block(64 * kCrWaves);
  switch (n) {
    case 1: hipLaunchKernelGGL(spmspv_cr_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(spmspv_cr_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(spmspv_cr_kernel<3>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(spmspv_cr_kernel<4>, grid, block, 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spmspv_cr_reduce, dim3(unsigned(a.mb), unsigned(n)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace swm
