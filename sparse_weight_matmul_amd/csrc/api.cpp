// C ABI of the sparse-weight matmul library: handle management, argument
// checks, dispatch by token count, error mapping.  No entry point aborts or
// throws across the boundary; nothing is printed unless SWM_LOG=1, which
// writes one line per dispatch decision to stderr.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "kernels.h"
#include "swm.h"
#include "swm_internal.h"

struct swm_format {
  swm::Header h;
  std::vector<uint8_t> blob;  // host copy of the export blob
  int device = 0;
  void* dev_mem = nullptr;     // one allocation for every device section
  swm::DevFormat d;
  swm::DecodePlan plan;       // decode split for N <= 4
  swm::DecodePlan plan8;      // 4 < N <= 8
  swm::DecodePlan plan_wide;  // 8 < N <= 16
  swm::DecodePlan plan_pair;  // 16 < N <= 32 (two token groups, looped kernel)
  void* cr_mem = nullptr;  // column-run encoding for activation skipping (optional)
  swm::DevColRuns cr;
  bool res24 = true;       // some row keeps 3 or 4 of an aligned group of 4 columns
  void* smf_mem = nullptr; // SWM_CFG_SMFMAC: the 2:4 layers (and residual layer), compacted once
  swm::Sparse24Layout smf_layout;
};

namespace {

std::atomic<int32_t> g_last_hip{0};

// SWM_LOG=1 (read once): one stderr line per dispatch decision.
bool log_on() {
  static const bool v = [] {
    const char* e = getenv("SWM_LOG");
    return e && *e == '1';
  }();
  return v;
}

__attribute__((format(printf, 1, 2))) void swm_log(const char* fmt, ...) {
  if (!log_on()) return;
  char line[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof(line), fmt, ap);
  va_end(ap);
  fprintf(stderr, "[swm] %s\n", line);
}

// SWM_SKIP (read once): "off" never takes the column-run kernel, "on" takes
// it for every token count it serves (n <= 4), anything else (default) up to
// the measured break-even token count.  An ablation switch: the result
// changes only in fp32 summation order.
int skip_mode() {
  static const int v = [] {
    const char* e = getenv("SWM_SKIP");
    if (e && !strcmp(e, "off")) return 0;
    if (e && !strcmp(e, "on")) return 2;
    return 1;
  }();
  return v;
}

swm_status hip_fail(hipError_t e) {
  g_last_hip.store(int32_t(e));
  return SWM_ERR_HIP;
}

#define SWM_HIP(expr)                              \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hip_fail(e_);     \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int num_cus(int dev) {
  static std::mutex mu;
  static std::vector<int> cache;
  std::lock_guard<std::mutex> g(mu);
  if (dev >= int(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

swm_status upload(std::vector<uint8_t>&& blob, const swm::Header& h, hipStream_t s, swm_format** out) {
  swm_format* f = new (std::nothrow) swm_format;
  if (!f) return SWM_ERR_OOM;
  f->h = h;
  f->blob = std::move(blob);
  if (hipGetDevice(&f->device) != hipSuccess) {
    delete f;
    return hip_fail(hipErrorNoDevice);
  }
  // Decode splits, one per size of the activation rows a wave stages (4, 8
  // or 16 tokens): the split with the most waves resident per CU.  The
  // looped kernel's split (17-32 tokens) targets about 32 waves per CU.
  const uint32_t* tp = reinterpret_cast<const uint32_t*>(f->blob.data() + h.off_tile_ptr());
  f->plan = swm::plan_decode(h, tp, num_cus(f->device), 64, true, 1);
  f->plan8 = swm::plan_decode(h, tp, num_cus(f->device), 32, true, 2);
  f->plan_wide = swm::plan_decode(h, tp, num_cus(f->device), 32, true, 4);
  f->plan_pair = swm::plan_decode(h, tp, num_cus(f->device), 32, false);
  f->res24 = swm::mask_exceeds_2_of_4(h, f->blob.data());
  const size_t T = h.tiles();
  const size_t b_tp = 4 * (T + 1), b_bits = 8 * h.n_bits(), b_vals = 2 * h.padded_len + 1024;
  const size_t n_zero = size_t(h.kt) * h.tk + 64;
  size_t off = 0;
  const size_t o_tp = off;
  off = align_up(off + b_tp, 256);
  const size_t o_bits = off;
  off = align_up(off + b_bits, 256);
  const size_t o_vals = off;
  off = align_up(off + b_vals, 256);
  const size_t o_zero = off;
  off = align_up(off + 2 * n_zero, 256);
  if (hipMalloc(&f->dev_mem, off) != hipSuccess) {
    delete f;
    return SWM_ERR_OOM;
  }
  uint8_t* base = static_cast<uint8_t*>(f->dev_mem);
  const uint8_t* hb = f->blob.data();
  hipError_t e = hipMemsetAsync(base, 0, off, s);
  if (e == hipSuccess && b_tp) e = hipMemcpyAsync(base + o_tp, hb + h.off_tile_ptr(), b_tp, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && b_bits) e = hipMemcpyAsync(base + o_bits, hb + h.off_bits(), b_bits, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && h.padded_len)
    e = hipMemcpyAsync(base + o_vals, hb + h.off_values(), 2 * h.padded_len, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(f->dev_mem);
    delete f;
    return hip_fail(e);
  }
  f->d.h = h;
  f->d.tile_ptr = reinterpret_cast<const uint32_t*>(base + o_tp);
  f->d.bits = reinterpret_cast<const uint64_t*>(base + o_bits);
  f->d.vals = reinterpret_cast<const uint16_t*>(base + o_vals);
  f->d.zeros = reinterpret_cast<const uint16_t*>(base + o_zero);
  *out = f;
  return SWM_OK;
}

swm_status check_tile_supported(const swm::Header& h) {
  if (h.tm != 16 || h.tk != 64) return SWM_ERR_UNSUPPORTED;
  if (h.m > (int64_t(1) << 31) - 64 || h.k > (int64_t(1) << 31) - 64) return SWM_ERR_UNSUPPORTED;
  return SWM_OK;
}

bool on_current_device(const swm_format* f) {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == f->device;
}

}  // namespace

extern "C" {

const char* swm_status_str(swm_status s) {
  switch (s) {
    case SWM_OK: return "ok";
    case SWM_ERR_INVALID_ARG: return "invalid argument";
    case SWM_ERR_SHAPE: return "shape mismatch";
    case SWM_ERR_ALIGN: return "alignment";
    case SWM_ERR_OOM: return "out of memory";
    case SWM_ERR_OVERFLOW: return "size overflow";
    case SWM_ERR_FORMAT: return "invalid format";
    case SWM_ERR_HIP: return "HIP runtime error";
    case SWM_ERR_UNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

int32_t swm_last_hip_error(void) { return g_last_hip.load(); }

int32_t swm_version(void) { return 200; }  // 0.2.0: the gated steps at prefill sizes

swm_status swm_encode_blob(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm,
                           int64_t M, int64_t K, const swm_tile_cfg* cfg, void* buf, size_t cap,
                           size_t* size) {
  if (!size) return SWM_ERR_INVALID_ARG;
  std::vector<uint8_t> blob;
  swm_status st = swm::encode_blob(W, ldw, mask, ldm, M, K, cfg, &blob);
  if (st != SWM_OK) return st;
  *size = blob.size();
  if (!buf) return SWM_OK;
  if (cap < blob.size()) return SWM_ERR_INVALID_ARG;
  std::memcpy(buf, blob.data(), blob.size());
  return SWM_OK;
}

swm_status swm_sparse_compress(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm,
                               int64_t M, int64_t K, const swm_tile_cfg* cfg, void* stream,
                               swm_format** out) {
  if (!out) return SWM_ERR_INVALID_ARG;
  if (cfg && (cfg->flags & ~int32_t(SWM_CFG_SKIPPING | SWM_CFG_SMFMAC))) return SWM_ERR_INVALID_ARG;
  std::vector<uint8_t> blob;
  swm_status st = swm::encode_blob(W, ldw, mask, ldm, M, K, cfg, &blob);
  if (st != SWM_OK) return st;
  swm::Header h;
  st = swm::read_header(blob.data(), blob.size(), &h);
  if (st != SWM_OK) return st;
  swm_format* f = nullptr;
  st = upload(std::move(blob), h, static_cast<hipStream_t>(stream), &f);
  if (st != SWM_OK) return st;
  if (cfg && (cfg->flags & SWM_CFG_SMFMAC)) {
    st = swm_format_enable_smfmac(f, stream, nullptr);
    if (st != SWM_OK) {
      (void)swm_format_destroy(f);
      return st;
    }
  }
  swm_log("sparse_compress M=%lld K=%lld nnz=%llu blob=%zu B flags=%d: decode split %d / %d / %d tiles per wave "
          "(N <= 4 / <= 8 / <= 16%s), %s",
          (long long)h.m, (long long)h.k, (unsigned long long)h.nnz, f->blob.size(), cfg ? cfg->flags : 0,
          f->plan.tiles_per_wave, f->plan8.tiles_per_wave, f->plan_wide.tiles_per_wave,
          f->plan_wide.direct_b ? ", B operands from memory" : "",
          f->res24 ? "mask exceeds 2:4 (SMFMAC needs a residual layer)" : "mask within 2:4");

  if (cfg && (cfg->flags & SWM_CFG_SKIPPING)) {
    st = swm_format_enable_skipping(f, stream, nullptr);
    if (st != SWM_OK) {
      (void)swm_format_destroy(f);
      return st;
    }
  }
  *out = f;
  return SWM_OK;
}

swm_status swm_format_export(const swm_format* f, void* buf, size_t cap, size_t* size) {
  if (!f || !size) return SWM_ERR_INVALID_ARG;
  *size = f->blob.size();
  if (!buf) return SWM_OK;
  if (cap < f->blob.size()) return SWM_ERR_INVALID_ARG;
  std::memcpy(buf, f->blob.data(), f->blob.size());
  return SWM_OK;
}

swm_status swm_format_validate_blob(const void* buf, size_t size) {
  if (!buf) return SWM_ERR_INVALID_ARG;
  return swm::validate_blob(buf, size, nullptr);
}

swm_status swm_format_import(const void* buf, size_t size, void* stream, swm_format** out) {
  if (!buf || !out) return SWM_ERR_INVALID_ARG;
  swm::Header h;
  swm_status st = swm::validate_blob(buf, size, &h);
  if (st != SWM_OK) return st;
  std::vector<uint8_t> blob;
  try {
    blob.assign(static_cast<const uint8_t*>(buf), static_cast<const uint8_t*>(buf) + size);
  } catch (...) {
    return SWM_ERR_OOM;
  }
  return upload(std::move(blob), h, static_cast<hipStream_t>(stream), out);
}

swm_status swm_format_query(const swm_format* f, swm_format_info* info) {
  if (!f || !info) return SWM_ERR_INVALID_ARG;
  swm::fill_info(f->h, info);
  return SWM_OK;
}

swm_status swm_size_dry_run(int64_t M, int64_t K, uint64_t nnz, const swm_tile_cfg* cfg,
                            swm_format_info* info) {
  if (!info) return SWM_ERR_INVALID_ARG;
  swm::Header h;
  swm_status st = swm::plan_grid(M, K, cfg, &h);
  if (st != SWM_OK) return st;
  if (nnz > uint64_t(M) * uint64_t(K)) return SWM_ERR_INVALID_ARG;
  // Worst case: every tile pads by 7 values.
  const unsigned __int128 worst = (unsigned __int128)nnz + (unsigned __int128)h.tiles() * 7u;
  if (worst >= ((unsigned __int128)1 << 32)) return SWM_ERR_OVERFLOW;
  h.nnz = nnz;
  h.padded_len = uint64_t(worst);
  h.max_tile = uint32_t(std::min<uint64_t>(uint64_t(h.tm) * h.tk, h.padded_len));
  swm::fill_info(h, info);
  return SWM_OK;
}

swm_status swm_format_destroy(swm_format* f) {
  if (!f) return SWM_OK;
  swm_status st = SWM_OK;
  if (f->dev_mem || f->cr_mem || f->smf_mem) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    if (cur != f->device) (void)hipSetDevice(f->device);
    if (f->dev_mem) {
      hipError_t e = hipFree(f->dev_mem);
      if (e != hipSuccess) st = hip_fail(e);
    }
    if (f->smf_mem) {
      hipError_t e = hipFree(f->smf_mem);
      if (e != hipSuccess) st = hip_fail(e);
    }
    if (f->cr_mem) {
      hipError_t e = hipFree(f->cr_mem);
      if (e != hipSuccess) st = hip_fail(e);
    }
    if (cur != f->device) (void)hipSetDevice(cur);
  }
  delete f;
  return st;
}

swm_status swm_colruns_encode_blob(const void* tcb_blob, size_t size, void* out, size_t cap, size_t* size_out) {
  if (!tcb_blob || !size_out) return SWM_ERR_INVALID_ARG;
  swm::ColRunsHost c;
  swm_status st = swm::colruns_from_tcb(tcb_blob, size, &c);
  if (st != SWM_OK) return st;
  const size_t need = swm::colruns_blob_bytes(c);
  *size_out = need;
  if (!out) return SWM_OK;
  if (cap < need) return SWM_ERR_INVALID_ARG;
  swm::colruns_write_blob(c, static_cast<uint8_t*>(out));
  return SWM_OK;
}

swm_status swm_format_enable_smfmac(swm_format* f, void* stream, uint64_t* bytes) {
  if (!f) return SWM_ERR_INVALID_ARG;
  if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
  if (f->h.tm != 16 || f->h.tk != 64) return SWM_ERR_UNSUPPORTED;
  if (!f->smf_mem && f->h.m > 0) {
    // compact once into the sparse-matrix-core layers; they stay with the handle
    const swm::Sparse24Layout L = swm::sparse24_layout(f->h, f->res24);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* mem = nullptr;
    if (hipMalloc(&mem, L.bytes) != hipSuccess) return SWM_ERR_OOM;
    hipError_t e = swm::launch_compact24(f->d, L, f->res24, mem, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      (void)hipFree(mem);
      return hip_fail(e);
    }
    f->smf_layout = L;
    f->smf_mem = mem;
    swm_log("enable_smfmac M=%lld K=%lld: 2:4 layers resident, %zu B (%s)", (long long)f->h.m, (long long)f->h.k,
            L.bytes, f->res24 ? "2:4 layer + residual layer" : "2:4 layer only");
  }
  if (bytes) *bytes = f->smf_mem ? f->smf_layout.bytes : 0;
  return SWM_OK;
}

swm_status swm_format_enable_skipping(swm_format* f, void* stream, uint64_t* bytes) {
  if (!f) return SWM_ERR_INVALID_ARG;
  if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
  if (f->cr_mem) {
    if (bytes) *bytes = f->cr.bytes;
    return SWM_OK;
  }
  if (f->h.m > (int64_t(1) << 31) - 256 || f->h.k > (int64_t(1) << 31) - 64) return SWM_ERR_UNSUPPORTED;
  swm::ColRunsHost c;
  swm_status st = swm::colruns_from_tcb(f->blob.data(), f->blob.size(), &c);
  if (st != SWM_OK) return st;
  const swm::ColRunsPlan plan = swm::plan_colruns(c.m, c.k);
  const uint64_t E = c.entries();
  const size_t b_ptr = 4 * (E + 1), b_bits = 32 * E, b_vals = 2 * c.values.size() + 16;
  const size_t b_part = 4 * size_t(plan.mb) * size_t(plan.splits) * 4 * 256;
  size_t off = 0;
  const size_t o_ptr = off;
  off = align_up(off + b_ptr, 256);
  const size_t o_bits = off;
  off = align_up(off + b_bits, 256);
  const size_t o_vals = off;
  off = align_up(off + b_vals, 256);
  const size_t o_part = off;
  off = align_up(off + b_part, 256);
  void* mem = nullptr;
  if (hipMalloc(&mem, off) != hipSuccess) return SWM_ERR_OOM;
  uint8_t* base = static_cast<uint8_t*>(mem);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemsetAsync(base, 0, off, s);
  if (e == hipSuccess) e = hipMemcpyAsync(base + o_ptr, c.ptr.data(), b_ptr, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && E) e = hipMemcpyAsync(base + o_bits, c.bits.data(), b_bits, hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !c.values.empty())
    e = hipMemcpyAsync(base + o_vals, c.values.data(), 2 * c.values.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(mem);
    return hip_fail(e);
  }
  f->cr.m = c.m;
  f->cr.k = c.k;
  f->cr.ptr = reinterpret_cast<const uint32_t*>(base + o_ptr);
  f->cr.bits = reinterpret_cast<const uint64_t*>(base + o_bits);
  f->cr.vals = reinterpret_cast<const uint16_t*>(base + o_vals);
  f->cr.partials = reinterpret_cast<float*>(base + o_part);
  f->cr.plan = plan;
  f->cr.bytes = b_ptr + b_bits + 2 * c.values.size();
  f->cr_mem = mem;
  if (bytes) *bytes = f->cr.bytes;
  return SWM_OK;
}

swm_status swm_decompress(const swm_format* f, void* W_dev, int64_t ldw, void* stream) {
  if (!f || !W_dev) return SWM_ERR_INVALID_ARG;
  if (ldw < f->h.k) return SWM_ERR_INVALID_ARG;
  swm_status st = check_tile_supported(f->h);
  if (st != SWM_OK) return st;
  if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
  SWM_HIP(swm::launch_decompress(f->d, static_cast<uint16_t*>(W_dev), ldw, static_cast<hipStream_t>(stream)));
  return SWM_OK;
}

static const swm::DecodePlan& decode_plan(const swm_format* f, int64_t n) {
  return n <= 4 ? f->plan : n <= 8 ? f->plan8 : n <= 16 ? f->plan_wide : f->plan_pair;
}

static bool run_smf(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t N,
                    hipStream_t s, swm_status* st);

static swm_status run_products(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy,
                               int64_t N, bool skip, hipStream_t s) {
  if (!f || !X || !Y) return SWM_ERR_INVALID_ARG;
  if (N <= 0 || ldx < f->h.k || ldy < f->h.m || ldx <= 0 || ldy <= 0) return SWM_ERR_INVALID_ARG;
  swm_status st = check_tile_supported(f->h);
  if (st != SWM_OK) return st;
  if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint16_t* y = static_cast<uint16_t*>(Y);
  // N <= 32 is memory bound (the weights are read once per call): the decode
  // kernels, with one or two 16-token groups per decoded operand.
  if (N <= 16 || (N <= 32 && !skip)) {
    const swm::DecodePlan& p = decode_plan(f, N);
    swm_log("%s M=%lld K=%lld N=%lld: decode (%s, %d tiles x %d waves per slab)", skip ? "spmspv" : "spmm",
            (long long)f->h.m, (long long)f->h.k, (long long)N, p.seq_segs > 0 && N <= 16 ? "straight-line" : "looped",
            p.tiles_per_wave, p.waves);
    SWM_HIP(swm::launch_decode(f->d, p, x, ldx, y, ldy, int(N), skip, s));
    return SWM_OK;
  }
  swm_status sst = SWM_OK;
  if (!skip && run_smf(f, X, ldx, Y, ldy, N, s, &sst)) return sst;
  if (!skip && swm::prefill_supported(f->h.k, ldx, X) && swm::prefill_sparse_lds(f->h) <= 160 * 1024 &&
      swm::prefill_sparse_fits(f->h, N, ldx)) {
    swm_log("spmm M=%lld K=%lld N=%lld: on-chip prefill (128x256 blocks)", (long long)f->h.m, (long long)f->h.k,
            (long long)N);
    SWM_HIP(swm::launch_prefill_sparse(f->d, x, ldx, y, ldy, N, s));
    return SWM_OK;
  }
  swm_log("%s M=%lld K=%lld N=%lld: decode in %d-token slices", skip ? "spmspv" : "spmm", (long long)f->h.m,
          (long long)f->h.k, (long long)N, skip ? 16 : 32);
  // Otherwise: token slices through the decode kernel (32 at a time; 16 when
  // skipping, whose decode kernel serves one group of 16).
  const int64_t slice = skip ? 16 : 32;
  for (int64_t n0 = 0; n0 < N; n0 += slice) {
    const int nn = int(std::min<int64_t>(slice, N - n0));
    SWM_HIP(swm::launch_decode(f->d, decode_plan(f, nn), x + n0 * ldx, ldx, y + n0 * ldy, ldy, nn, skip, s));
  }
  return SWM_OK;
}

swm_status swm_spmm(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy,
                    int64_t N, void* stream) {
  return run_products(f, X, ldx, Y, ldy, N, false, static_cast<hipStream_t>(stream));
}

// When swm_spmm_ws expands W once into the workspace and runs the dense MFMA
// kernel instead of the on-chip prefill kernel (128 x 256 blocks): from 1024
// tokens, and from 256 tokens when the on-chip kernel's blocks would leave
// at least half of the CUs idle or spill into a second round, where the
// dense kernel's block choice fits the chip better (measured at N = 256-1024:
// q_proj 4096x4096 71 against 80 us, down 4096x11008 168 against 200 us,
// up 11008x4096 at N = 640 107 against 162 us).  SWM_EXPAND_MIN_N replaces
// the rule by a plain token threshold (read once per process; at least 33:
// from there swm_spmm's own prefill kernel sums each output in the same
// order as the dense kernel, so the route does not change the bits of a
// result).
static int64_t expand_min_n() {
  static const int64_t v = [] {
    const char* e = getenv("SWM_EXPAND_MIN_N");
    const long long n = e ? atoll(e) : 0;
    return n > 0 ? std::max<int64_t>(int64_t(n), 33) : int64_t(0);
  }();
  return v;
}

static bool expand_route(const swm::Header& h, int64_t N) {
  if (!(h.k >= 8 && h.k % 8 == 0 && h.m > 0)) return false;
  if (expand_min_n() > 0) return N >= expand_min_n();
  if (N >= 1024) return true;
  if (N < 256) return false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const int64_t cus = num_cus(dev);
  const int64_t blocks = ((h.m + 127) / 128) * ((N + 255) / 256);
  return 2 * blocks <= cus || blocks > cus;
}

// The sparse-matrix-core route: for handles compressed with SWM_CFG_SMFMAC,
// whose 2:4 layer (plus a residual layer where the mask needs one) was
// compacted once at compress time, swm_spmm and swm_spmm_ws multiply with
// v_smfmac where the expansion route would run (same token counts), with no
// workspace.  SWM_SMFMAC = 0 turns it off (read once).  It is opt-in because
// it needs the layers resident beside the tiled format and only pays with a
// 2:4 mask at full block occupancy (q_proj 4096x4096 at N = 4096); a residual
// layer doubles its matrix instructions.
static int smfmac_mode() {
  static const int v = [] {
    const char* e = getenv("SWM_SMFMAC");
    return e ? atoi(e) : -1;
  }();
  return v;
}

static bool smf_route(const swm_format* f, int64_t N) {
  if (!f->smf_mem || f->h.tm != 16 || f->h.tk != 64 || smfmac_mode() == 0) return false;
  return expand_route(f->h, N);
}

// The cached layers through v_smfmac; false when the operands do not fit the
// kernel's 32-bit offsets or alignment (then the caller takes another route).
static bool run_smf(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t N,
                    hipStream_t s, swm_status* st) {
  if (!smf_route(f, N) || !swm::prefill_supported(f->h.k, ldx, X) || !swm::smf_fits(f->h, N, ldx)) return false;
  swm_log("spmm M=%lld K=%lld N=%lld: resident 2:4 layers + SMFMAC (%s)", (long long)f->h.m, (long long)f->h.k,
          (long long)N, f->res24 ? "with residual layer" : "no residual");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = swm::launch_smf(f->h, f->smf_layout, f->res24, f->smf_mem, static_cast<const uint16_t*>(X), ldx,
                        static_cast<uint16_t*>(Y), ldy, N, num_cus(dev), s);
  *st = e == hipSuccess ? SWM_OK : hip_fail(e);
  return true;
}

size_t swm_spmm_workspace_bytes(const swm_format* f, int64_t N) {
  if (!f || !expand_route(f->h, N) || smf_route(f, N)) return 0;
  return align_up(size_t(f->h.m) * size_t(f->h.k) * 2, 256);
}

swm_status swm_spmm_ws(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t N,
                       void* workspace, size_t ws_bytes, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!f || !X || !Y) return SWM_ERR_INVALID_ARG;
  if (!workspace && ws_bytes == 0) return run_products(f, X, ldx, Y, ldy, N, false, s);
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return SWM_ERR_ALIGN;
  if (!workspace) return SWM_ERR_INVALID_ARG;
  const size_t need = swm_spmm_workspace_bytes(f, N);
  if (need == 0 || !swm::prefill_supported(f->h.k, ldx, X)) return run_products(f, X, ldx, Y, ldy, N, false, s);
  if (ws_bytes < need) return SWM_ERR_INVALID_ARG;
  if (N <= 0 || ldx < f->h.k || ldy < f->h.m) return SWM_ERR_INVALID_ARG;
  swm_status st = check_tile_supported(f->h);
  if (st != SWM_OK) return st;
  if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
  swm_log("spmm_ws M=%lld K=%lld N=%lld: expand into the workspace + dense MFMA", (long long)f->h.m,
          (long long)f->h.k, (long long)N);
  uint16_t* w = static_cast<uint16_t*>(workspace);
  SWM_HIP(swm::launch_decompress(f->d, w, f->h.k, s));
  int dev = 0;
  SWM_HIP(hipGetDevice(&dev));
  SWM_HIP(swm::launch_prefill_dense(w, f->h.k, static_cast<const uint16_t*>(X), ldx, static_cast<uint16_t*>(Y),
                                    ldy, f->h.m, f->h.k, N, num_cus(dev), s));
  return SWM_OK;
}

static swm_status run_colruns(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy, int32_t n,
                              float tau, void* stream) {
  if (!x || !y || ldx < f->h.k || ldy < f->h.m || ldx <= 0 || ldy <= 0) return SWM_ERR_INVALID_ARG;
  if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
  SWM_HIP(swm::launch_spmspv_cr(f->cr, static_cast<const uint16_t*>(x), ldx, static_cast<uint16_t*>(y), ldy, n, tau,
                                static_cast<hipStream_t>(stream)));
  return SWM_OK;
}

// Tokens up to which swm_spmspv takes the skipping kernel when the handle
// carries the column-run encoding.  Measured on down_proj 4096x11008 at 50%
// with SiLU-gated activations: at n = 1 it pays from about 65% inactive
// columns, at n = 2-4 from about 74%; the columns inactive in all of n tokens
// shrink like a power of n, and at n = 4 the column-run decode (five vector
// instructions plus one per token per 64-row word) is issue bound, so three
// or more tokens run the full product.
constexpr int32_t kSkipMaxTokens = 2;

// Whether swm_spmspv takes the column-run kernel (SWM_SKIP can force either way).
static bool skip_route(const swm_format* f, int32_t n) {
  const int mode = skip_mode();
  const bool r = f && f->cr_mem && mode > 0 && n <= (mode == 2 ? 4 : kSkipMaxTokens);
  if (f && r)
    swm_log("spmspv M=%lld K=%lld n=%d: column-run skipping kernel + reduce", (long long)f->h.m, (long long)f->h.k, n);
  return r;
}

swm_status swm_spmspv(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy,
                      int32_t n, void* stream) {
  if (n < 1 || n > 16) return SWM_ERR_INVALID_ARG;
  if (skip_route(f, n)) return run_colruns(f, x, ldx, y, ldy, n, 0.f, stream);
  return run_products(f, x, ldx, y, ldy, n, true, static_cast<hipStream_t>(stream));
}

swm_status swm_spmspv_noalloc(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy,
                              int32_t n, void* stream) {
  if (n < 1 || n > 16) return SWM_ERR_INVALID_ARG;
  if (skip_route(f, n)) {
    float* scr = nullptr;
    size_t cap = 0;
    SWM_HIP(swm::spmspv_scratch(&scr, &cap));
    if (swm::colruns_partial_floats(f->cr.plan) > cap) return SWM_ERR_UNSUPPORTED;
    if (!x || !y || ldx < f->h.k || ldy < f->h.m || ldx <= 0 || ldy <= 0) return SWM_ERR_INVALID_ARG;
    if (!on_current_device(f)) return SWM_ERR_INVALID_ARG;
    swm::DevColRuns c = f->cr;
    c.partials = scr;
    SWM_HIP(swm::launch_spmspv_cr(c, static_cast<const uint16_t*>(x), ldx, static_cast<uint16_t*>(y), ldy, n, 0.f,
                                  static_cast<hipStream_t>(stream)));
    return SWM_OK;
  }
  return run_products(f, x, ldx, y, ldy, n, true, static_cast<hipStream_t>(stream));
}

swm_status swm_spmspv_threshold(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy,
                                int32_t n, float tau, void* stream) {
  if (!f || n < 1 || n > 16 || !(tau >= 0.f) || !(tau <= 65504.f)) return SWM_ERR_INVALID_ARG;
  if (!f->cr_mem || n > 4) return SWM_ERR_UNSUPPORTED;
  return run_colruns(f, x, ldx, y, ldy, n, tau, stream);
}

swm_status swm_gate_up_silu(const swm_format* g, const swm_format* u, const void* X, int64_t ldx, void* H,
                            int64_t ldh, int32_t n, float tau, void* stream) {
  if (!g || !u || !X || !H) return SWM_ERR_INVALID_ARG;
  if (n < 1 || n > 32 || !(tau >= 0.f) || !(tau <= 65504.f)) return SWM_ERR_INVALID_ARG;
  if (g->h.m != u->h.m || g->h.k != u->h.k) return SWM_ERR_INVALID_ARG;
  if (ldx < g->h.k || ldh < g->h.m || ldx <= 0 || ldh <= 0) return SWM_ERR_INVALID_ARG;
  swm_status st = check_tile_supported(g->h);
  if (st == SWM_OK) st = check_tile_supported(u->h);
  if (st != SWM_OK) return st;
  if (!on_current_device(g) || !on_current_device(u)) return SWM_ERR_INVALID_ARG;
  if (g->h.k < 8 || g->h.k % 8 != 0) return SWM_ERR_UNSUPPORTED;
  if (ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15) != 0) return SWM_ERR_ALIGN;
  if (2 * ((int64_t(n) - 1) * ldx + g->h.k) >= (int64_t(1) << 32)) return SWM_ERR_UNSUPPORTED;
  int dev = 0;
  SWM_HIP(hipGetDevice(&dev));
  // Up to 16 tokens per launch (the straight-line kernel stages at most 16
  // activation rows per wave); 17-32 tokens take two launches.
  const int n0 = std::min(n, 16);
  const swm::DecodePlan p0 = swm::plan_decode_glu(g->h, u->h, num_cus(dev), n0);
  const swm::DecodePlan p1 = swm::plan_decode_glu(g->h, u->h, num_cus(dev), std::max(n - 16, 1));
  if (p0.seq_segs == 0 || p1.seq_segs == 0) return SWM_ERR_UNSUPPORTED;
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint16_t* h = static_cast<uint16_t*>(H);
  hipStream_t s = static_cast<hipStream_t>(stream);
  swm_log("gate_up_silu M=%lld K=%lld n=%d: one gated decode launch per 16 tokens (%d tiles per wave)",
          (long long)g->h.m, (long long)g->h.k, n, p0.tiles_per_wave);
  SWM_HIP(swm::launch_decode_glu(g->d, u->d, p0, x, ldx, h, ldh, n0, tau, s));
  if (n > 16) SWM_HIP(swm::launch_decode_glu(g->d, u->d, p1, x + 16 * ldx, ldx, h + 16 * ldh, ldh, n - 16, tau, s));
  return SWM_OK;
}

// Prefill sizes of the gated FFN step: from this token count the gate and up
// weights are expanded into the workspace and multiplied by the dense MFMA
// kernel with the gated epilogue; below it, swm_gate_up_silu's decode
// launches.
constexpr int64_t kGluExpandMinN = 33;

size_t swm_gate_up_silu_workspace_bytes(const swm_format* g, const swm_format* u, int64_t n) {
  if (!g || !u || n < kGluExpandMinN || g->h.m != u->h.m || g->h.k != u->h.k) return 0;
  return align_up(size_t(2) * size_t(g->h.m) * size_t(g->h.k) * 2, 256);
}

swm_status swm_gate_up_silu_ws(const swm_format* g, const swm_format* u, const void* X, int64_t ldx, void* H,
                               int64_t ldh, int64_t n, float tau, void* workspace, size_t ws_bytes,
                               void* stream) {
  if (!g || !u || !X || !H) return SWM_ERR_INVALID_ARG;
  if (n < 1 || !(tau >= 0.f) || !(tau <= 65504.f)) return SWM_ERR_INVALID_ARG;
  if (n < kGluExpandMinN) return swm_gate_up_silu(g, u, X, ldx, H, ldh, int32_t(n), tau, stream);
  if (g->h.m != u->h.m || g->h.k != u->h.k) return SWM_ERR_INVALID_ARG;
  if (ldx < g->h.k || ldh < g->h.m || ldx <= 0 || ldh <= 0) return SWM_ERR_INVALID_ARG;
  if (g->h.m == 0) return SWM_OK;  // nothing to compute, no workspace needed
  if (!workspace || ws_bytes < swm_gate_up_silu_workspace_bytes(g, u, n)) return SWM_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return SWM_ERR_ALIGN;
  swm_status st = check_tile_supported(g->h);
  if (st == SWM_OK) st = check_tile_supported(u->h);
  if (st != SWM_OK) return st;
  if (!on_current_device(g) || !on_current_device(u)) return SWM_ERR_INVALID_ARG;
  if (g->h.k < 8 || g->h.k % 8 != 0) return SWM_ERR_UNSUPPORTED;
  if (ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15) != 0) return SWM_ERR_ALIGN;
  const int64_t M = int64_t(g->h.m), K = int64_t(g->h.k);
  if (2 * M > (int64_t(1) << 31) - 64 || !swm::prefill_dense_dma_fits(2 * M, K, K, n, ldx))
    return SWM_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  SWM_HIP(hipGetDevice(&dev));
  swm_log("gate_up_silu_ws M=%lld K=%lld n=%lld: gate and up expanded as interleaved rows + dense MFMA with the "
          "gated epilogue",
          (long long)M, (long long)K, (long long)n);
  // gate row m -> workspace row 2m, up row m -> row 2m + 1 (row stride K)
  uint16_t* w = static_cast<uint16_t*>(workspace);
  SWM_HIP(swm::launch_decompress(g->d, w, 2 * K, s));
  SWM_HIP(swm::launch_decompress(u->d, w + K, 2 * K, s));
  SWM_HIP(swm::launch_prefill_dense_glu(w, K, static_cast<const uint16_t*>(X), ldx, static_cast<uint16_t*>(H), ldh,
                                        2 * M, K, n, tau, num_cus(dev), s));
  return SWM_OK;
}

swm_status swm_dense_gate_up_silu(const void* W2, int64_t ldw, const void* X, int64_t ldx, void* H, int64_t ldh,
                                  int64_t M, int64_t K, int64_t N, float tau, void* stream) {
  if (!W2 || !X || !H) return SWM_ERR_INVALID_ARG;
  if (M < 0 || K < 0 || N <= 0 || ldw < K || ldx < K || ldh < M || ldw <= 0 || ldx <= 0 || ldh <= 0)
    return SWM_ERR_INVALID_ARG;
  if (!(tau >= 0.f) || !(tau <= 65504.f)) return SWM_ERR_INVALID_ARG;
  if (M == 0) return SWM_OK;
  if (K < 8 || K % 8 != 0) return SWM_ERR_UNSUPPORTED;
  if (ldx % 8 != 0 || ldw % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(W2) & 15) != 0)
    return SWM_ERR_ALIGN;
  if (2 * M > (int64_t(1) << 31) - 64 || !swm::prefill_dense_dma_fits(2 * M, ldw, K, N, ldx))
    return SWM_ERR_UNSUPPORTED;
  int dev = 0;
  SWM_HIP(hipGetDevice(&dev));
  swm_log("dense_gate_up_silu M=%lld K=%lld N=%lld: dense MFMA with the gated epilogue", (long long)M,
          (long long)K, (long long)N);
  SWM_HIP(swm::launch_prefill_dense_glu(static_cast<const uint16_t*>(W2), ldw, static_cast<const uint16_t*>(X), ldx,
                                        static_cast<uint16_t*>(H), ldh, 2 * M, K, N, tau, num_cus(dev),
                                        static_cast<hipStream_t>(stream)));
  return SWM_OK;
}

swm_status swm_hbm_stream(const void* buf, size_t bytes, int32_t unroll, int32_t blocks,
                          uint32_t* out, void* stream) {
  if (!buf || !out || bytes % 16 || blocks <= 0) return SWM_ERR_INVALID_ARG;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16) return SWM_ERR_INVALID_ARG;
  SWM_HIP(swm::launch_stream(buf, bytes, unroll, blocks, out, static_cast<hipStream_t>(stream)));
  return SWM_OK;
}

swm_status swm_dense_gemm(const void* W, int64_t ldw, const void* X, int64_t ldx, void* Y,
                          int64_t ldy, int64_t M, int64_t K, int64_t N, void* stream) {
  if (!W || !X || !Y) return SWM_ERR_INVALID_ARG;
  if (M < 0 || K < 0 || N <= 0 || ldw < K || ldx < K || ldy < M || ldw <= 0 || ldx <= 0 || ldy <= 0)
    return SWM_ERR_INVALID_ARG;
  if (M > (int64_t(1) << 31) - 64 || K > (int64_t(1) << 31) - 64) return SWM_ERR_UNSUPPORTED;
  if (M == 0) return SWM_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  SWM_HIP(hipGetDevice(&dev));
  // The MFMA-tiled kernel for N > 16, unless N <= 32 and its 256x256 output
  // blocks (at least one per 256 tokens) would occupy under a quarter of the
  // CUs: then two 16-token passes of the streaming kernel are faster (each
  // reads W once at full bandwidth).
  const int64_t tiled_blocks = ((M + 255) / 256) * ((N + 255) / 256);
  const bool small_tiled = N <= 32 && tiled_blocks * 4 < num_cus(dev);
  if (N > 16 && !small_tiled && swm::prefill_supported(K, ldx, X) && ldw % 8 == 0 &&
      (reinterpret_cast<uintptr_t>(W) & 15) == 0) {
    swm_log("dense_gemm M=%lld K=%lld N=%lld: MFMA tiled", (long long)M, (long long)K, (long long)N);
    SWM_HIP(swm::launch_prefill_dense(static_cast<const uint16_t*>(W), ldw, static_cast<const uint16_t*>(X),
                                      ldx, static_cast<uint16_t*>(Y), ldy, M, K, N, num_cus(dev), s));
    return SWM_OK;
  }
  const auto p = swm::plan_dense_small(M, K, int(std::min<int64_t>(N, 16)), num_cus(dev));
  swm_log("dense_gemm M=%lld K=%lld N=%lld: streaming, %d waves per slab, 16 tokens a pass", (long long)M,
          (long long)K, (long long)N, p.waves);
  const uint16_t* w = static_cast<const uint16_t*>(W);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint16_t* y = static_cast<uint16_t*>(Y);
  for (int64_t n0 = 0; n0 < N; n0 += 16) {
    const int nn = int(std::min<int64_t>(16, N - n0));
    SWM_HIP(swm::launch_dense_small(p, w, ldw, x + n0 * ldx, ldx, y + n0 * ldy, ldy, M, K, nn, s));
  }
  return SWM_OK;
}

}  // extern "C"
