/*
 * swm.h -- C ABI of the MI355X (gfx950) sparse-weight matmul library.
 *
 * The library multiplies a statically pruned fp16 weight matrix W (out x in,
 * M x K, moderate unstructured sparsity, stored compressed) by dense fp16
 * activations, in the decode regime (N = 1..16 tokens, bandwidth bound), with
 * optional skipping of input channels whose activation is zero, and in the
 * prefill regime (N in the hundreds to thousands, matrix-core bound).  A dense
 * GEMM of the same shapes is exported beside it as the honest baseline.
 *
 * Sources of the operations (the pages this library is built from):
 *  - "Unified Static-Dynamic Pruning for Efficient LLM Inference" (SPDP),
 *    abstract: unstructured static pruning stored in a tiled column-wise
 *    bitmap compressed format; a decode kernel that skips zero activations at
 *    run time (sparse matrix x sparse vector); a prefill SpMM on the matrix
 *    cores over the same format.
 *  - "Accelerating GPU inference of LLMs with moderately unstructured sparse
 *    weight matrices", Sec. 1 (Challenges 1-3) and Sec. 2.1: the pattern is
 *    computed offline and stored in a dedicated format; prefill inputs are
 *    [BL, H] and decode inputs [B, H]; at ~50% sparsity position metadata and
 *    on-chip decoding decide whether a sparse kernel beats the dense one.
 *
 * Conventions shared by every entry point
 *  - fp16 data is passed as raw IEEE binary16 bits (uint16_t / void*).
 *  - W is row-major M x K with leading dimension ldw >= K (elements).
 *  - Activations are TOKEN-MAJOR: X is N rows of K elements, row n is token
 *    n, leading dimension ldx >= K.  The mathematical operand is X^T (K x N).
 *  - Outputs are token-major too: Y is N rows of M elements, ldy >= M, and is
 *    OVERWRITTEN (no accumulation into existing contents).
 *    Y[n][m] = sum_k mask[m][k] * W[m][k] * X[n][k], accumulated in fp32 and
 *    rounded once to fp16 (round to nearest even).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Launching entry points are asynchronous on that stream; the caller keeps
 *    X and Y alive until the stream work completes.  Y must not alias X.
 *  - Device pointers must belong to the device that is current when the call
 *    is made; a format handle is bound to the device current at creation.
 *  - Every call returns an swm_status.  Nothing aborts or throws, and nothing
 *    prints unless SWM_LOG=1 (read once), which writes one stderr line per
 *    dispatch decision (kernel route, work split) of compress and the
 *    product calls.
 *    On a validation error no output is touched.  Kernel faults are reported
 *    as SWM_ERR_HIP by a later checked call (swm_last_hip_error() holds the
 *    hipError_t of the last failing runtime call).
 *  - Handles are read-only after creation, except that
 *    swm_format_enable_skipping attaches the column-run encoding and its
 *    partial-sum workspace; skipping calls on one handle share that workspace
 *    and must be ordered on one stream.  Other product calls on one handle may
 *    run concurrently.
 *  - Environment variables, for tuning and measurement only (they change the
 *    work split, so a result can change only in its fp32 summation order;
 *    the defaults are the measured best): SWM_DECODE_PATH=loop or
 *    SWM_DECODE_LOOP (use the looped decode kernel, read when a handle is
 *    created), SWM_SKIP = off / on (swm_spmspv never / for every n <= 4 takes
 *    the column-run skipping kernel on a handle that carries it; default up
 *    to 2 tokens; read once), SWM_DENSE_DMA=0 (the register-staged tiled
 *    dense kernel; read once), SWM_DECODE_TPW (decode tiles per wave, read
 *    when a handle is created), SWM_DECODE_WAVES_PER_CU (waves per CU of the
 *    17-32-token decode split, read when a handle is created),
 *    SWM_DENSE_WAVES_PER_CU (streaming dense kernel), SWM_DENSE_BLOCK = 1 / 2
 *    / 3 (tiled dense block 256x256 / 256x128 / 128x128), SWM_EXPAND_MIN_N
 *    (tokens from which swm_spmm_ws expands W, at least 33; read once),
 *    SWM_GLU_TPW (tiles per wave of swm_gate_up_silu; read once), SWM_SMFMAC
 *    (0: the sparse-matrix-core route of SWM_CFG_SMFMAC handles off;
 *    read once), SWM_SMF_WAVES=4 (that route's 2:4 kernel with four waves
 *    per block instead of eight; read once).
 */
#ifndef SWM_H_
#define SWM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swm_status {
  SWM_OK = 0,
  SWM_ERR_INVALID_ARG = 1, /* null pointer, ld < dim, N <= 0, n outside [1,16] */
  SWM_ERR_SHAPE = 2,       /* dimensions inconsistent with the format */
  SWM_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks an alignment rule */
  SWM_ERR_OOM = 4,         /* host or device allocation failed */
  SWM_ERR_OVERFLOW = 5,    /* padded value count would reach 2^32, or a size overflows */
  SWM_ERR_FORMAT = 6,      /* blob or handle fails validation */
  SWM_ERR_HIP = 7,         /* HIP runtime or launch error */
  SWM_ERR_UNSUPPORTED = 8  /* tile shape or size this build has no kernel for */
} swm_status;

/* Opaque compressed-weight handle (owns all of its device memory). */
typedef struct swm_format swm_format;

/* Compress options (swm_tile_cfg.flags). */
#define SWM_CFG_SKIPPING 1 /* also build the column-run encoding of swm_format_enable_skipping */
#define SWM_CFG_SMFMAC 2   /* keep 2:4 layers for the sparse-matrix-core route (see swm_spmm_ws) */

/* Tile shape and compress options.  tm: rows per tile, must be 16.  tk:
 * columns per tile, a multiple of 32 (the product kernels take 64).  flags:
 * 0 or a combination of SWM_CFG_SKIPPING and SWM_CFG_SMFMAC (other bits give
 * SWM_ERR_INVALID_ARG); the host encoders (swm_encode_blob, swm_size_dry_run)
 * ignore it.  NULL = {16, 64, 0}. */
typedef struct swm_tile_cfg {
  int32_t tm;
  int32_t tk;
  int32_t flags;
} swm_tile_cfg;

/* Sizes of a format; bytes_* are the sections of the export blob. */
typedef struct swm_format_info {
  int64_t m, k;
  int32_t tm, tk;
  int64_t mt, kt;          /* tile grid */
  uint64_t nnz;            /* kept entries (unpadded) */
  uint64_t padded_len;     /* stored values including per-tile padding */
  uint32_t max_tile;       /* largest padded tile run, in values */
  uint32_t reserved;
  uint64_t bytes_header, bytes_tile_ptr, bytes_bits, bytes_values, bytes_total;
} swm_format_info;

/* ------------------------------------------------------------------ format */

/* sparse_compress: build the tiled column-bitmap format (SWM-TCB v2) from a
 * dense fp16 W and an optional mask, and upload it to the current device.
 * Source: SPDP abstract (Tiled-CBC format, unstructured static pruning) and
 * the moderate-sparsity page, Sec. 2.1 (pattern precomputed offline).
 *  W, mask: HOST pointers.  mask is uint8 M x K (ldm >= K), nonzero = keep;
 *  NULL keeps every entry whose value is not +0/-0.  Kept entries are stored
 *  with their exact bits (also a kept +-0); pruned entries decode to +0.
 *  Layout: tiles of 16 x tk; every tile column has a 16-bit bitmap and the
 *  bitmaps are stored four to a 64-bit word: word w = 8s + e of a tile holds
 *  in bits 16q..16q+15 the bitmap of tile column 32s + 8q + e, so bit b is
 *  (row b%16, column 32s + 8(b/16) + e).  Kept values are packed word by word,
 *  bit by bit (column by column), each tile run padded to 8 values; uint32
 *  exclusive prefix of run lengths per tile.
 *  With cfg->flags = SWM_CFG_SKIPPING the handle also carries the column-run
 *  encoding that lets swm_spmspv skip zero activations (the same as calling
 *  swm_format_enable_skipping afterwards; the resident size roughly doubles).
 *  With SWM_CFG_SMFMAC it also compacts W (.) mask on the device into the 2:4
 *  layers of the sparse-matrix-core route (see swm_spmm_ws) and keeps them
 *  (M*Kp*1.125 bytes per layer, Kp = K rounded up to 64; one layer for a
 *  mask within 2:4, two otherwise).  An export blob does not carry them: an
 *  imported handle runs the other routes.
 *  Synchronous: returns after the upload on `stream` has completed.
 *  *out receives a new handle owned by the caller (swm_format_destroy). */
swm_status swm_sparse_compress(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm,
                               int64_t M, int64_t K, const swm_tile_cfg* cfg, void* stream,
                               swm_format** out);

/* Host-only encoder: the same bytes swm_sparse_compress uploads, written as an
 * export blob into buf (capacity cap bytes).  buf may be NULL to query the
 * size, which is returned in *size either way.  Touches no GPU. */
swm_status swm_encode_blob(const uint16_t* W, int64_t ldw, const uint8_t* mask, int64_t ldm,
                           int64_t M, int64_t K, const swm_tile_cfg* cfg, void* buf, size_t cap,
                           size_t* size);

/* Export the handle as a little-endian blob: 64-byte header ("SWMT", version
 * 2, M, K, tm, tk, nnz, padded_len, mt, kt, max_tile, 0) || tile_ptr (uint32,
 * mt*kt+1) || bits (uint64, mt*kt*tk/4) || values (uint16, padded_len).
 * buf NULL = size query. */
swm_status swm_format_export(const swm_format* f, void* buf, size_t cap, size_t* size);

/* Validate a blob and upload it as a new handle (synchronous on stream). */
swm_status swm_format_import(const void* buf, size_t size, void* stream, swm_format** out);

/* Check a blob without uploading: header fields, section sizes, monotone
 * tile_ptr with runs that are multiples of 8, run length >= popcount of the
 * tile's bitmaps and < popcount + 8, zero padding, no bits for rows >= M or
 * columns >= K, nnz and max_tile consistent.  Returns SWM_ERR_FORMAT if not. */
swm_status swm_format_validate_blob(const void* buf, size_t size);

/* Fill *info from a handle. */
swm_status swm_format_query(const swm_format* f, swm_format_info* info);

/* Worst-case sizes for an M x K matrix with nnz kept entries (padding at most
 * 7 values per tile); SWM_ERR_OVERFLOW if the padded length could reach 2^32
 * or the byte count overflows.  No allocation. */
swm_status swm_size_dry_run(int64_t M, int64_t K, uint64_t nnz, const swm_tile_cfg* cfg,
                            swm_format_info* info);

/* Release a handle and its device memory (NULL is a no-op). */
swm_status swm_format_destroy(swm_format* f);

/* Expand the handle into dense fp16 W (.) mask on the device: W_dev is M x K,
 * ldw >= K, fully overwritten (pruned positions get +0).  Asynchronous. */
swm_status swm_decompress(const swm_format* f, void* W_dev, int64_t ldw, void* stream);

/* ------------------------------------------------------------------ products */

/* spmm: Y = (W (.) mask) X for any N >= 1 (conventions above).
 * Source: SPDP abstract (decode-phase spMspV kernel and prefill SpMM kernel over
 * one format); moderate-sparsity page Sec. 2.1 (prefill [BL,H], decode [B,H]).
 *  X: DEVICE fp16 token-major N x K (ldx >= K).  Y: DEVICE fp16 N x M (ldy >=
 *  M), overwritten.  N <= 32 runs the decode kernels (the weights are read
 *  once; N > 16 feeds each decoded operand to two 16-token MFMAs), larger N
 *  the prefill kernel.  Asynchronous on stream. */
swm_status swm_spmm(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy,
                    int64_t N, void* stream);

/* Bytes of device workspace swm_spmm_ws uses for N tokens on the current
 * device: M*K*2 rounded up to 256 when that call would expand W (0 where a
 * SWM_CFG_SMFMAC handle takes the sparse-matrix-core route instead) (K a
 * multiple of 8, and N >= 1024, or N >= 256 with the on-chip prefill
 * kernel's ceil(M/128)*ceil(N/256) blocks at most half the CUs or above one
 * round of them), else 0.  The SWM_EXPAND_MIN_N environment variable, read
 * once per process, replaces the rule by N >= its value (values below 33
 * count as 33).  NULL handle -> 0.  Queries the device's CU count only. */
size_t swm_spmm_workspace_bytes(const swm_format* f, int64_t N);

/* spmm_ws: swm_spmm with a caller-owned device workspace; same operation,
 * arguments and result (moderate-sparsity page Sec. 2.1, the prefill
 * product [BL, H] x W^T).  At prefill sizes the product is bound by the
 * matrix cores, and with unstructured sparsity it executes as many MFMAs as
 * the dense product; the on-chip path re-expands every tile once per
 * 256-token block.  When swm_spmm_workspace_bytes(f, N) > 0 and X is 16-byte
 * aligned with ldx % 8 == 0, this call instead expands W (.) mask once into
 * the workspace (row-major, leading dimension K, the layout of
 * swm_decompress) and runs the library's dense MFMA kernel on it: two
 * launches on stream, the second reading what the first wrote.  Otherwise it
 * runs swm_spmm's kernels and leaves the workspace untouched.
 *  Sparse-matrix-core route (handles compressed with SWM_CFG_SMFMAC; the
 *  SWM_SMFMAC environment variable 0 turns it off): at compress time W (.)
 *  mask is compacted once into a 2:4 layer (in every aligned group of 4
 *  columns of a row, the first two kept entries) and, when some row keeps 3
 *  or 4 of a group, a residual layer with the rest, each as values [M][Kp/2]
 *  fp16 plus 2-bit positions [M][Kp/16] uint16 (Kp = K rounded up to 64;
 *  M*Kp*1.125 bytes per layer, device memory held by the handle beside the
 *  tiled format).  Where this call (or swm_spmm) would expand W, it instead
 *  multiplies both layers with v_smfmac_f32_32x32x32_f16 into one fp32
 *  accumulator, with no workspace (moderate-sparsity page, abstract and Sec.
 *  1: a sparse-tensor-core layer plus a residual layer).  The result is the
 *  same product (fp32 summation order differs).  It pays only with a 2:4
 *  mask and 256x256 output blocks on every CU (q_proj 4096x4096 at N = 4096
 *  on one MI355X); a residual layer doubles its matrix instructions, hence
 *  opt-in.  The activations must fit 32-bit byte offsets ((N-1)*ldx + K <
 *  2^31) and M*Kp < 2^32, with X 16-byte aligned and ldx % 8 == 0; otherwise
 *  the call takes the other routes.
 *  workspace: DEVICE, 16-byte aligned, ws_bytes >= swm_spmm_workspace_bytes(f,
 *  N), owned by the caller, contents undefined afterwards; it may be shared by
 *  the handles of several layers as long as the calls are ordered on one
 *  stream (concurrent calls sharing it race).  workspace NULL with ws_bytes 0
 *  is swm_spmm.  SWM_ERR_INVALID_ARG: NULL handle, X or Y; a workspace that
 *  is NULL with ws_bytes > 0 or too small for a call that expands; swm_spmm's
 *  argument errors.  SWM_ERR_ALIGN: a workspace that is not 16-byte aligned.
 *  Asynchronous on stream. */
swm_status swm_spmm_ws(const swm_format* f, const void* X, int64_t ldx, void* Y, int64_t ldy, int64_t N,
                       void* workspace, size_t ws_bytes, void* stream);

/* gate_up_silu: the hidden activation of a gated FFN block for 1 <= n <= 32
 * decode tokens (17-32 tokens run as two launches of at most 16, each
 * reading the weights once), H = SiLU(X W_g^T) (.) (X W_u^T), with the input-adaptive
 * threshold applied: an entry whose magnitude (after rounding to fp16) is
 * below tau is stored as +0.  Source: "Reduced Matrix Multiplication" blog
 * page, Sec. 3.2 (SiLU leaves many hidden channels near zero) and Secs.
 * 4.1-4.2 (H = activation(X W_up) with the model's gate output as the score;
 * only high-response channels of H enter the down projection).  SiLU(z) =
 * z / (1 + e^-z).  Both products run in one launch of the decode kernel (the
 * waves of a slab's workgroup split between the two formats); g and u stay
 * in fp32 and h = SiLU(g) * u is rounded once to fp16.  The output is the
 * input of swm_spmspv / swm_spmspv_threshold on the down projection.
 *  g, u: handles of the gate and up weights, same M and K.  X: DEVICE fp16
 *  token-major n x K (ldx >= K).  H: DEVICE fp16 n x M (ldh >= M),
 *  overwritten.  tau: 0 <= tau <= 65504 (0 keeps every entry).
 *  SWM_ERR_INVALID_ARG: NULL pointers, n outside 1..32, tau outside its
 *  range or NaN, shapes that differ, leading dimensions too small, a handle
 *  on another device.  SWM_ERR_ALIGN: X not 16-byte aligned or ldx % 8 != 0.
 *  SWM_ERR_UNSUPPORTED: K < 8 or K % 8 != 0, n*ldx beyond 32-bit byte
 *  offsets, tiles other than 16 x 64, or K above 8192 (more than 128 tiles
 *  per row: the two formats no longer fit one workgroup).  Asynchronous on
 *  stream. */
swm_status swm_gate_up_silu(const swm_format* g, const swm_format* u, const void* X, int64_t ldx, void* H,
                            int64_t ldh, int32_t n, float tau, void* stream);

/* Bytes of device workspace swm_gate_up_silu_ws uses for n tokens: 0 below
 * 33 tokens (the decode launches of swm_gate_up_silu), else 2*M*K*2 rounded
 * up to 256 (the gate and up weights expanded side by side); 0 for NULL or
 * mismatched handles. */
size_t swm_gate_up_silu_workspace_bytes(const swm_format* g, const swm_format* u, int64_t n);

/* gate_up_silu_ws: swm_gate_up_silu for any token count n >= 1, the same
 * hidden activation H = SiLU(X W_g^T) (.) (X W_u^T) with |H| < tau (after
 * rounding to fp16) stored as +0 ("Reduced Matrix Multiplication" blog page,
 * Secs. 3.2 and 4.1-4.2; the FFN of the prefill input, moderate-sparsity
 * page Sec. 2.1).  Below 33 tokens it is swm_gate_up_silu (the workspace is
 * not touched).  From 33 tokens both weights are expanded into the workspace
 * as one matrix of interleaved rows (gate row m at row 2m, up row m at row
 * 2m + 1) and one dense MFMA product computes both, its epilogue forming
 * h = SiLU(g) * u from the fp32 accumulators of the two rows, rounded once
 * to fp16: no g or u buffer and no separate element-wise pass.  The result
 * equals SiLU(g) * u of two swm_spmm_ws calls up to fp32 summation order.
 *  g, u: handles of the gate and up weights, same M and K.  X: DEVICE fp16
 *  token-major n x K (ldx >= K).  H: DEVICE fp16 n x M (ldh >= M),
 *  overwritten.  tau: 0 <= tau <= 65504 (0 keeps every entry).
 *  workspace: DEVICE, 16-byte aligned, ws_bytes >=
 *  swm_gate_up_silu_workspace_bytes(g, u, n), owned by the caller, contents
 *  undefined afterwards (calls sharing it must be ordered on one stream).
 *  SWM_ERR_INVALID_ARG: NULL handles, X or H; n < 1; tau outside its range
 *  or NaN; shapes that differ; leading dimensions too small; a workspace
 *  that is NULL or too small when n >= 33; a handle on another device.
 *  SWM_ERR_ALIGN: X not 16-byte aligned or ldx % 8 != 0, or a workspace that
 *  is not 16-byte aligned.  SWM_ERR_UNSUPPORTED: K < 8 or K % 8 != 0, tiles
 *  other than 16 x 64, or (from 33 tokens) 2*M*K or (n-1)*ldx + K beyond the
 *  product kernel's 32-bit byte offsets; below 33 tokens swm_gate_up_silu's
 *  errors.  Asynchronous on stream. */
swm_status swm_gate_up_silu_ws(const swm_format* g, const swm_format* u, const void* X, int64_t ldx, void* H,
                               int64_t ldh, int64_t n, float tau, void* workspace, size_t ws_bytes,
                               void* stream);

/* dense_gate_up_silu: the dense counterpart of swm_gate_up_silu_ws, the
 * in-house dense baseline of the gated FFN step (the full-matmul fallback
 * the "Reduced Matrix Multiplication" blog page keeps beside its reduced
 * product): H = SiLU(X Wg^T) (.) (X Wu^T) with |H| < tau (after rounding to
 * fp16) stored as +0, by the dense MFMA kernel with the gated epilogue for
 * every N.  Given the masked weights (W (.) mask, pruned entries +0) it
 * returns the same bits as swm_gate_up_silu_ws from 33 tokens.
 *  W2: DEVICE fp16, 2M x K row-major (ldw >= K), the gate and up weights
 *  interleaved by row: row 2m is gate row m, row 2m + 1 is up row m.
 *  X: DEVICE fp16 token-major N x K (ldx >= K).  H: DEVICE fp16 N x M
 *  (ldh >= M), overwritten.  tau: 0 <= tau <= 65504.
 *  SWM_ERR_INVALID_ARG: NULL pointers, M < 0, K < 0, N <= 0, leading
 *  dimensions too small, tau outside its range or NaN.  SWM_ERR_ALIGN: W2 or
 *  X not 16-byte aligned, ldw % 8 != 0 or ldx % 8 != 0.  SWM_ERR_UNSUPPORTED:
 *  K < 8 or K % 8 != 0, or 2M rows of W2 or the activations beyond the
 *  kernel's 32-bit byte offsets.  M == 0 returns SWM_OK.  Asynchronous on
 *  stream. */
swm_status swm_dense_gate_up_silu(const void* W2, int64_t ldw, const void* X, int64_t ldx, void* H, int64_t ldh,
                                  int64_t M, int64_t K, int64_t N, float tau, void* stream);

/* spmspv: as swm_spmm for 1 <= n <= 16 tokens, for activations with zero
 * input channels (x[t][k] == +0 or -0 for all tokens t).  Such channels
 * contribute exact zeros, so the result equals swm_spmm's up to fp32
 * summation order.
 * Source: SPDP abstract (input-adaptive dynamic pruning; run-time activation
 * skipping in the spMspV kernel); "Reduced Matrix Multiplication" blog page,
 * Sec. 4.2 (an FFN down projection multiplies only the kept channels).
 *  Which kernel runs:
 *  - the handle carries the column-run encoding (SWM_CFG_SKIPPING at
 *    compress time, or swm_format_enable_skipping) and n <= 2: the skipping
 *    kernel.  Per 256-row block it lists the active input columns (any of the
 *    n tokens nonzero) and reads and decodes only their runs, bitmaps and
 *    pointers; a second launch adds the column ranges' partial sums in a
 *    fixed order (bitwise reproducible).  It uses the handle's workspace:
 *    skipping calls on one handle must be ordered on one stream.  Measured on
 *    one MI355X (4096 x 11008 at 50%, one token): 1.1x faster than the full
 *    product at 70% inactive columns, 1.4x at 86%, 1.5x at 92%; it breaks
 *    even near 65% at one token and near 74% at two to four;
 *  - otherwise the full product on the tiled format (swm_spmm's kernels):
 *    with three or more tokens the columns inactive in every token are too
 *    few, and the column-run decode costs 1.5-2.3x the vector instructions
 *    per position of the tiled one.  On the aligned path (K % 8 == 0,
 *    16-byte aligned x, ldx % 8 == 0) nothing is skipped: a 16-row tile
 *    stores each column in at most 32 bytes and packs four columns into each
 *    bitmap word, so dropping inactive columns saves neither fetches nor
 *    decode work; the unaligned path skips the decode of bitmap words whose
 *    four columns are all inactive.
 *  swm_spmspv_threshold runs the skipping kernel for up to 4 tokens. */
swm_status swm_spmspv(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy,
                      int32_t n, void* stream);

/* spmspv_noalloc: swm_spmspv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and result as swm_spmspv, bitwise; the
 * difference is where the skipping path keeps its per-workgroup partial sums:
 * in a fixed array of 4 MiB compiled into the library (each GPU the library
 * runs on holds its own copy until the process ends) instead of the handle's
 * workspace.  The call allocates and frees nothing.
 *  The skipping path (column-run encoding on f, n <= 2) needs
 *  ceil(M/256) * S * 4 * 256 floats of partials (S column splits of the
 *  handle; 1 MiB for a 4096 x 11008 weight); a handle that needs more than
 *  the 4 MiB array gives SWM_ERR_UNSUPPORTED and launches nothing.  Every
 *  call on one GPU shares that GPU's array: calls that overlap in time on one
 *  GPU (concurrent streams, or host threads) race and must be ordered on one
 *  stream.  Each call writes every partial it reads, so no state carries
 *  over between calls.  Other errors as swm_spmspv. */
swm_status swm_spmspv_noalloc(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy,
                              int32_t n, void* stream);

/* spmspv_threshold: swm_spmspv with input-adaptive channel selection fused
 * in: an activation with |x[t][k]| < tau counts as zero, so
 *   Y = (W (.) mask) x~,  x~[t][k] = (|x[t][k]| < tau) ? 0 : x[t][k].
 * The comparison takes the fp16 activation exactly in fp32 against tau (fp32);
 * a column whose every token is below tau is skipped like a zero column.
 * tau = 0 gives swm_spmspv's result bitwise.  A NaN activation is never
 * below tau: it is kept and propagates into the outputs it touches.
 * Source: SPDP abstract (input-adaptive dynamic pruning in the decode spMspV
 * kernel); "Reduced Matrix Multiplication" blog page, Sec. 4.2 (an FFN keeps
 * only the high-response channels of its hidden activation and multiplies
 * them with the matching part of the down projection).
 *  Runs on the column-run path only: f must carry the column-run encoding
 *  (SWM_CFG_SKIPPING or swm_format_enable_skipping) and 1 <= n <= 4, else
 *  SWM_ERR_UNSUPPORTED (nothing launched).
 *  Same buffers, ownership, ordering and errors as swm_spmspv; tau < 0, NaN
 *  or above 65504 gives SWM_ERR_INVALID_ARG. */
swm_status swm_spmspv_threshold(const swm_format* f, const void* x, int64_t ldx, void* y, int64_t ldy,
                                int32_t n, float tau, void* stream);

/* format_enable_skipping: attach to f the column-run encoding (SWM-CR v2)
 * that lets swm_spmspv skip zero activations, and upload it to f's device.
 * Source: SPDP abstract (run-time skipping of zero activations in the decode
 * spMspV kernel); "Reduced Matrix Multiplication" blog page, Sec. 4.2 (the
 * product over the kept input channels equals the full product).
 *  The encoding holds the same kept entries as f, regrouped column by column
 *  inside blocks of 256 rows, the blocks of a column stored four at a time:
 *  block b = 4g + j, entry e = (g*K + k)*4 + j (column k of block b; blocks
 *  past the last one are empty entries) has 4 bitmap words (bit i of word q
 *  <=> row 256b + 64q + i), a run of its kept fp16 values in row order padded
 *  to 4 values, and a uint32 exclusive prefix of run lengths.  The handle owns the device copy (freed by
 *  swm_format_destroy) and a workspace for the per-workgroup partial sums.
 *  Synchronous.  Idempotent.  Call it before f is used by other threads or
 *  streams (like creation).  *bytes (nullable) receives the encoding's size.
 *  Errors: SWM_ERR_INVALID_ARG (null f, f on another device), SWM_ERR_OOM,
 *  SWM_ERR_OVERFLOW, SWM_ERR_UNSUPPORTED (M or K too large), SWM_ERR_HIP. */
swm_status swm_format_enable_skipping(swm_format* f, void* stream, uint64_t* bytes);

/* format_enable_smfmac: attach to f the 2:4 layers of the sparse-matrix-core
 * prefill route (see swm_spmm_ws) and keep them on f's device, as
 * SWM_CFG_SMFMAC does at compress time; also for handles from
 * swm_format_import, whose blob does not carry them.  Source: the
 * moderate-sparsity page, abstract and Sec. 1 (a sparse-tensor-core layer
 * plus a residual layer).  The layers hold the same kept entries as f:
 * values [M][Kp/2] fp16 and 2-bit positions [M][Kp/16] uint16 per layer (Kp
 * = K rounded up to 64), a residual layer only when some row keeps 3 or 4 of
 * an aligned group of 4 columns.  Synchronous; idempotent; call it before f
 * is used by other threads or streams.  *bytes (nullable) receives the
 * layers' size.  Errors: SWM_ERR_INVALID_ARG (null f, f on another device),
 * SWM_ERR_UNSUPPORTED (tiles other than 16 x 64), SWM_ERR_OOM, SWM_ERR_HIP. */
swm_status swm_format_enable_smfmac(swm_format* f, void* stream, uint64_t* bytes);

/* colruns_encode_blob: host-only derivation of the SWM-CR v2 blob (32-byte
 * header b"SWMC", u32 version 2, i64 M, i64 K, u32 rows per block = 256,
 * u32 row blocks; then ptr, bits, values as described above) from a SWM-TCB v2
 * export blob, for byte-exact checks of the encoding.  Same sizing protocol as
 * swm_format_export: *size receives the blob size; out may be NULL to query;
 * cap < size gives SWM_ERR_INVALID_ARG.  An invalid input blob gives the
 * validator's status.  Source: as swm_format_enable_skipping. */
swm_status swm_colruns_encode_blob(const void* tcb_blob, size_t size, void* out, size_t cap, size_t* size_out);

/* dense_gemm: Y = W X with a DENSE fp16 W (row-major M x K, ldw >= K, device),
 * the same X / Y conventions, any N >= 1.  The in-house dense baseline and the
 * fallback to the full product.  N <= 16 runs the streaming kernel; larger N
 * the MFMA-tiled kernel, except N <= 32 when its 256x256 blocks would occupy
 * under a quarter of the CUs (then two 16-token streaming passes).
 * Asynchronous on stream; allocates nothing and never synchronizes, so it
 * may be captured into a graph on any call.
 * Source: moderate-sparsity page, Sec. 1 (a sparse kernel is only useful if it
 * beats the dense product at the same shape). */
swm_status swm_dense_gemm(const void* W, int64_t ldw, const void* X, int64_t ldx, void* Y,
                          int64_t ldy, int64_t M, int64_t K, int64_t N, void* stream);

/* ------------------------------------------------------------------ measurement */

/* hbm_stream: read `bytes` (a multiple of 16) from the device buffer `buf` with
 * `blocks` workgroups of 256 threads, each lane keeping `unroll` (1, 2, 4, 8 or
 * 16) 16-byte loads in flight, and fold them into out[] (device, blocks*4
 * uint32, overwritten).  A calibration kernel: it gives the read bandwidth the
 * memory system reaches for a given byte count and launch shape, the
 * "achievable" reference next to the 8 TB/s peak.  Asynchronous. */
swm_status swm_hbm_stream(const void* buf, size_t bytes, int32_t unroll, int32_t blocks,
                          uint32_t* out, void* stream);

/* ------------------------------------------------------------------ misc */

/* Static string for a status code (never NULL). */
const char* swm_status_str(swm_status s);

/* hipError_t value of the last failing HIP call in this process (0 if none). */
int32_t swm_last_hip_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int32_t swm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWM_H_ */
