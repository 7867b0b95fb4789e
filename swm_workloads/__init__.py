"""Seeded synthetic inputs for the sparse-weight matmul path.

This module only *makes inputs*: fp16 weight matrices, pruning masks and
activations with the shapes and value distributions of the Llama-2-7B-shaped
workloads.  It holds none of the product's arithmetic (no matmul, no format
encoding) and is the only code shared by the oracle side and the GPU side.

Conventions
-----------
* ``W`` is ``(M, K)`` fp16, out x in (the ``nn.Linear.weight`` layout).
* ``mask`` is ``(M, K)`` bool; pruned entries of ``W`` are set to exactly +0.
* Activations are returned *token-major*: ``X`` has shape ``(N, K)``, i.e. row
  ``n`` is token ``n`` and is contiguous over the input dimension.  The
  mathematical operand of the product is its transpose, ``X.T`` (K x N).

Random streams are numpy ``default_rng([config, role, index])`` (PCG64 seeded
through SeedSequence).  Roles: W = 0, mask = 1, X = 2, g = 3, u = 4.  Normals
are drawn in float64, scaled, then cast with ``astype(np.float16)`` (round to
nearest even).  Activations are drawn once at the largest token count of a
workload and sliced, so an N sweep shares its data.
"""
from __future__ import annotations

import numpy as np

ROLE_W, ROLE_MASK, ROLE_X, ROLE_G, ROLE_U = 0, 1, 2, 3, 4

# Workload ids (the first element of every seed).
CFG_TINY, CFG_DECODE, CFG_SPMSPV, CFG_PREFILL, CFG_LAYER, CFG_WIDE = 1, 2, 3, 4, 5, 6

LLAMA7B_LINEARS = (
    ("q_proj", 4096, 4096),
    ("k_proj", 4096, 4096),
    ("v_proj", 4096, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 11008, 4096),
    ("up_proj", 11008, 4096),
    ("down_proj", 4096, 11008),
)


def rng(config: int, role: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(config), int(role), int(index)])


def normal_fp16(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    return (scale * g.standard_normal(shape)).astype(np.float16)


def keep_count(K: int, sparsity: float) -> int:
    """Entries kept per row: K - round_half_even(s*K)."""
    return int(K - np.round(sparsity * K))


def magnitude_prune_mask(W: np.ndarray, sparsity: float) -> np.ndarray:
    """Per-row magnitude pruning of an fp16 matrix.

    Each row keeps its ``keep_count(K, s)`` largest-|w| entries.  Magnitudes are
    compared on the fp16 values themselves; equal magnitudes are ranked by the
    lower column index first (a stable descending order).
    """
    W = np.asarray(W, dtype=np.float16)
    M, K = W.shape
    keep = keep_count(K, sparsity)
    mask = np.zeros((M, K), dtype=bool)
    if keep <= 0:
        return mask
    if keep >= K:
        mask[:] = True
        return mask
    # |w| of a finite fp16 is monotone in its low 15 bits; build a unique key
    # that sorts larger magnitude first and, among equals, lower column first.
    absbits = (W.view(np.uint16) & np.uint16(0x7FFF)).astype(np.uint32)
    key = ((np.uint32(0x7FFF) - absbits) << np.uint32(16)) | np.arange(K, dtype=np.uint32)[None, :]
    part = np.argpartition(key, keep - 1, axis=1)[:, :keep]
    rows = np.repeat(np.arange(M), keep)
    mask[rows, part.ravel()] = True
    return mask


def prune_2_4_mask(W: np.ndarray) -> np.ndarray:
    """2:4 pruning along K: in every group of 4 consecutive columns of a row the
    2 largest-|w| entries are kept (equal magnitudes: lower column first); a
    trailing group shorter than 4 keeps its first half, rounded up."""
    W = np.asarray(W, dtype=np.float16)
    M, K = W.shape
    mask = np.zeros((M, K), dtype=bool)
    K4 = K - K % 4
    if K4:
        absbits = (W[:, :K4].view(np.uint16) & np.uint16(0x7FFF)).astype(np.int32).reshape(M, K4 // 4, 4)
        key = (0x7FFF - absbits) * 4 + np.arange(4, dtype=np.int32)  # larger |w| first, then lower column
        order = np.argsort(key, axis=2, kind="stable")[:, :, :2]
        g = np.zeros((M, K4 // 4, 4), dtype=bool)
        np.put_along_axis(g, order, True, axis=2)
        mask[:, :K4] = g.reshape(M, K4)
    if K % 4:
        mask[:, K4:K4 + (K % 4 + 1) // 2] = True
    return mask


def apply_mask(W: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """W with pruned entries replaced by +0 (bit pattern 0x0000)."""
    out = np.asarray(W, dtype=np.float16).copy()
    out[~np.asarray(mask, dtype=bool)] = np.float16(0.0)
    return out


def pruned_weight(config: int, index: int, M: int, K: int, sparsity: float, scale: float = 0.02):
    """0.02*N(0,1) fp16 weight, magnitude-pruned per row; returns (W_pruned, mask)."""
    W = normal_fp16(rng(config, ROLE_W, index), (M, K), scale)
    mask = magnitude_prune_mask(W, sparsity)
    return apply_mask(W, mask), mask


def activations(config: int, index: int, N: int, K: int) -> np.ndarray:
    """Token-major N(0,1) fp16 activations, shape (N, K)."""
    return normal_fp16(rng(config, ROLE_X, index), (N, K))


def silu_gated_sparse(config: int, index: int, N: int, K: int, tau: float = 0.3) -> np.ndarray:
    """Token-major x = SiLU(g)*u with g, u ~ N(0,1), small entries zeroed.

    The product is formed in float64, rounded to fp16, and every fp16 entry with
    |x| < tau is replaced by +0.  Shape (N, K).
    """
    g = rng(config, ROLE_G, index).standard_normal((N, K))
    u = rng(config, ROLE_U, index).standard_normal((N, K))
    x = (g / (1.0 + np.exp(-g)) * u).astype(np.float16)
    x[np.abs(x.astype(np.float64)) < tau] = np.float16(0.0)
    return x


# ---------------------------------------------------------------- workloads
def tiny():
    """256x512 W ~ 0.02 N(0,1), i.i.d. Bernoulli(0.5) mask, X 8 tokens."""
    M, K, N = 256, 512, 8
    W = normal_fp16(rng(CFG_TINY, ROLE_W), (M, K), 0.02)
    mask = rng(CFG_TINY, ROLE_MASK).random((M, K)) < 0.5
    return apply_mask(W, mask), mask, activations(CFG_TINY, 0, N, K)


def decode_qproj(n_max: int = 16):
    """q_proj 4096x4096 at 50% per-row magnitude pruning; X (n_max, 4096)."""
    W, mask = pruned_weight(CFG_DECODE, 0, 4096, 4096, 0.5)
    return W, mask, activations(CFG_DECODE, 0, n_max, 4096)


def decode_qproj_sparsity(sparsity: float, n_max: int = 16):
    """q_proj 4096x4096 magnitude-pruned to 0.6 or 0.7 (the pages' 60% / 70% points)."""
    idx = {0.6: 1, 0.7: 2}[sparsity]
    W, mask = pruned_weight(CFG_WIDE, idx, 4096, 4096, sparsity)
    return W, mask, activations(CFG_WIDE, idx, n_max, 4096)


def decode_qproj_2_4(n_max: int = 16):
    """q_proj 4096x4096 with a 2:4 magnitude mask along K (the pages' 2:4 point)."""
    W = normal_fp16(rng(CFG_WIDE, ROLE_W, 3), (4096, 4096), 0.02)
    mask = prune_2_4_mask(W)
    return apply_mask(W, mask), mask, activations(CFG_WIDE, 3, n_max, 4096)


def fig1_shape(n: int = 32, M: int = 65536, K: int = 16384):
    """The moderate-sparsity paper's Fig. 1 shape, M/K/N = 66K/16K/32 (66K read as
    65536), at 50%: i.i.d. Bernoulli(0.5) mask (per-row magnitude pruning of 2^30
    entries is left out to keep generation short), W ~ 0.02 N(0,1), X ~ N(0,1).
    Generated in row chunks of float32 to bound host memory."""
    gw, gm = rng(CFG_WIDE, ROLE_W, 4), rng(CFG_WIDE, ROLE_MASK, 4)
    W = np.empty((M, K), dtype=np.float16)
    mask = np.empty((M, K), dtype=bool)
    step = 4096
    for r in range(0, M, step):
        h = min(step, M - r)
        W[r:r + h] = (0.02 * gw.standard_normal((h, K), dtype=np.float32)).astype(np.float16)
        mask[r:r + h] = gm.random((h, K), dtype=np.float32) < 0.5
    W[~mask] = np.float16(0.0)
    return W, mask, activations(CFG_WIDE, 4, n, K)


def spmspv_down(n_max: int = 4, tau: float = 0.3):
    """down_proj 4096x11008 at 50%; x = SiLU(g)*u thresholded at tau."""
    W, mask = pruned_weight(CFG_SPMSPV, 0, 4096, 11008, 0.5)
    return W, mask, silu_gated_sparse(CFG_SPMSPV, 0, n_max, 11008, tau)


PREFILL_SPARSITIES = (0.5, 0.6, 0.7)


def prefill_upgate(sparsity: float = 0.5, n_max: int = 4096):
    """up/gate 11008x4096 magnitude-pruned to ``sparsity``; X (n_max, 4096)."""
    idx = PREFILL_SPARSITIES.index(sparsity) if sparsity in PREFILL_SPARSITIES else 9
    W, mask = pruned_weight(CFG_PREFILL, idx, 11008, 4096, sparsity)
    return W, mask, activations(CFG_PREFILL, 0, n_max, 4096)


def layer_linear(i: int, n_max: int):
    """Linear i (q,k,v,o,gate,up,down = 0..6) of a Llama-2-7B-shaped layer."""
    _, M, K = LLAMA7B_LINEARS[i]
    W, mask = pruned_weight(CFG_LAYER, i, M, K, 0.5)
    return W, mask, activations(CFG_LAYER, i, n_max, K)


def layer_linear_2_4(i: int, n_max: int):
    """Linear i of the same layer pruned 2:4 along K instead (the same dense
    weights, the two largest |w| of every 4 columns kept)."""
    _, M, K = LLAMA7B_LINEARS[i]
    W = normal_fp16(rng(CFG_LAYER, ROLE_W, i), (M, K), 0.02)
    mask = prune_2_4_mask(W)
    return apply_mask(W, mask), mask, activations(CFG_LAYER, i, n_max, K)


# The layer's projections as an inference engine launches them: q, k, v read
# the same input and are stacked by rows into one 12288x4096 matrix, gate and
# up likewise into one 22016x4096 matrix.
LAYER_FUSED = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))


def stack_linears(parts):
    """Row-stack (W, mask, X) triples that share their input: the stacked W,
    mask, and the first part's X."""
    W = np.concatenate([p[0] for p in parts], axis=0)
    mask = np.concatenate([p[1] for p in parts], axis=0)
    return W, mask, parts[0][2]


def layer_fused(g: int, n_max: int):
    """Projection group g (qkv, o, gate_up, down = 0..3) of the layer, its
    linears row-stacked, with the group's shared input."""
    _, idx = LAYER_FUSED[g]
    return stack_linears([layer_linear(i, n_max) for i in idx])
