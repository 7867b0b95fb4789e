"""fp64 reference of the sparse-weight product (test infrastructure only).

Definition followed
-------------------
A statically pruned weight matrix multiplies dense activations:
Y = (W (.) mask) X with W of shape M x K (out x in) and X of shape K x N.
  * "Unified Static-Dynamic Pruning for Efficient LLM Inference" (SPDP),
    abstract: unstructured static pruning removes weights permanently; the
    product must be the exact sparse product.
  * "Accelerating GPU inference of LLMs with moderately unstructured sparse
    weight matrices", abstract and Sec. 2.1: prefill inputs are [BL, H], decode
    inputs [B, H]; the pattern is computed offline and the residual layer keeps
    the SpMM correct, i.e. the sparse kernel is exact, not an approximation.

Dynamic (input-adaptive) pruning, the spMspV half of SPDP, skips input
channels whose activation is zero.  The reduced-product form Y = W[:, I] x[I]
over the kept channels I is the one of the "Reduced Matrix Multiplication"
blog page, Sec. 4.2 (channel selection for FFN down projections), with I taken
as the channels whose activation is non-zero in at least one token: dropped
terms are then exact zeros and the result equals the full product.

All arithmetic is float64 on the exact fp16 input values.  Accumulation order
is numpy's; the pins in the tests bound it against exact integer arithmetic.
"""
from __future__ import annotations

import numpy as np


def _masked_fp64(W: np.ndarray, mask: np.ndarray | None) -> np.ndarray:
    W64 = np.asarray(W, dtype=np.float16).astype(np.float64)
    if mask is None:
        return W64
    return np.where(np.asarray(mask, dtype=bool), W64, 0.0)


def masked_matmul(W: np.ndarray, mask: np.ndarray | None, X_tok: np.ndarray) -> np.ndarray:
    """Y = (W (.) mask) @ X in float64.

    ``X_tok`` is token-major (N, K); the result is token-major (N, M), i.e.
    ``Y_tok[n, m] = sum_k mask[m,k] W[m,k] X_tok[n,k]``.
    """
    Wm = _masked_fp64(W, mask)
    X64 = np.asarray(X_tok, dtype=np.float16).astype(np.float64)
    return (Wm @ X64.T).T


def active_inputs(X_tok: np.ndarray) -> np.ndarray:
    """Boolean (K,) vector: input channel k is active iff x[n, k] != 0 for some n.

    +0 and -0 both count as zero (fp16 comparison).
    """
    X = np.asarray(X_tok, dtype=np.float16)
    return np.any(X != 0, axis=0)


def masked_matmul_skip(W: np.ndarray, mask: np.ndarray | None, X_tok: np.ndarray) -> np.ndarray:
    """Zero-activation-skipping product: only active input channels take part.

    Steps in the order the pages give them: (1) find the channels that carry a
    non-zero activation, (2) multiply only the weight columns of those channels,
    (3) the result lands in the full output (no scatter is needed for input-side
    selection).
    """
    act = active_inputs(X_tok)
    Wm = _masked_fp64(W, mask)[:, act]
    X64 = np.asarray(X_tok, dtype=np.float16).astype(np.float64)[:, act]
    if Wm.shape[1] == 0:
        return np.zeros((X64.shape[0], Wm.shape[0]), dtype=np.float64)
    return (Wm @ X64.T).T


def threshold_activations(X_tok: np.ndarray, tau: float) -> np.ndarray:
    """Input-adaptive channel selection ("Reduced Matrix Multiplication" blog
    page, Sec. 4.2: an FFN keeps only the high-response channels of its hidden
    activation).  An activation whose magnitude is below tau is dropped (+0);
    every other one is kept unchanged (a NaN is not below tau, so it stays and
    propagates, as in the plain product).  The comparison takes the fp16 value
    exactly in float32 against tau as float32."""
    X = np.asarray(X_tok, dtype=np.float16)
    with np.errstate(invalid="ignore"):
        keep = ~(np.abs(X.astype(np.float32)) < np.float32(tau))
    return np.where(keep, X, np.float16(0.0))


def masked_matmul_threshold(W: np.ndarray, mask: np.ndarray | None, X_tok: np.ndarray, tau: float) -> np.ndarray:
    """Thresholded spMspV: (1) drop activations below tau, (2) the skipping
    product over the channels that stay active (SPDP abstract: input-adaptive
    dynamic pruning at decode)."""
    return masked_matmul_skip(W, mask, threshold_activations(X_tok, tau))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) in float64: the activation
    whose saturation at negative inputs leaves many FFN hidden channels near
    zero ("Reduced Matrix Multiplication" blog page, Sec. 3.2)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gate_up_silu(Wg: np.ndarray, mg: np.ndarray | None, Wu: np.ndarray, mu: np.ndarray | None,
                 X_tok: np.ndarray, tau: float = 0.0) -> np.ndarray:
    """Hidden activation of a gated FFN block and its input-adaptive threshold.

    The blog page (Sec. 4.2) writes the FFN as H = activation(X W_up),
    Y = H W_down, and keeps only the high-response channels of H before the
    down projection; Sec. 4.1 lists the model's own gate output as a ready
    score.  For the gated (Llama-style) block of these workloads this reads
    H = SiLU(g) * u with g, u the statically pruned gate and up products of
    the same tokens (both shaped (N, M)).  A channel is then dropped (+0)
    when |H| rounded to fp16 is below tau (compared in float32, the same
    decision rule as threshold_activations); kept entries are returned
    unrounded, in float64.
    """
    g = masked_matmul(Wg, mg, X_tok)
    u = masked_matmul(Wu, mu, X_tok)
    h = silu(g) * u
    keep = np.abs(h.astype(np.float16).astype(np.float32)) >= np.float32(tau)
    return np.where(keep, h, 0.0)


def to_fp16(Y: np.ndarray) -> np.ndarray:
    """Round a float64 result to fp16, round-to-nearest-even."""
    return np.asarray(Y, dtype=np.float64).astype(np.float16)
