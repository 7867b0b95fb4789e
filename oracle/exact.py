"""Exact integer brute force for pinning the fp64 reference (test infra only).

Every finite fp16 value is an integer multiple of 2**-24 (the smallest
subnormal), so w * x is an integer multiple of 2**-48 and a dot product over K
terms is exact in Python integers.  This is independent of numpy's BLAS and of
any summation order.
"""
from __future__ import annotations

import numpy as np

_SCALE = float(2 ** 24)


def _to_int(a: np.ndarray) -> np.ndarray:
    a64 = np.asarray(a, dtype=np.float16).astype(np.float64)
    if not np.all(np.isfinite(a64)):
        raise ValueError("exact brute force needs finite inputs")
    scaled = a64 * _SCALE  # exact: power-of-two scaling of an fp16 value
    out = np.empty(a64.shape, dtype=object)
    flat = out.reshape(-1)
    for i, v in enumerate(scaled.reshape(-1)):
        flat[i] = int(v)
    return out


def exact_masked_matmul(W, mask, X_tok):
    """Exact Y_tok[n, m] * 2**48 as Python ints, object array of shape (N, M)."""
    W = np.asarray(W, dtype=np.float16)
    M, K = W.shape
    iw = _to_int(W)
    if mask is not None:
        m = np.asarray(mask, dtype=bool)
        iw = np.where(m, iw, 0)
    ix = _to_int(np.asarray(X_tok, dtype=np.float16))
    N = ix.shape[0]
    out = np.empty((N, M), dtype=object)
    for n in range(N):
        xr = ix[n]
        for mi in range(M):
            out[n, mi] = int(np.dot(iw[mi], xr))
    return out


def exact_to_float(Yint) -> np.ndarray:
    """Nearest float64 of the exact integer results (divided by 2**48)."""
    from fractions import Fraction
    f = np.empty(Yint.shape, dtype=np.float64)
    den = 2 ** 48
    for idx, v in np.ndenumerate(Yint):
        f[idx] = float(Fraction(v, den))
    return f


def fp64_error_bound(W, mask, X_tok) -> np.ndarray:
    """Deterministic bound gamma_K * sum|w x| on any float64 summation order.

    gamma_K = K u / (1 - K u) with u = 2**-53 (Higham, Thm 3.1); products of two
    fp16 values are exact in float64, so only the additions round.
    """
    W64 = np.abs(np.asarray(W, dtype=np.float16).astype(np.float64))
    if mask is not None:
        W64 = np.where(np.asarray(mask, dtype=bool), W64, 0.0)
    X64 = np.abs(np.asarray(X_tok, dtype=np.float16).astype(np.float64))
    K = W64.shape[1]
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    return gamma * (W64 @ X64.T).T
