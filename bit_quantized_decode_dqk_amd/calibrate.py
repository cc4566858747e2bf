"""Offline construction of the paired transforms A, B from second-moment statistics.

Dual-QK ("Sharp Queries and Flat Keys for Prunable 2-bit KV Caches", arXiv
abstract; tech.dede.sh summary, "Paired transforms instead of shared rotation")
replaces one shared rotation of queries and keys by a pair of non-orthogonal
transforms: the key transform flattens the keys (partial whitening, so that few
outlier channels dominate the 2-bit groups less) and the query transform
concentrates query energy in few channels (a query-aligned basis, so that
pruning to the top channels keeps most of each logit).  The pages name the two
ingredients but print no formula.  This module's reading, for key covariance
S_k, query covariance S_q and a whitening strength alpha in [0, 1]:

    M = S_k^(alpha/2) S_q S_k^(alpha/2),   M R = R diag(lam), lam descending,
    A = S_k^(alpha/2) R,                   B = S_k^(-alpha/2) R.

With row vectors q' = q A and k' = k B:
  - A B^T = I, so q'.k' = q.k (the pair keeps every dot product);
  - E[q'^T q'] = R^T M R = diag(lam): the channels are uncorrelated and ordered
    by query energy, so channel 0 (the protected fp16 channel) carries the most;
  - E[k'^T k'] = R^T S_k^(1 - alpha) R: alpha = 1 whitens the keys fully,
    alpha = 0 gives the plain rotation A = B = R of the query eigenbasis.

This is a host-side fit (numpy, fp64) done once per model layer and KV head
from calibration activations; its outputs are inputs of the decode path, which
never calls it.  Real calibration needs model activations that are not part of
this library, so the fit is exercised on synthetic covariances.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def sym_power(s: np.ndarray, p: float, floor: float = 1e-12) -> np.ndarray:
    """S^p for a symmetric positive semi-definite S (eigenvalues clipped at
    floor * the largest, so that negative powers stay finite)."""
    s = np.asarray(s, dtype=np.float64)
    w, v = np.linalg.eigh(0.5 * (s + s.T))
    w = np.maximum(w, floor * max(float(w.max()), 0.0) + 1e-300)
    return (v * w ** p) @ v.T


def fit_transforms(sigma_k: np.ndarray, sigma_q: np.ndarray, alpha: float = 0.5,
                   dtype=np.float32) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(A, B, lam): the paired transforms of the reading above ([d][d], row-major,
    q' = q A, k' = k B; rounded to `dtype`, fp32 for the library) and the query
    energy per transformed channel, descending (fp64)."""
    if not 0.0 <= alpha <= 1.0:
        raise ValueError("alpha must be in [0, 1]")
    sk_half = sym_power(sigma_k, alpha / 2.0)
    sk_mhalf = sym_power(sigma_k, -alpha / 2.0)
    m = sk_half @ np.asarray(sigma_q, dtype=np.float64) @ sk_half
    lam, r = np.linalg.eigh(0.5 * (m + m.T))
    order = np.argsort(-lam, kind="stable")
    lam, r = lam[order], r[:, order]
    a = sk_half @ r
    b = sk_mhalf @ r
    return a.astype(dtype), b.astype(dtype), lam


def rotation_transforms(d: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The baseline Dual-QK departs from: one random orthogonal rotation R shared
    by queries and keys (A = B = R; fp32)."""
    rng = np.random.default_rng(seed)
    q, rr = np.linalg.qr(rng.standard_normal((d, d)))
    q = q * np.sign(np.diag(rr))[None, :]
    return q.astype(np.float32), q.astype(np.float32)

