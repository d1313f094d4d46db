"""Offline SVDQuant decomposition of a dense linear layer into the library's inputs.

Stages 2 and 3 of the SVDQuant overview figure (Nunchaku README, "Method > Quantization method -
SVDQuant"): per input channel k the activation range is migrated into the weights with
lambda_k = sqrt(max|X[:, k]| / max|W[k, :]|) (1 when either is 0), the runtime keeps
inv_k = float32(1 / lambda_k) and the weights take lambda'_k = 1 / float64(inv_k) so the two
cancel exactly; the smoothed weight W_hat = diag(lambda') W is split by a truncated SVD into
L1 = U_r S_r and L2 = V_r^T, whose bf16 roundings form the 16-bit branch; the residual
R = W_hat - bf16(L1) bf16(L2) (float64, stored float32) is what the packer quantizes to 4 bits.

This runs once per layer on the host, before any inference call, like a checkpoint converter;
it is not part of the layer's forward pass. numpy (LAPACK) provides the SVD.
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def _bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 value (ties to even), kept as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).reshape(np.shape(a))


def decompose(x_calib: np.ndarray, w: np.ndarray, rank: int, svd=None) -> Dict[str, np.ndarray]:
    """x_calib float32 [M, K] (calibration activations), w float32 [K, N] (y = x @ w).

    Returns ``inv_smooth`` float32 [K], ``l1`` float32 [K, r] and ``l2`` float32 [r, N] (bf16-exact
    values), ``resid`` float32 [K, N], and ``svd``: the (u, s, vt) of the smoothed weight, which a
    later call on the same x_calib and w may pass back in to get another rank without a new SVD.
    """
    xa = np.abs(np.asarray(x_calib, dtype=np.float64)).max(axis=0)
    wa = np.abs(np.asarray(w, dtype=np.float64)).max(axis=1)
    lam = np.where((xa > 0) & (wa > 0), np.sqrt(np.divide(xa, wa, out=np.ones_like(xa), where=wa > 0)), 1.0)
    inv = (1.0 / lam).astype(np.float32)
    w_hat = (1.0 / inv.astype(np.float64))[:, None] * np.asarray(w, dtype=np.float64)
    K, N = w_hat.shape
    if rank > 0:
        if svd is None:
            svd = np.linalg.svd(w_hat, full_matrices=False)
        u, s, vt = svd
        l1 = _bf16_values((u[:, :rank] * s[:rank]).astype(np.float32))
        l2 = _bf16_values(vt[:rank].astype(np.float32))
        resid = (w_hat - l1.astype(np.float64) @ l2.astype(np.float64)).astype(np.float32)
    else:
        l1 = np.zeros((K, 0), np.float32)
        l2 = np.zeros((0, N), np.float32)
        resid = w_hat.astype(np.float32)
    return {"inv_smooth": inv, "l1": l1, "l2": l2, "resid": resid, "svd": svd}
