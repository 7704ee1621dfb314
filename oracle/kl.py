"""Per-step KL(full || compressed) through a seeded vocab projection.

Test infrastructure only (see the package docstring).

Sources: DistillCache paper, Sec. 3.1.4 (Reward): the fidelity signal is
D_KL(P_t || P_hat_t) between the next-token distributions of the full cache
(P) and the pruned cache (P_hat), computed from logits with standard
numerical stabilization.

Reading (no model weights): logits = RMSNorm(x) (no gain, eps 1e-6) rounded
to the projection's dtype, times the seeded projection W [vocab][d_model]:
    KL = sum_v P_v (y_v - y_hat_v) - lse(y) + lse(y_hat),   P = softmax(y).
"""
from __future__ import annotations

import numpy as np

from .common import to64, round_to, logsumexp

EPS = 1e-6


def rmsnorm_cast(x: np.ndarray, w_dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + EPS)
    return round_to(x * r, w_dtype)


def kl_rows(x_full, x_comp, W, w_dtype: str) -> np.ndarray:
    """x_full, x_comp: float32 [n][d_model]; W: [vocab][d_model].
    Returns float32 KL per row."""
    Wm = to64(W)
    y = rmsnorm_cast(x_full, w_dtype) @ Wm.T
    yh = rmsnorm_cast(x_comp, w_dtype) @ Wm.T
    ly, lyh = logsumexp(y, axis=1), logsumexp(yh, axis=1)
    P = np.exp(y - ly[:, None])
    kl = (P * (y - yh)).sum(axis=1) - ly + lyh
    return kl.astype(np.float32)
