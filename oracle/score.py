"""Probe attention scores and per-token features.

Test infrastructure only (see the package docstring).

Sources:
* GraceKV page, '03 Bottom-up value flow': direct attention from question
  and sequence-tail probes identifies explicit evidence.
* DistillCache paper, Sec. 3.1.1 (State Space): per-token features
  [attention mass, value L2 norm, variance of mass across heads,
  attention-weighted entropy of the attending queries, normalized position].
* GraceKV page, '03 Bottom-up value flow': a layer/KV-head sensitivity
  multiplier (no formula is given; reading below).

Readings where the pages leave a step open:
* Probes are query vectors already rotated at positions after the context;
  each probe row sees every cached key of its sequence (no mask).
* Relevance r0_i is the attention mass summed over all probe rows of the KV
  group (G query heads x P probes), so it sums to G*P per (layer, KV head).
* The "recent queries" of the entropy feature are the probe rows.
* Variance across heads is the population variance over the G query heads of
  the per-head mass m_gi = sum_p a_(g,p),i.
* Head sensitivity s = sum_i r0_i ||v_i|| / sum_i r0_i.
"""
from __future__ import annotations

import numpy as np

from .common import to64


def _unit_scores(Q: np.ndarray, K: np.ndarray, V: np.ndarray, G: int, P: int):
    """One (sequence, layer, KV head) unit. Q: [G*P, d]; K, V: [L, d]."""
    L, d = K.shape
    c = 1.0 / np.sqrt(d)
    S = c * (Q @ K.T)                                  # [R, L] logits
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]                        # log-partition per row
    A = np.exp(S - lse[:, None])                       # softmax rows
    ent = lse - (A * S).sum(axis=1)                    # H(a_rho) = -sum a log a
    r0 = A.sum(axis=0)
    mg = A.reshape(G, P, L).sum(axis=1)                # [G, L]
    sigma = mg.var(axis=0)                             # population variance over g
    wsum = (A * ent[:, None]).sum(axis=0)
    Hi = np.where(r0 > 0, wsum / np.where(r0 > 0, r0, 1.0), 0.0)
    vn = np.sqrt((V * V).sum(axis=1))
    pos = np.arange(L, dtype=np.float64) / max(L - 1, 1)
    den = r0.sum()
    sens = (r0 * vn).sum() / den if den > 0 else 0.0
    return r0, np.stack([r0, vn, sigma, Hi, pos]), lse, ent, sens


def probe_scores(K, V, Qp, cu, cfg):
    """Score every cached token with the probe rows of its KV group.

    K, V: [Ly][H][T][d]; Qp: [S][Ly][H*G][P][d]; cu: [S+1] offsets.
    Returns float32 arrays: r0 [Ly][H][T], feats [5][Ly][H][T],
    lse and ent [S][Ly][H*G][P], head_sens [S][Ly][H].
    """
    Ly, H, T, d = K.shape
    S = len(cu) - 1
    G, P = cfg.G, cfg.P
    r0 = np.zeros((Ly, H, T))
    feats = np.zeros((5, Ly, H, T))
    lse = np.zeros((S, Ly, H * G, P))
    ent = np.zeros((S, Ly, H * G, P))
    sens = np.zeros((S, Ly, H))
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for l in range(Ly):
            for h in range(H):
                Q = to64(Qp[s, l, h * G:(h + 1) * G]).reshape(G * P, d)
                Ku = to64(K[l, h, a:b])
                Vu = to64(V[l, h, a:b])
                r, f, ls, en, sn = _unit_scores(Q, Ku, Vu, G, P)
                r0[l, h, a:b] = r
                feats[:, l, h, a:b] = f
                lse[s, l, h * G:(h + 1) * G] = ls.reshape(G, P)
                ent[s, l, h * G:(h + 1) * G] = en.reshape(G, P)
                sens[s, l, h] = sn
    f32 = np.float32
    return {"r0": r0.astype(f32), "feats": feats.astype(f32), "lse": lse.astype(f32),
            "ent": ent.astype(f32), "head_sens": sens.astype(f32)}
