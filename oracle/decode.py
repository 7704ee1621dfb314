"""Decode attention over a (compressed or full) ragged cache.

Test infrastructure only (see the package docstring).

Sources:
* GraceKV page, '05 Physical cache packing': decoding reads the physical
  ragged cache; newly generated tokens are appended with multiplicity one.
* DistillCache paper, Sec. 3.1.3: teacher (full) and student (pruned) caches
  both append each new (k_t, v_t).
* GraceKV page, 'Inside one cache entry' (multiplicity): a prototype counts
  for mu tokens, read here as a logit bias ln(mu).

Reading: no model runs. Step t appends one seeded (k, v) per (layer, KV head)
at position L + t; the seeded query of each (layer, query head) attends over
the segment plus the appended tokens 0..t:
    z_e = c <q, k_e> + ln(mu_e),   o = sum_e softmax(z)_e v_e,
and the step's output row is x = sum over layers of the concatenated heads
(layer order), a residual-stream stand-in that feeds the vocab projection.
"""
from __future__ import annotations

import numpy as np

from .common import to64, logsumexp


def full_view(K, V, cu):
    """The uncompressed cache as a ragged cache (every token, ln mu = 0)."""
    Ly, H, T, d = K.shape
    S = len(cu) - 1
    seg_off = np.zeros((S, Ly, H), dtype=np.int64)
    seg_len = np.zeros((S, Ly, H), dtype=np.int32)
    for l in range(Ly):
        for h in range(H):
            for s in range(S):
                seg_off[s, l, h] = (l * H + h) * T + int(cu[s])
                seg_len[s, l, h] = int(cu[s + 1] - cu[s])
    return {"K": to64(K).reshape(Ly * H * T, d), "V": to64(V).reshape(Ly * H * T, d),
            "lnmu": np.zeros(Ly * H * T, dtype=np.float32),
            "pos": None, "seg_off": seg_off, "seg_len": seg_len}


def decode_step(cache, Kd, Vd, Qd_t, t, G):
    """One decode step. cache: ragged dict (float64 K/V); Kd, Vd:
    [Ly][H][S][T_dec][d]; Qd_t: [S][Ly][H*G][d]. Returns x [S][H*G*d] (float64)
    and o [S][Ly][H*G][d]."""
    S, Ly, HG, d = Qd_t.shape
    H = HG // G
    c = 1.0 / np.sqrt(d)
    Kd64, Vd64 = to64(Kd), to64(Vd)
    q64 = to64(Qd_t)
    o = np.zeros((S, Ly, HG, d))
    for s in range(S):
        for l in range(Ly):
            for h in range(H):
                off, n = int(cache["seg_off"][s, l, h]), int(cache["seg_len"][s, l, h])
                Ke = np.concatenate([cache["K"][off:off + n], Kd64[l, h, s, : t + 1]], axis=0)
                Ve = np.concatenate([cache["V"][off:off + n], Vd64[l, h, s, : t + 1]], axis=0)
                bias = np.concatenate([np.asarray(cache["lnmu"][off:off + n], dtype=np.float64),
                                       np.zeros(t + 1)])
                z = c * (q64[s, l, h * G:(h + 1) * G] @ Ke.T) + bias[None, :]   # [G, n+t+1]
                p = np.exp(z - logsumexp(z, axis=1)[:, None])
                o[s, l, h * G:(h + 1) * G] = p @ Ve
    x = np.zeros((S, HG * d))
    for l in range(Ly):
        x += o[:, l].reshape(S, HG * d)
    return x, o


def decode_all(cache, Kd, Vd, Qd, G):
    """All steps: returns x float32 [S][T_dec][H*G*d]."""
    Td = Qd.shape[0]
    S = Qd.shape[1]
    xs = np.zeros((S, Td, Qd.shape[3] * Qd.shape[4]))
    for t in range(Td):
        x, _ = decode_step(cache, Kd, Vd, Qd[t], t, G)
        xs[:, t] = x
    return xs.astype(np.float32)
