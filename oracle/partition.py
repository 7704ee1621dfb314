"""Slot partition of the compressible region.

Test infrastructure only (see the package docstring).

Source: GraceKV page, '01 Curvature-guided partition' and 'Technical details
and default settings' (slot construction): normalized hidden states form a
trajectory over positions; turns are good boundaries; a dynamic program also
weighs within-slot dispersion and reasonable slot lengths; slots are 16-128
tokens with a target of 64.

Readings (the pages give no constants):
* h_hat_i = h_i / ||h_i||.
* Turning score of a cut before token b: the mean, over windows w in {2, 8}
  for which b-w >= 0, b+w <= L-1 and both difference vectors are nonzero, of
  (1 - cos(h_hat_b - h_hat_{b-w}, h_hat_{b+w} - h_hat_b)) / 2; 0 if none.
* Cost of a slot [a, a+n): sum_i ||h_hat_i - mean||^2
  + lambda_len * ((n - target) / target)^2. A cut before token c earns
  lambda_curv * kappa_c. Both are quantized to integers as
  round-half-away(x * 2^20) before the DP, which then runs in exact integer
  arithmetic; ties go to the earlier previous cut. Surprisal is not used.
* Several sampled depths (hidden [D][T][dim], 'Technical details': turns
  stabilized across sampled depths and windows): the turning score is the
  mean over every valid (depth, window) pair and the dispersion term the mean
  over depths of each depth's dispersion.
* Surprisal (a smaller auxiliary boundary signal): a cut before token b also
  earns lambda_surp * s_b / max s over the sequence (0 when that maximum is
  not positive), added to lambda_curv * kappa_b before quantization.
* Regions shorter than slot_min form a single slot.
* Fixed-length mode: slots of slot_len tokens, the last one shorter.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np

from .common import to64, regions

QSCALE = float(2 ** 20)
WINDOWS = (2, 8)


def _q(x: float) -> int:
    # round half away from zero (all quantized quantities are >= 0)
    return int(math.floor(x * QSCALE + 0.5)) if x >= 0 else -int(math.floor(-x * QSCALE + 0.5))


def normalize(h: np.ndarray) -> np.ndarray:
    n = np.sqrt((h * h).sum(axis=1, keepdims=True))
    return np.where(n > 0, h / np.where(n > 0, n, 1.0), 0.0)


def turning_values(hn: np.ndarray, b: int) -> list:
    """The valid window turning values at position b of one trajectory."""
    L = hn.shape[0]
    vals = []
    for w in WINDOWS:
        if b - w < 0 or b + w > L - 1:
            continue
        u = hn[b] - hn[b - w]
        v = hn[b + w] - hn[b]
        nu, nv = np.linalg.norm(u), np.linalg.norm(v)
        if nu == 0 or nv == 0:
            continue
        vals.append((1.0 - float(u @ v) / (nu * nv)) / 2.0)
    return vals


def turning_score(hn: np.ndarray, b: int) -> float:
    """kappa_b of one trajectory: the mean of its valid window values, 0 if
    there are none."""
    vals = turning_values(hn, b)
    return float(np.mean(vals)) if vals else 0.0


def slot_cost(hn: np.ndarray, a: int, n: int, cfg) -> float:
    x = hn[a:a + n]
    mu = x.mean(axis=0)
    disp = float(((x - mu) ** 2).sum())
    t = float(cfg.slot_target)
    return disp + float(np.float32(cfg.lambda_len)) * ((n - t) / t) ** 2


def slot_costs(hidden, cu, cfg, surprisal=None):
    """Quantized DP inputs in the boundary layout.

    hidden: [T][dim] or [D][T][dim] (D sampled depths); surprisal: [T] or None.
    cost_q int64 [T][slot_max - slot_min + 1]: row = index of a slot's LAST
    token (global token index), column = n - slot_min; cut_q int64 [T]: cut
    before that token. Rows outside a sequence's compressible region, and
    slots that would start before it, are left at 0 (never read).
    """
    H = to64(hidden)
    if H.ndim == 2:
        H = H[None]
    D, T = H.shape[0], H.shape[1]
    nmin, nmax = cfg.slot_min, cfg.slot_max
    cost_q = np.zeros((T, nmax - nmin + 1), dtype=np.int64)
    cut_q = np.zeros((T,), dtype=np.int64)
    lam_c = float(np.float32(cfg.lambda_curv))
    lam_s = float(np.float32(getattr(cfg, "lambda_surp", 0.0)))
    sur = None if surprisal is None else to64(surprisal)
    t_len = float(cfg.slot_target)
    lam_len = float(np.float32(cfg.lambda_len))
    for s in range(len(cu) - 1):
        a0, b0 = int(cu[s]), int(cu[s + 1])
        L = b0 - a0
        if L == 0:
            continue
        hns = [normalize(H[dd, a0:b0]) for dd in range(D)]
        pe, c0, c1, ss = regions(L, cfg)
        smax = float(sur[a0:b0].max()) if sur is not None else 0.0
        for c in range(c0, c1):
            vals = [v for hn in hns for v in turning_values(hn, c)]
            bonus = lam_c * (float(np.mean(vals)) if vals else 0.0)
            if sur is not None and smax > 0:
                bonus += lam_s * float(sur[a0 + c]) / smax
            cut_q[a0 + c] = _q(bonus)
        for e in range(c0 + 1, c1 + 1):                # exclusive slot end
            for n in range(nmin, nmax + 1):
                st = e - n
                if st < c0:
                    break
                disp = 0.0
                for hn in hns:
                    x = hn[st:st + n]
                    disp += float(((x - x.mean(axis=0)) ** 2).sum())
                cost = disp / D + lam_len * ((n - t_len) / t_len) ** 2
                cost_q[a0 + e - 1, n - nmin] = _q(cost)
    return cost_q, cut_q


def dp_slots(cost_q: np.ndarray, cut_q: np.ndarray, a0: int, c0: int, c1: int, cfg
             ) -> List[Tuple[int, int]]:
    """Minimum-cost segmentation of [c0, c1) (sequence positions) into slots of
    slot_min..slot_max tokens. Returns [(start, n)] in position order."""
    nmin, nmax = cfg.slot_min, cfg.slot_max
    Lc = c1 - c0
    if Lc <= 0:
        return []
    if Lc < nmin:
        return [(c0, Lc)]
    INF = None
    f = [INF] * (Lc + 1)
    arg = [0] * (Lc + 1)
    f[0] = 0
    for e in range(1, Lc + 1):
        best, bn = INF, 0
        for n in range(min(nmax, e), nmin - 1, -1):     # larger n = earlier cut first
            p = e - n
            if f[p] is None:
                continue
            v = f[p] + int(cost_q[a0 + c0 + e - 1, n - nmin])
            if p > 0:
                v -= int(cut_q[a0 + c0 + p])
            if best is None or v < best:
                best, bn = v, n
        f[e] = best
        arg[e] = bn
    assert f[Lc] is not None, "no valid segmentation"
    out = []
    e = Lc
    while e > 0:
        n = arg[e]
        out.append((c0 + e - n, n))
        e -= n
    return out[::-1]


def fixed_slots(c0: int, c1: int, n: int) -> List[Tuple[int, int]]:
    return [(a, min(n, c1 - a)) for a in range(c0, c1, n)]


def slots_for(cu, cfg, cost_q=None, cut_q=None) -> List[List[Tuple[int, int]]]:
    """Slot lists per sequence, [(start, n)] in sequence positions."""
    out = []
    for s in range(len(cu) - 1):
        a0, b0 = int(cu[s]), int(cu[s + 1])
        L = b0 - a0
        pe, c0, c1, ss = regions(L, cfg)
        if cfg.token_mode:
            out.append([])
        elif cfg.slot_len > 0:
            out.append(fixed_slots(c0, c1, cfg.slot_len))
        else:
            out.append(dp_slots(cost_q, cut_q, a0, c0, c1, cfg))
    return out
