"""Shared oracle helpers: exact dtype conversion, regions, budgets, RoPE.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np
import torch


def to64(t) -> np.ndarray:
    """Exact conversion of a bf16/fp32/fp64 tensor (or array) to float64."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.float()
        return t.double().numpy()
    return np.asarray(t, dtype=np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (returned as float64 holding bf16 values)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch.bfloat16).double().numpy()


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def regions(L: int, cfg) -> Tuple[int, int, int, int]:
    """Token regions of one sequence (GraceKV page, 'Core idea': the prompt and
    the question/suffix stay exact outside the budget, a recent window stays
    exact inside it, the long context in between competes in the auction).

    Returns (prompt_end, comp_start, comp_end, suffix_start) with
    [0, prompt_end) prompt, [comp_start, comp_end) compressible,
    [comp_end, suffix_start) recent window, [suffix_start, L) suffix.
    Short sequences clamp the regions in the order prompt, suffix, recent.
    """
    pe = min(cfg.prompt_exact, L)
    ss = max(pe, L - cfg.suffix_exact)
    rs = max(pe, ss - cfg.recent_exact)
    return pe, pe, rs, ss


def budgets(lens: List[int], cfg) -> List[dict]:
    """Per-sequence entry budget.

    DistillCache, Algorithm 1 (budget step): B = max(floor(r * |C|), B_min).
    One budget covers every (layer, KV head) entry of a sequence (GraceKV
    page, 'Core idea': one budget across layers, heads and slots), so |C| is
    L * Ly * H. The recent window is charged first; the rest is allocatable.
    The singleton floor may spend at most floor(phi * allocatable) entries
    (GraceKV page, 'Technical details and default settings', singleton floor).
    Head-level hybrid (DistillCache paper, Appendix E.3: the most important
    heads get their full cache, token selection runs in the others, under
    the same overall budget): K = min(floor(f * Ly*H), floor(alloc / C))
    units keep all C compressible tokens and are paid first; the selection
    and the floor share the rest, alloc - K*C. With f = 0, K = 0.
    """
    out = []
    U = cfg.Ly * cfg.H
    f = float(np.float32(getattr(cfg, "hybrid_frac", 0.0)))
    for L in lens:
        B = max(int(math.floor(float(np.float32(cfg.budget_ratio)) * (L * U))), cfg.budget_min)
        pe, cs, ce, ss = regions(L, cfg)
        recent = (ss - ce) * U
        alloc = B - recent
        C = ce - cs
        K = 0
        if f > 0 and C > 0 and alloc > 0:
            K = min(int(math.floor(f * U)), alloc // C, U)
        rest = alloc - K * C
        F = int(math.floor(float(np.float32(cfg.floor_frac)) * rest)) if rest > 0 else 0
        out.append({"B": B, "alloc": alloc, "floor": F, "recent": recent,
                    "free": (pe + (L - ss)) * U, "full_units": K, "comp_len": C, "rest": rest})
    return out


def rope_angles(pos, d: int, base: float) -> np.ndarray:
    """theta_j(pos) = pos * base^(-2j/d), j < d/2, in float64."""
    j = np.arange(d // 2, dtype=np.float64)
    inv = base ** (-2.0 * j / d)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), inv)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate-half RoPE: pairs (j, j + d/2) rotated by theta_j(pos).

    x: [..., d]; pos broadcast against x[..., 0].
    """
    d = x.shape[-1]
    h = d // 2
    ang = rope_angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_inv(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Inverse rotation (rotation by -theta)."""
    d = x.shape[-1]
    h = d // 2
    ang = rope_angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def logsumexp(x: np.ndarray, axis=-1) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))).squeeze(axis)
