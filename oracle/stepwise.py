"""Step-wise eviction: score every cached token after each decode step and
keep the top-B (DistillCache paper, Sec. 3.1.1 state features, Sec. 3.1.2
deterministic top-B at inference, Algorithm 1 inference loop).

Test infrastructure only (see the package docstring).

Readings (the paper leaves these open):
* N1 recent queries. The window holds the w most recent query vectors of every
  (layer, query head): before the first step the last w prefill queries, then
  each decode query replaces the oldest. The features only sum over the
  window, so its order does not matter. Every window query attends the whole
  current cache (a_q is a distribution over all cached keys), no mask.
* N2 features of cached token i over all layers, query heads and window
  queries (the paper: across all heads and layers):
  alpha_i = mean of a_q(i); sigma_i = population variance over the Ly*H*G
  query heads of the window-mean mass; H_i = sum a_q(i) H(a_q) / sum a_q(i)
  with H(a) = -sum a ln a (0 when the sum is 0); vnorm_i = mean over (l, h)
  of ||v_i||; pos_i = p_i / max(n_seen - 1, 1) with p_i the token's sequence
  position and n_seen the tokens seen so far.
* N3 policy f_phi: Linear(5, 128) -> LayerNorm -> ReLU -> Linear(128, 128) ->
  LayerNorm -> ReLU -> Linear(128, 1), LayerNorm eps 1e-5, seeded weights
  (the trained policy is not available).
* N4 budget: B = max(floor(r * n_seen), B_min), n_seen = L before the first
  step and L + t + 1 after the t-th decode token: |C_t| is read as the
  context seen so far, so the cache keeps a fraction r of it (read literally
  as the pruned cache's own size, the budget would shrink geometrically).
* N5 prune: keep the top-B tokens by (fp32 score desc, position asc); the same
  tokens leave every (layer, KV head). No region is protected (the paper's
  loop has no hard-coded protection); exact regions of the other modes are
  not used here.
* N6 order inside step t: append (k_t, v_t) to both caches, decode q_t over
  each, push q_t into the window, score, prune (the prune prepares the next
  step).
"""
from __future__ import annotations

import math

import numpy as np

from .common import to64, logsumexp
from .decode import decode_all, full_view
from .kl import kl_rows

LN_EPS = 1e-5


def _layernorm(h, g, b):
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    return (h - mu) / np.sqrt(var + LN_EPS) * g + b


def policy_scores(x, pol):
    """N3: x [n][5] float64 -> scores [n] float64."""
    w = {k: to64(v) for k, v in pol.items()}
    h = np.maximum(_layernorm(x @ w["w1"].T + w["b1"], w["g1"], w["be1"]), 0.0)
    h = np.maximum(_layernorm(h @ w["w2"].T + w["b2"], w["g2"], w["be2"]), 0.0)
    return h @ w["w3"] + w["b3"][0]


def window_features(Kc, Vc, pos, Qwin, n_seen):
    """N2 for one sequence. Kc, Vc: [Ly][H][n][d] float64; pos [n];
    Qwin: [Ly][H*G][w][d] float64. Returns [n][5] float64 columns
    (alpha, vnorm, sigma, H, pos)."""
    Ly, H, n, d = Kc.shape
    HG, w = Qwin.shape[1], Qwin.shape[2]
    G = HG // H
    c = 1.0 / math.sqrt(d)
    mass = np.zeros((Ly, HG, n))      # window-mean mass per query head
    hnum = np.zeros(n)
    hden = np.zeros(n)
    for l in range(Ly):
        for qh in range(HG):
            z = c * (Qwin[l, qh] @ Kc[l, qh // G].T)          # [w][n]
            a = np.exp(z - logsumexp(z, axis=1)[:, None])
            ent = -np.sum(np.where(a > 0, a * np.log(np.where(a > 0, a, 1.0)), 0.0), axis=1)  # [w]
            mass[l, qh] = a.mean(axis=0)
            hnum += (a * ent[:, None]).sum(axis=0)
            hden += a.sum(axis=0)
    alpha = mass.reshape(-1, n).mean(axis=0)
    sigma = mass.reshape(-1, n).var(axis=0)
    hfeat = np.where(hden > 0, hnum / np.where(hden > 0, hden, 1.0), 0.0)
    vnorm = np.sqrt((Vc ** 2).sum(axis=-1)).reshape(-1, n).mean(axis=0)
    posf = np.asarray(pos, dtype=np.float64) / max(n_seen - 1, 1)
    return np.stack([alpha, vnorm, sigma, hfeat, posf], axis=1)


def step_budget(n_seen, cfg):
    """N4."""
    return max(int(math.floor(float(np.float32(cfg.budget_ratio)) * n_seen)), cfg.budget_min)


def keep_top(scores32, pos, B):
    """N5: indices (into the cache) of the kept tokens, in cache order."""
    n = len(pos)
    if B >= n:
        return np.arange(n)
    order = sorted(range(n), key=lambda i: (-float(scores32[i]), int(pos[i])))
    return np.sort(np.array(order[:B], dtype=np.int64))


def run_stepwise(inp, cfg, pol, trace=None):
    """Algorithm 1 over the decode steps of every sequence.

    Returns x_comp [S][T_dec][H*G*d] float32 (the student's outputs), x_full,
    kl [S][T_dec], and per sequence the kept positions after the last step.
    If ``trace`` is a list, each prune appends (s, step, cache size before,
    B, kept positions, fp32 scores, features)."""
    K, V = to64(inp["K"]), to64(inp["V"])
    Qctx, Qd, Kd, Vd = to64(inp["Qctx"]), to64(inp["Qd"]), to64(inp["Kd"]), to64(inp["Vd"])
    cu = inp["cu_seqlens"].numpy()
    Ly, H, T, d = K.shape
    G, w = cfg.G, cfg.window
    Td = Qd.shape[0]
    S = len(cu) - 1
    c = 1.0 / math.sqrt(d)
    x_comp = np.zeros((S, Td, H * G * d))
    kept_final = []
    for s in range(S):
        a0, L = int(cu[s]), int(cu[s + 1] - cu[s])
        Kc, Vc = K[:, :, a0:a0 + L].copy(), V[:, :, a0:a0 + L].copy()
        pos = np.arange(L)
        hist = [Qctx[:, :, a0 + i] for i in range(L)]      # query history, each [Ly][H*G][d]

        def prune(n_seen, step):
            nonlocal Kc, Vc, pos
            Qwin = np.stack(hist[-w:], axis=2)               # [Ly][H*G][w'][d]
            f = window_features(Kc, Vc, pos, Qwin, n_seen)
            sc32 = policy_scores(f, pol).astype(np.float32)
            B = step_budget(n_seen, cfg)
            keep = keep_top(sc32, pos, B)
            if trace is not None:
                trace.append((s, step, len(pos), B, pos[keep].copy(), sc32, f))
            Kc, Vc, pos = Kc[:, :, keep], Vc[:, :, keep], pos[keep]

        prune(L, -1)
        for t in range(Td):
            Kc = np.concatenate([Kc, Kd[:, :, s, t:t + 1]], axis=2)
            Vc = np.concatenate([Vc, Vd[:, :, s, t:t + 1]], axis=2)
            pos = np.append(pos, L + t)
            q = Qd[t, s]                                      # [Ly][H*G][d]
            for l in range(Ly):
                for qh in range(H * G):
                    z = c * (Kc[l, qh // G] @ q[l, qh])
                    p = np.exp(z - logsumexp(z))
                    x_comp[s, t, qh * d:(qh + 1) * d] += p @ Vc[l, qh // G]
            hist.append(q)
            prune(L + t + 1, t)
        kept_final.append(pos.copy())
    x_full = decode_all(full_view(inp["K"], inp["V"], cu), inp["Kd"], inp["Vd"], inp["Qd"], G)
    x_comp = x_comp.astype(np.float32)
    n = S * Td
    kl = kl_rows(x_full.reshape(n, -1), x_comp.reshape(n, -1), inp["W"], cfg.w_dtype).reshape(S, Td)
    return {"x_comp": x_comp, "x_full": x_full, "kl": kl, "kept": kept_final}
