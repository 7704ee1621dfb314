"""Token-to-token relevance propagation.

Test infrastructure only (see the package docstring).

Source: GraceKV page, '03 Bottom-up value flow' and 'Technical details and
default settings' (value flow): probes seed direct relevance, then two graph
hops with default weight 0.3 recover indirect evidence such as a bridge
entity the question does not attend to on its own.

Reading (the pages give no formula): the graph is the causal prefill
attention of the cached tokens, reused from the prefill pass. Each hop takes
the M most relevant tokens of the previous increment as seeds; a seed j
passes w * delta(j) to the keys its own prefill query attends, split by its
causal softmax row averaged over the G query heads of the KV group:

    delta_t(i) = w * sum_{j in seeds_t} delta_{t-1}(j) * (1/G) sum_g b_jg(i),
    b_jg = softmax_{i <= j}(c <q_jg, k_i>),     r = r0 + delta_1 + delta_2.

Seeds are the top-M tokens by delta_{t-1} (ties to the lower index); all
tokens when L <= M.
"""
from __future__ import annotations

import numpy as np

from .common import to64, logsumexp


def _seeds(delta: np.ndarray, M: int) -> np.ndarray:
    L = delta.shape[0]
    order = np.lexsort((np.arange(L), -delta))      # delta desc, index asc
    return np.sort(order[:min(M, L)])


def _unit(Qc: np.ndarray, K: np.ndarray, r0: np.ndarray, G: int, hops: int, M: int, w: float):
    """Qc: [G][L][d] prefill queries of the unit's KV group; K: [L][d]."""
    L, d = K.shape
    c = 1.0 / np.sqrt(d)
    total = r0.copy()
    prev = r0.copy()
    seeds_out = []
    for _ in range(hops):
        seeds = _seeds(prev, M)
        seeds_out.append(seeds)
        delta = np.zeros(L)
        for j in seeds:
            logits = c * (Qc[:, j, :] @ K[: j + 1].T)          # [G, j+1]
            b = np.exp(logits - logsumexp(logits, axis=1)[:, None])
            delta[: j + 1] += w * prev[j] * b.mean(axis=0)
        total = total + delta
        prev = delta
    return total, seeds_out


def propagate(K, Qctx, r0, cu, cfg):
    """K: [Ly][H][T][d]; Qctx: [Ly][H*G][T][d]; r0: float32 [Ly][H][T].

    Returns rel float32 [Ly][H][T] and seeds int32 [hops][S][Ly][H][M]
    (token index within the sequence, ascending, -1 padded).
    """
    Ly, H, T, d = K.shape
    S = len(cu) - 1
    G, M, hops = cfg.G, cfg.n_seeds, cfg.n_hops
    rel = np.zeros((Ly, H, T))
    seeds = -np.ones((hops, S, Ly, H, M), dtype=np.int32)
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for l in range(Ly):
            for h in range(H):
                Ku = to64(K[l, h, a:b])
                Qc = to64(Qctx[l, h * G:(h + 1) * G, a:b])
                r = np.asarray(r0[l, h, a:b], dtype=np.float64)
                tot, sd = _unit(Qc, Ku, r, G, hops, M, float(np.float32(cfg.hop_weight)))
                rel[l, h, a:b] = tot
                for t, sv in enumerate(sd):
                    seeds[t, s, l, h, : len(sv)] = sv
    return {"rel": rel.astype(np.float32), "seeds": seeds}


def propagate_ar(K, Qctx, r0, cu, cfg):
    """The "A r" direction (parity pinned by the matrix form w * A_hat r).

    Reading: the same causal prefill attention graph, with relevance flowing
    from an attended token to every token attending it: token i receives the
    GQA-mean causal softmax average of the previous increment over its prefix,
        delta_t(i) = w * (1/G) sum_g sum_{j<=i} b_ig(j) delta_{t-1}(j),
    r = r0 + delta_1 + ... . Every token is a receiver (no seed cut-off).
    Returns rel float32 [Ly][H][T].
    """
    Ly, H, T, d = K.shape
    S = len(cu) - 1
    G, hops = cfg.G, cfg.n_hops
    w = float(np.float32(cfg.hop_weight))
    c = 1.0 / np.sqrt(d)
    rel = np.zeros((Ly, H, T))
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        if L == 0:
            continue
        mask = np.tril(np.ones((L, L), dtype=bool))
        for l in range(Ly):
            for h in range(H):
                Ku = to64(K[l, h, a:b])
                Qc = to64(Qctx[l, h * G:(h + 1) * G, a:b])
                Ahat = np.zeros((L, L))
                for g in range(G):
                    z = np.where(mask, c * (Qc[g] @ Ku.T), -np.inf)
                    Ahat += np.exp(z - logsumexp(z, axis=1)[:, None])
                Ahat /= G
                prev = np.asarray(r0[l, h, a:b], dtype=np.float64)
                tot = prev.copy()
                for _ in range(hops):
                    prev = w * (Ahat @ prev)
                    tot += prev
                rel[l, h, a:b] = tot
    return {"rel": rel.astype(np.float32)}
