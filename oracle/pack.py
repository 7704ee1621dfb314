"""Physical ragged cache packing.

Test infrastructure only (see the package docstring).

Source: GraceKV page, '05 Physical cache packing': each layer-head pair gets
an independently sized ragged cache; an unselected root writes no entry, an
internal frontier node writes a packed prototype, a singleton writes the
original K/V; with the budget back at full scale every tree expands to its
leaves and the original entries are recovered exactly.

Layout written (the C ABI's ragged layout): segments in (layer, KV head,
sequence) order; within a segment, entries in position order: prompt tokens,
then each slot's frontier nodes left to right (or the kept tokens in token
mode), then the recent window, then the suffix. A token entry carries its
original K/V bits, ln(mu) = 0 and its position; a prototype carries
round(k_hat), round(v_hat) in the cache dtype, ln(mu) and p_rep.
"""
from __future__ import annotations

import numpy as np

from .common import to64, rope, rope_inv, regions, round_to
from .trees import slot_nodes


def _frontier(nodes, taken, base):
    """Frontier node indices (pre-order) of a slot whose ops start at base."""
    out = []
    if not taken[base]:
        return out
    stack = [0]
    while stack:
        j = stack.pop()
        ch = nodes[j][2]
        if ch and taken[base + 1 + j]:
            stack.extend(reversed(ch))
        else:
            out.append(j)
    return out


def prototype_entry(Ku, Vu, r, a, m, rel, mu, cfg):
    """The packed entry of an internal frontier node covering positions
    [a, a + m) of one (sequence, layer, KV head) ('Inside one cache entry'):
    keys inverse-rotated, averaged and re-rotated at p_rep = a + (m-1)//2;
    value weights (1 - beta) r_i / rel + beta / m (uniform when rel = 0);
    key and value rounded to the cache dtype; ln(mu) as fp32.
    Returns (k, v, lnmu, p_rep)."""
    beta = float(np.float32(cfg.value_base))
    pos = np.arange(a, a + m, dtype=np.float64)
    kt = rope_inv(Ku[a:a + m], pos, cfg.rope_base).mean(axis=0)
    prep = a + (m - 1) // 2
    kh = rope(kt, prep, cfg.rope_base)
    if rel > 0:
        w = (1.0 - beta) * r[a:a + m] / rel + beta / m
    else:
        w = np.full(m, 1.0 / m)
    vh = w @ Vu[a:a + m]
    return round_to(kh, cfg.dtype), round_to(vh, cfg.dtype), float(np.float32(np.log(mu))), prep


def pack(K, V, rel_tok, trees, taken, cu, slots, cfg):
    """K, V: [Ly][H][T][d]; rel_tok float32 [Ly][H][T]; trees: dict with
    float32 node_rel/node_mu [Ly][H][2T] and the uint32 node_topo records
    (absent or None: midpoint trees); taken: uint8 op_taken [Ly][H][2T]
    (tree mode) or [Ly][H][T] (token mode); slots: per sequence.

    Returns dict: K, V float64 [N][d] (values of the cache dtype), lnmu
    float32 [N], pos int32 [N], seg_off int64 [S][Ly][H], seg_len int32.
    """
    Ly, H, T, d = K.shape
    S = len(cu) - 1
    Ks, Vs, lm, ps = [], [], [], []
    seg_off = np.zeros((S, Ly, H), dtype=np.int64)
    seg_len = np.zeros((S, Ly, H), dtype=np.int32)
    n_tot = 0
    tk = taken.reshape(-1)
    for l in range(Ly):
        for h in range(H):
            for s in range(S):
                a0, b0 = int(cu[s]), int(cu[s + 1])
                L = b0 - a0
                pe, c0, c1, ss = regions(L, cfg)
                Ku = to64(K[l, h, a0:b0])
                Vu = to64(V[l, h, a0:b0])
                ents = []          # (k, v, lnmu, pos)

                def tok(i):
                    ents.append((Ku[i], Vu[i], 0.0, i))

                for i in range(0, pe):
                    tok(i)
                if cfg.token_mode:
                    for i in range(c0, c1):
                        if taken[l, h, a0 + i]:
                            tok(i)
                else:
                    r = np.asarray(rel_tok[l, h, a0:b0], dtype=np.float64)
                    for (st, n) in slots[s]:
                        nodes = slot_nodes(trees.get("node_topo"), l, h, a0, st, n)
                        base = (l * H + h) * 2 * T + 2 * (a0 + st)
                        nb = (l * H + h, 2 * (a0 + st))
                        for j in _frontier(nodes, tk, base):
                            a, m = nodes[j][0], nodes[j][1]
                            if m == 1:
                                tok(a)
                                continue
                            rel = float(trees["node_rel"][l, h, nb[1] + j])
                            mu = float(trees["node_mu"][l, h, nb[1] + j])
                            ents.append(prototype_entry(Ku, Vu, r, a, m, rel, mu, cfg))
                for i in range(c1, L):
                    tok(i)
                seg_off[s, l, h] = n_tot
                seg_len[s, l, h] = len(ents)
                n_tot += len(ents)
                for (k, v, lmu, p) in ents:
                    Ks.append(k)
                    Vs.append(v)
                    lm.append(lmu)
                    ps.append(p)
    N = n_tot
    return {"K": np.array(Ks).reshape(N, d), "V": np.array(Vs).reshape(N, d),
            "lnmu": np.array(lm, dtype=np.float32).reshape(N),
            "pos": np.array(ps, dtype=np.int32).reshape(N),
            "seg_off": seg_off, "seg_len": seg_len}
