"""Prototype trees per (sequence, layer, KV head, slot).

Test infrastructure only (see the package docstring).

Sources (GraceKV page):
* '02 Progressively refinable representation': every (layer, KV head, slot)
  owns a prototype tree; a frontier (non-overlapping node set) states how the
  slot is stored: nothing, the root, finer nodes, or every token leaf.
* 'Inside one cache entry': keys are inverse-rotated, averaged in a shared
  frame and re-rotated at a representative position; values are weighted by
  relevance with a 10% uniform base; a multiplicity from key coherence keeps
  incoherent merges from drawing too much attention.
* '03 Bottom-up value flow': a parent's value is the sum of its children's.
* 'Technical details and default settings' (prototype fidelity): a
  probe-based distortion weighs attention-partition error and value-aggregate
  error at 0.25 : 0.75.
* '04 Top-down budget flow': Add (cover an absent slot with its root) and
  Split (replace a node with its children) are priced as
  relevance x fidelity gain x head sensitivity / new physical entries.

Readings (the pages give no formulas):
* Binary trees, midpoint split, left child = ceil(n/2) tokens. Nodes are
  numbered in pre-order, so a parent precedes its children and any set of
  disjoint nodes is in position order when sorted by number.
* Representative position p_rep = a + floor((n-1)/2); unweighted key mean in
  the unrotated frame.
* v_hat = sum_i ((1-beta) r_i/rel + beta/n) v_i, beta = 0.1; uniform if rel = 0.
* Multiplicity mu = max(1, n * rho), rho = ||sum k~_i|| / sum ||k~_i|| (1 if
  the denominator is 0); decode adds ln(mu) to the prototype's logit.
* Distortion over the P_d = min(n_dprobe, G*P) probe rows with index
  rho = g*P + p divisible by G*P/P_d, with a_rho,i = exp(c<q_rho,k_i> - lse_rho):
    Z = sum_node a,   Z_hat = mu * exp(c<q_rho, k_hat> - lse_rho),
    u = sum_node a_i v_i,
    e_A = sum_rho |Z_hat - Z| / sum_rho Z,
    e_V = sum_rho ||u - Z v_hat|| / sum_rho ||u||,
    D = min(1, 0.25 e_A + 0.75 e_V); a leaf has D = 0; 0/0 counts as 0.
* Fidelity gain: Add gains rel_root (1 - D_root) (dropping counts as D = 1);
  Split(q) gains rel_q D_q - sum_children rel_c D_c; cost = children - 1.
  Utility u = fp32(s_lh * gain / cost).

Layout written (the C ABI's tree layout): for the slot starting at token t0
(global token index) of unit (l, h), node j (pre-order, j < 2n-1) lives at
index (l*H + h)*2T + 2*t0 + j of the node arrays; op 0 of the slot is its
Add, op 1+j is Split(node j) (cost 0 for leaves: no such op).
"""
from __future__ import annotations

import numpy as np

from .common import to64, rope, rope_inv


def tree_nodes(a: int, n: int):
    """Pre-order list of (start, length, left_index, right_index); -1 = leaf."""
    out = []

    def rec(st, m):
        j = len(out)
        out.append([st, m, -1, -1])
        if m > 1:
            nl = (m + 1) // 2
            out[j][2] = rec(st, nl)
            out[j][3] = rec(st + nl, m - nl)
        return j

    rec(a, n)
    return out


def _slot(ktil, knorm, V, r, Ad, Qd, lse_d, a, n, pos0, cfg, rope_base):
    """One slot. ktil/knorm/V/r/Ad are unit arrays indexed by position within
    the sequence; returns per-node (rel, D, mu, khat, vhat) and the nodes."""
    nodes = tree_nodes(a, n)
    m = len(nodes)
    rel = np.zeros(m)
    # bottom-up value flow: leaves hold r_i, a parent sums its two children
    for j in range(m - 1, -1, -1):
        st, ln, lc, rc = nodes[j]
        rel[j] = r[st] if lc < 0 else rel[lc] + rel[rc]
    d = V.shape[1]
    c = 1.0 / np.sqrt(d)
    beta = float(np.float32(cfg.value_base))
    wA, wV = float(np.float32(cfg.w_attn)), float(np.float32(cfg.w_value))
    D = np.zeros(m)
    mu = np.ones(m)
    khat = np.zeros((m, d))
    vhat = np.zeros((m, d))
    for j, (st, ln, lc, rc) in enumerate(nodes):
        sl = slice(st, st + ln)
        skt = ktil[sl].sum(axis=0)
        sn = knorm[sl].sum()
        rho = np.sqrt((skt * skt).sum()) / sn if sn > 0 else 1.0
        mu[j] = max(1.0, ln * rho)
        prep = st + (ln - 1) // 2
        khat[j] = rope(skt / ln, pos0 + prep, rope_base)
        if rel[j] > 0:
            w = (1.0 - beta) * r[sl] / rel[j] + beta / ln
        else:
            w = np.full(ln, 1.0 / ln)
        vhat[j] = w @ V[sl]
        if lc < 0:
            continue
        A = Ad[:, sl]                                      # [P_d, n]
        Z = A.sum(axis=1)
        Zh = mu[j] * np.exp(c * (Qd @ khat[j]) - lse_d)
        u = A @ V[sl]                                      # [P_d, d]
        num_a, den_a = np.abs(Zh - Z).sum(), Z.sum()
        eA = num_a / den_a if den_a > 0 else 0.0
        num_v = np.sqrt(((u - Z[:, None] * vhat[j][None, :]) ** 2).sum(axis=1)).sum()
        den_v = np.sqrt((u * u).sum(axis=1)).sum()
        eV = num_v / den_v if den_v > 0 else 0.0
        D[j] = min(1.0, wA * eA + wV * eV)
    return nodes, rel, D, mu, khat, vhat


def dprobe_rows(cfg):
    """Probe rows of the distortion: P_d = min(n_dprobe, G*P) rows, every
    (G*P // P_d)-th row index rho = g*P + p starting at 0."""
    R = cfg.G * cfg.P
    Pd = min(cfg.n_dprobe, R)
    stride = R // Pd
    return np.arange(0, R, stride)[:Pd]


def op_utilities(nodes, rel, D, sens):
    """Operations of one slot and their utilities ('04 Top-down budget flow':
    relevance x fidelity gain x head sensitivity per new physical entry).

    Returns (util, cost) over the slot's 2n op indices: op 0 = Add(slot),
    op 1 + j = Split(node j) for internal j (cost 0 marks "no such op": the
    leaves). Gains: Add covers the absent slot with its root, so it gains
    rel_root (1 - D_root) (an absent slot counts as D = 1); Split(j) replaces
    node j by its children and gains rel_j D_j - sum_c rel_c D_c; every op
    adds (children - 1) = 1 entry. util = fp32(sens * gain / cost)."""
    m = len(nodes)
    util = np.zeros(m + 1, dtype=np.float32)
    cost = np.zeros(m + 1, dtype=np.uint8)
    util[0] = np.float32(sens * (rel[0] * (1.0 - D[0])))
    cost[0] = 1
    for j, (_, _, lc, rc) in enumerate(nodes):
        if lc < 0:
            continue
        gain = rel[j] * D[j] - (rel[lc] * D[lc] + rel[rc] * D[rc])
        util[1 + j] = np.float32(sens * gain / 1.0)
        cost[1 + j] = 1
    return util, cost


def build_trees(K, V, Qp, lse, rel_tok, head_sens, cu, slots, cfg, keep_protos=False):
    """Build every tree. K, V: [Ly][H][T][d]; Qp: [S][Ly][H*G][P][d];
    lse: float32 [S][Ly][H*G][P]; rel_tok, head_sens: float32; slots: per
    sequence [(start, n)].

    Returns float32 node_rel/node_D/node_mu and op_util [Ly][H][2T], uint8
    op_cost [Ly][H][2T]; with keep_protos, also a dict of per-slot prototype
    arrays keyed by (s, l, h, slot_start).
    """
    Ly, H, T, d = K.shape
    G, P = cfg.G, cfg.P
    rows = dprobe_rows(cfg)
    node_rel = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    node_D = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    node_mu = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    op_util = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    op_cost = np.zeros((Ly, H, 2 * T), dtype=np.uint8)
    protos = {}
    for s in range(len(cu) - 1):
        a0, b0 = int(cu[s]), int(cu[s + 1])
        L = b0 - a0
        if L == 0 or not slots[s]:
            continue
        for l in range(Ly):
            for h in range(H):
                Ku = to64(K[l, h, a0:b0])
                Vu = to64(V[l, h, a0:b0])
                pos = np.arange(L, dtype=np.float64)
                ktil = rope_inv(Ku, pos, cfg.rope_base)
                knorm = np.sqrt((ktil * ktil).sum(axis=1))
                Q = to64(Qp[s, l, h * G:(h + 1) * G]).reshape(G * P, d)[rows]
                ls = np.asarray(lse[s, l, h * G:(h + 1) * G], dtype=np.float64).reshape(G * P)[rows]
                c = 1.0 / np.sqrt(d)
                Ad = np.exp(c * (Q @ Ku.T) - ls[:, None])          # [P_d, L]
                r = np.asarray(rel_tok[l, h, a0:b0], dtype=np.float64)
                sens = float(head_sens[s, l, h])
                for (st, n) in slots[s]:
                    nodes, rel, D, mu, kh, vh = _slot(ktil, knorm, Vu, r, Ad, Q, ls, st, n, 0,
                                                      cfg, cfg.rope_base)
                    base = 2 * (a0 + st)
                    m = len(nodes)
                    node_rel[l, h, base:base + m] = rel
                    node_D[l, h, base:base + m] = D
                    node_mu[l, h, base:base + m] = mu
                    u, cst = op_utilities(nodes, rel, D, sens)
                    op_util[l, h, base:base + m + 1] = u
                    op_cost[l, h, base:base + m + 1] = cst
                    if keep_protos:
                        protos[(s, l, h, st)] = {"nodes": nodes, "khat": kh, "vhat": vh,
                                                 "mu": mu, "rel": rel, "D": D}
    return {"node_rel": node_rel, "node_D": node_D, "node_mu": node_mu,
            "op_util": op_util, "op_cost": op_cost, "protos": protos}
