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
* split_mode 0: binary trees, midpoint split, left child = ceil(n/2) tokens.
  Nodes are numbered in pre-order (children in position order), so a parent
  precedes its children and any set of disjoint nodes is in position order
  when sorted by number.
* split_mode 1 ('Technical details and default settings': tree construction
  weighs high-curvature split candidates beside the midpoint and may isolate
  a salient token in a three-way child set), decided top-down per node
  [st, st+n), n >= 2, before any distortion is known:
  - salient token: i = the first position of the node's largest relevance
    (fp32 values); if n >= 3, the node's relevance S (a left-to-right float64
    sum of the fp32 values) is positive, 2 r_i > S (the token holds more than
    half of it) and i lies at least q = max(floor(n/4), 1) tokens from either
    end, the node splits three ways: [st, i), {i}, [i+1, st+n);
  - otherwise one cut b (left child [st, b)): candidates are every cut that
    leaves both children at least ceil(n/4) tokens, the midpoint among them;
    with the partition's quantized cut scores available (DP slots; the same
    score a slot boundary earns there), the cut with the largest score wins,
    ties to the midpoint, then the cut nearest to it, then the lower one;
    without them (fixed slots) the midpoint.
  Every child has at most n - max(ceil(n/4), 1) tokens (or n - 1 - q), so a
  tree over 128 tokens is at most 15 levels deep. Both decisions are integer
  comparisons or a sum in a fixed order, so every implementation that follows
  them builds the same tree from the same fp32 relevance.
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
  Split(q) gains rel_q D_q - sum_children rel_c D_c; cost = children - 1
  (1 for a binary split, 2 for a three-way one). Utility u = fp32(s_lh *
  gain / cost).

Layout written (the C ABI's tree layout): for the slot starting at token t0
(global token index) of unit (l, h), node j (pre-order, j < m <= 2n-1) lives
at index (l*H + h)*2T + 2*t0 + j of the node arrays; op 0 of the slot is its
Add, op 1+j is Split(node j) (cost 0 for leaves: no such op). node_topo
holds one 32-bit record per node: bits 0-7 the node's first token relative to
the slot, bits 8-15 its length - 1, bits 16-23 its parent's index + 1 (0 for
the root), bits 24-31 the index of its next sibling (0: none); entries past
the slot's last node are 0xFFFFFFFF.
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


TOPO_NONE = 0xFFFFFFFF


def seq_sum(x) -> float:
    """Left-to-right float64 sum (a cumulative sum's last element)."""
    x = np.asarray(x, dtype=np.float64)
    return float(np.cumsum(x)[-1]) if x.size else 0.0


def split_children(st: int, n: int, r, cut_q=None, mode: int = 0):
    """Child intervals [(start, length)] of a node covering sequence
    positions [st, st + n), n >= 2 (readings in the module docstring). r:
    fp32 relevance and cut_q: quantized cut scores (cut before that position),
    both indexed by sequence position; cut_q None without DP slots."""
    b = (n + 1) // 2
    if mode == 0:
        return [(st, b), (st + b, n - b)]
    if n >= 3:
        seg = np.asarray(r[st:st + n], dtype=np.float32)
        i = int(np.argmax(seg))
        S = seq_sum(seg)
        q = max(n // 4, 1)
        if S > 0 and 2.0 * float(seg[i]) > S and q <= i <= n - 1 - q:
            return [(st, i), (st + i, 1), (st + i + 1, n - i - 1)]
    if cut_q is not None:
        m4 = -(-n // 4)
        lo, hi = max(1, m4), min(n - 1, n - m4)
        best, bv = b, int(cut_q[st + b])
        for c in range(lo, hi + 1):
            v = int(cut_q[st + c])
            if v > bv or (v == bv and (abs(c - b), c) < (abs(best - b), best)):
                best, bv = c, v
        b = best
    return [(st, b), (st + b, n - b)]


def slot_tree(st: int, n: int, r=None, cut_q=None, mode: int = 0):
    """Pre-order nodes of one slot as [start, length, children, parent]
    (children: node indices in position order; parent -1 for the root)."""
    out = []

    def rec(a, m, parent):
        j = len(out)
        out.append([a, m, [], parent])
        if m > 1:
            for (ca, cm) in split_children(a, m, r, cut_q, mode):
                out[j][2].append(rec(ca, cm, j))
        return j

    rec(st, n, -1)
    return out


def encode_topo(nodes, st: int, n: int) -> np.ndarray:
    """The node_topo records of one slot (2n entries)."""
    rec = np.full(2 * n, TOPO_NONE, dtype=np.uint32)
    nxt = {}
    for j, (_, _, ch, _) in enumerate(nodes):
        for x, y in zip(ch, ch[1:]):
            nxt[x] = y
    for j, (a, m, ch, p) in enumerate(nodes):
        rec[j] = (a - st) | ((m - 1) << 8) | ((p + 1) << 16) | (nxt.get(j, 0) << 24)
    return rec


def decode_topo(rec, st: int):
    """Nodes [start, length, children, parent] from one slot's records."""
    nodes = []
    for x in np.asarray(rec, dtype=np.uint32):
        x = int(x)
        if x == TOPO_NONE:
            break
        nodes.append([st + (x & 255), ((x >> 8) & 255) + 1, [], ((x >> 16) & 255) - 1])
    for j, nd in enumerate(nodes):
        if nd[3] >= 0:
            nodes[nd[3]][2].append(j)
    return nodes


def slot_nodes(topo, l: int, h: int, a0: int, st: int, n: int):
    """The nodes of one slot: from node_topo [Ly][H][2T] when given, else
    the midpoint tree."""
    if topo is None:
        return slot_tree(st, n)
    b = 2 * (a0 + st)
    return decode_topo(topo[l, h, b:b + 2 * n], st)


def _slot(ktil, knorm, V, r, Ad, Qd, lse_d, a, n, pos0, cfg, rope_base):
    """One midpoint-split slot [a, a+n): (tree_nodes(a, n), rel, D, mu, khat,
    vhat), see _slot_nodes."""
    out = _slot_nodes(slot_tree(a, n), ktil, knorm, V, r, Ad, Qd, lse_d, pos0, cfg, rope_base)
    return (tree_nodes(a, n),) + out


def _slot_nodes(nodes, ktil, knorm, V, r, Ad, Qd, lse_d, pos0, cfg, rope_base):
    """One slot with the given nodes. ktil/knorm/V/r/Ad are unit arrays
    indexed by position within the sequence; returns per-node (rel, D, mu,
    khat, vhat)."""
    m = len(nodes)
    rel = np.zeros(m)
    # bottom-up value flow: leaves hold r_i, a parent sums its children
    for j in range(m - 1, -1, -1):
        st, ln, ch, _ = nodes[j]
        rel[j] = r[st] if not ch else sum(rel[c] for c in ch)
    d = V.shape[1]
    c = 1.0 / np.sqrt(d)
    beta = float(np.float32(cfg.value_base))
    wA, wV = float(np.float32(cfg.w_attn)), float(np.float32(cfg.w_value))
    D = np.zeros(m)
    mu = np.ones(m)
    khat = np.zeros((m, d))
    vhat = np.zeros((m, d))
    for j, (st, ln, ch, _) in enumerate(nodes):
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
        if not ch:
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
    return rel, D, mu, khat, vhat


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
    node j by its children and gains rel_j D_j - sum_c rel_c D_c; Add adds one
    entry, a split (children - 1). util = fp32(sens * gain / cost)."""
    m = len(nodes)
    util = np.zeros(m + 1, dtype=np.float32)
    cost = np.zeros(m + 1, dtype=np.uint8)
    util[0] = np.float32(sens * (rel[0] * (1.0 - D[0])))
    cost[0] = 1
    for j, (_, _, ch, _) in enumerate(nodes):
        if not ch:
            continue
        gain = rel[j] * D[j] - sum(rel[c] * D[c] for c in ch)
        util[1 + j] = np.float32(sens * gain / float(len(ch) - 1))
        cost[1 + j] = len(ch) - 1
    return util, cost


def build_trees(K, V, Qp, lse, rel_tok, head_sens, cu, slots, cfg, keep_protos=False, cut_q=None, topo=None):
    """Build every tree. K, V: [Ly][H][T][d]; Qp: [S][Ly][H*G][P][d];
    lse: float32 [S][Ly][H*G][P]; rel_tok, head_sens: float32; slots: per
    sequence [(start, n)]; cut_q: the partition's int64 [T] cut scores (DP
    slots, split_mode 1) or None; topo: node_topo records [Ly][H][2T] whose
    shapes are used instead of deciding them (None: decide them).

    Returns float32 node_rel/node_D/node_mu and op_util [Ly][H][2T], uint8
    op_cost [Ly][H][2T], uint32 node_topo [Ly][H][2T]; with keep_protos, also
    a dict of per-slot prototype arrays keyed by (s, l, h, slot_start).
    """
    Ly, H, T, d = K.shape
    G, P = cfg.G, cfg.P
    rows = dprobe_rows(cfg)
    node_rel = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    node_D = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    node_mu = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    op_util = np.zeros((Ly, H, 2 * T), dtype=np.float32)
    op_cost = np.zeros((Ly, H, 2 * T), dtype=np.uint8)
    node_topo = np.full((Ly, H, 2 * T), TOPO_NONE, dtype=np.uint32)
    mode = int(getattr(cfg, "split_mode", 0))
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
                r32 = np.asarray(rel_tok[l, h, a0:b0], dtype=np.float32)
                r = r32.astype(np.float64)
                cq = None if cut_q is None else np.asarray(cut_q[a0:b0])
                sens = float(head_sens[s, l, h])
                for (st, n) in slots[s]:
                    nodes = (slot_tree(st, n, r32, cq, mode) if topo is None
                             else decode_topo(topo[l, h, 2 * (a0 + st):2 * (a0 + st) + 2 * n], st))
                    rel, D, mu, kh, vh = _slot_nodes(nodes, ktil, knorm, Vu, r, Ad, Q, ls, 0, cfg, cfg.rope_base)
                    base = 2 * (a0 + st)
                    m = len(nodes)
                    node_topo[l, h, base:base + 2 * n] = encode_topo(nodes, st, n)
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
            "op_util": op_util, "op_cost": op_cost, "node_topo": node_topo, "protos": protos}
