"""Budget spending: singleton floor, global Add/Split auction, token top-B.

Test infrastructure only (see the package docstring).

Sources:
* GraceKV page, 'Exact-information safeguard' and 'Technical details and
  default settings' (singleton floor): before the auction, a budget-capped set
  of high-value (layer, KV head, token) leaves is isolated; each realized
  singleton pays its complete tree path and shared ancestors are paid once;
  the cap is a hard maximum.
* GraceKV page, '04 Top-down budget flow': every feasible Add and Split sits
  in one global queue; the highest affordable marginal utility wins next.
  'Core idea': greedy solution, not exact global optimality.
* DistillCache paper, Sec. 3.1.2 and Algorithm 1: at inference the top-B
  tokens by score are kept deterministically (token-level mode).

Readings:
* Floor: F = floor(phi * allocatable budget). Candidates are the compressible
  leaves ordered by fp32(s_lh * r_i) descending, then flat id
  (l*H + h)*T + token ascending; the first F are scanned in that order, each
  paying the costs of the not-yet-taken operations on its root-to-leaf path
  and accepted if the floor spend stays <= F.
* Auction: best-first over the operation forest: every exposed operation is in
  a max-queue keyed by (utility, lower op id first); popping an affordable
  operation takes it and exposes the operations of the nodes it creates. The
  queue runs until the budget is spent or it is empty, so it fills the budget
  even with non-positive utilities. A NaN utility counts as -infinity.
* Token mode: the first B_alloc compressible tokens of the sequence by
  (r descending, flat id ascending).
* Head-level hybrid (DistillCache paper, Appendix E.3): per sequence the K
  units (l, h) with the largest head sensitivity s_lh (the probe pass's
  attention statistic; ties to the lower unit index l*H + h) keep every
  compressible token: in tree mode all their Add and Split operations are
  taken, in token mode all their tokens. K and the remaining budget come
  from common.budgets; the floor, the auction and the token top-B then run
  over the other units only.
"""
from __future__ import annotations

import heapq

import numpy as np

from .common import regions, budgets
from .trees import slot_nodes


def _f32key(x) -> float:
    v = float(x)
    return -np.inf if v != v else v


def _slot_ops(T, H, l, h, t0):
    return (l * H + h) * 2 * T + 2 * t0


def _leaf_path(nodes, i):
    """Internal node indices on the path from the root to the leaf of token i
    (nodes as [start, length, children, parent])."""
    path, j = [], 0
    while nodes[j][2]:
        path.append(j)
        j = next(c for c in nodes[j][2] if nodes[c][0] <= i < nodes[c][0] + nodes[c][1])
    return path


def hybrid_units(head_sens, cu, cfg):
    """Units kept whole: bool [S][Ly][H] (all False when hybrid_frac = 0)."""
    S = len(cu) - 1
    Ly, H = cfg.Ly, cfg.H
    full = np.zeros((S, Ly, H), dtype=bool)
    bud = budgets([int(cu[s + 1] - cu[s]) for s in range(S)], cfg)
    for s in range(S):
        K = bud[s]["full_units"]
        order = sorted(range(Ly * H), key=lambda u: (-_f32key(head_sens[s].reshape(-1)[u]), u))
        for u in order[:K]:
            full[s, u // H, u % H] = True
    return full


def floor_select(rel_tok, head_sens, op_cost, cu, slots, cfg, trace=None, full=None, topo=None):
    """Returns op_taken uint8 [Ly][H][2T] (floor ops only) and spent [S].
    If ``trace`` is a list, accepted candidates are appended as
    (leaf flat id, path cost paid). ``full`` [S][Ly][H] excludes the units
    kept whole by the head-level hybrid. ``topo``: the trees' node_topo
    (None: midpoint trees)."""
    Ly, H, T2 = op_cost.shape
    T = T2 // 2
    taken = np.zeros((Ly, H, 2 * T), dtype=np.uint8)
    cost = op_cost.reshape(-1)
    tk = taken.reshape(-1)
    bud = budgets([int(cu[s + 1] - cu[s]) for s in range(len(cu) - 1)], cfg)
    spent = np.zeros(len(cu) - 1, dtype=np.int64)
    for s in range(len(cu) - 1):
        F = bud[s]["floor"]
        if F <= 0 or not slots[s]:
            continue
        a0 = int(cu[s])
        cands = []
        for l in range(Ly):
            for h in range(H):
                if full is not None and full[s, l, h]:
                    continue
                sens = np.float64(head_sens[s, l, h])
                for (st, n) in slots[s]:
                    nodes = slot_nodes(topo, l, h, a0, st, n)
                    base = _slot_ops(T, H, l, h, a0 + st)
                    for i in range(st, st + n):
                        v = np.float32(sens * np.float64(rel_tok[l, h, a0 + i]))
                        fid = (l * H + h) * T + a0 + i
                        ops = [base] + [base + 1 + j for j in _leaf_path(nodes, i)]
                        cands.append((-_f32key(v), fid, ops))
        cands.sort(key=lambda c: (c[0], c[1]))
        for _, fid, ops in cands[:F]:
            c = sum(int(cost[o]) for o in ops if not tk[o])
            if spent[s] + c <= F:
                for o in ops:
                    tk[o] = 1
                spent[s] += c
                if trace is not None:
                    trace.append((fid, c))
    return taken, spent


def auction(op_util, op_cost, floor_taken, spent_floor, cu, slots, cfg, trace=None, full=None, topo=None):
    """Best-first greedy over every exposed op of each sequence.

    Returns op_taken uint8 [Ly][H][2T] (floor ops included) and spent [S]
    (floor + auction entries, and the units kept whole). If ``trace`` is a
    list, the taken ops are appended to it in the order the queue pops them.
    ``full`` [S][Ly][H]: units kept whole (every real op taken up front).
    ``topo``: the trees' node_topo (None: midpoint trees). An op that costs
    more than what is left is dropped (its subtree never becomes exposed) and
    the queue goes on."""
    Ly, H, T2 = op_util.shape
    T = T2 // 2
    taken = floor_taken.copy().reshape(-1)
    util = op_util.reshape(-1)
    cost = op_cost.reshape(-1)
    bud = budgets([int(cu[s + 1] - cu[s]) for s in range(len(cu) - 1)], cfg)
    spent = np.asarray(spent_floor, dtype=np.int64).copy()
    for s in range(len(cu) - 1):
        if not slots[s]:
            continue
        a0 = int(cu[s])
        if full is not None:
            for l in range(Ly):
                for h in range(H):
                    if not full[s, l, h]:
                        continue
                    for (st, n) in slots[s]:
                        base = _slot_ops(T, H, l, h, a0 + st)
                        for o in range(base, base + 2 * n):
                            if cost[o] > 0 and not taken[o]:
                                taken[o] = 1
                                spent[s] += int(cost[o])
        rem = bud[s]["alloc"] - int(spent[s])
        heap = []
        children = {}   # op id -> list of op ids it exposes

        def push(o):
            heapq.heappush(heap, (-_f32key(util[o]), o))

        for l in range(Ly):
            for h in range(H):
                for (st, n) in slots[s]:
                    nodes = slot_nodes(topo, l, h, a0, st, n)
                    base = _slot_ops(T, H, l, h, a0 + st)
                    split = lambda j: base + 1 + j  # noqa: E731
                    children[base] = [split(0)] if nodes[0][2] else []
                    for j, (_, _, ch, _) in enumerate(nodes):
                        if ch:
                            children[split(j)] = [split(c) for c in ch if nodes[c][2]]
                    # exposed ops given the floor's choices
                    stack = [base]
                    while stack:
                        o = stack.pop()
                        if taken[o]:
                            stack.extend(children[o])
                        else:
                            push(o)
        while heap and rem > 0:
            _, o = heapq.heappop(heap)
            c = int(cost[o])
            if c > rem:
                continue
            taken[o] = 1
            rem -= c
            spent[s] += c
            if trace is not None:
                trace.append(o)
            for ch in children[o]:
                push(ch)
    return taken.reshape(Ly, H, 2 * T), spent


def token_topk(rel_tok, cu, cfg, full=None):
    """Token-level mode: returns taken uint8 [Ly][H][T] and spent [S].
    ``full`` [S][Ly][H]: units kept whole by the head-level hybrid."""
    Ly, H, T = rel_tok.shape
    taken = np.zeros((Ly, H, T), dtype=np.uint8)
    bud = budgets([int(cu[s + 1] - cu[s]) for s in range(len(cu) - 1)], cfg)
    spent = np.zeros(len(cu) - 1, dtype=np.int64)
    for s in range(len(cu) - 1):
        a0, b0 = int(cu[s]), int(cu[s + 1])
        pe, c0, c1, ss = regions(b0 - a0, cfg)
        keys = []
        whole = 0
        for l in range(Ly):
            for h in range(H):
                if full is not None and full[s, l, h]:
                    taken[l, h, a0 + c0:a0 + c1] = 1
                    whole += c1 - c0
                    continue
                for i in range(c0, c1):
                    keys.append((-_f32key(rel_tok[l, h, a0 + i]), (l * H + h) * T + a0 + i, l, h, i))
        keys.sort(key=lambda k: (k[0], k[1]))
        k = max(0, min(bud[s]["alloc"] - whole, len(keys)))
        for _, _, l, h, i in keys[:k]:
            taken[l, h, a0 + i] = 1
        spent[s] = k + whole
    return taken, spent
