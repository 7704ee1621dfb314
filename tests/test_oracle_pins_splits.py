"""Pins of the oracle's curvature-candidate and salient three-way splits
(split_mode 1; GraceKV page, 'Technical details and default settings': tree
construction weighs high-curvature split candidates beside the midpoint and
may isolate a salient token in a three-way child set), with slips planted in
the oracle (monkeypatch) to show that the pins fail when the slip is there.

Pinned here:
* the topology rule on hand-built cases whose trees are written out by hand
  (salient token in and out of the middle window, exactly half of the node's
  relevance, the strongest cut, ties to the midpoint and then to the lower
  cut, cuts outside the window ignored, no cut scores = midpoint);
* invariants over random relevance and cut scores: children partition their
  parent in position order, pre-order numbering, at most 2n - 1 nodes, the
  depth bound, and the 32-bit node records round-tripping;
* utilities of three-way splits (cost 2) as the frontier loss decrease per
  new entry;
* the greedy auction with cost-2 operations against the page's greedy
  enumerated literally, and the threshold form the GPU library computes
  (weighted select, best-first walk of the tied group skipping what does not
  fit, then the best affordable exposed operation) against the same;
* the floor paying a three-way split's two entries once;
* pack's frontier: every reachable frontier of a three-way tree stores one
  entry per budget unit spent, in position order, covering the slot.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import trees as otrees, select as osel
from oracle.pack import _frontier
from workload import Config, small_config, make_inputs


def _cfg(**kw):
    base = dict(name="t", S=1, Ly=1, H=1, G=2, d=8, lens=[16], dtype="f32", rope_base=1e4,
                P=4, slot_len=8, T_dec=1, vocab=64, w_dtype="f32", plant="evidence", n_plant=0,
                split_mode=1)
    base.update(kw)
    return Config(**base)


def _shape(nodes):
    """(start, length, children) per node, as plain tuples."""
    return [(a, m, tuple(ch)) for a, m, ch, _ in nodes]


# ================================================================ topology, by hand
def check_topology_by_hand():
    f32 = lambda x: np.asarray(x, dtype=np.float32)  # noqa: E731
    # A: the salient token 3 holds more than half and sits in the middle
    # window [2, 5] of the 8-token root: three-way root; its sides split at
    # their midpoints
    r = f32([.1, .1, .1, 5, .1, .1, .1, .1])
    want = [(0, 8, (1, 6, 7)), (0, 3, (2, 5)), (0, 2, (3, 4)), (0, 1, ()), (1, 1, ()), (2, 1, ()),
            (3, 1, ()), (4, 4, (8, 11)), (4, 2, (9, 10)), (4, 1, ()), (5, 1, ()), (6, 2, (12, 13)),
            (6, 1, ()), (7, 1, ())]
    assert _shape(otrees.slot_tree(0, 8, r, None, 1)) == want
    # B: exactly half of the relevance is not more than half: midpoint tree
    r = f32([1, 1, 1, 3, 0, 0, 0, 0])
    assert _shape(otrees.slot_tree(0, 8, r, None, 1)) == _shape(otrees.slot_tree(0, 8))
    # C: salient token 1 is outside the root's window (q = 2) but inside the
    # window of the left child [0, 4) (q = 1)
    r = f32([.1, 5, .1, .1, .1, .1, .1, .1])
    want = [(0, 8, (1, 7)), (0, 4, (2, 3, 4)), (0, 1, ()), (1, 1, ()), (2, 2, (5, 6)), (2, 1, ()),
            (3, 1, ()), (4, 4, (8, 11)), (4, 2, (9, 10)), (4, 1, ()), (5, 1, ()), (6, 2, (12, 13)),
            (6, 1, ()), (7, 1, ())]
    assert _shape(otrees.slot_tree(0, 8, r, None, 1)) == want
    # E: five tokens, salient token 1 (q = 1): three-way [0,1), {1}, [2,5)
    r = f32([.1, 5, .1, .1, .1])
    got = _shape(otrees.slot_tree(0, 5, r, None, 1))
    assert got[0] == (0, 5, (1, 2, 3))
    assert got[3] == (2, 3, (4, 7))
    # D: cut scores (cut before that position). 8-token root, window of cuts
    # [2, 6], midpoint 4: the strongest cut 2 wins; the score 100 at 1 lies
    # outside the window
    zero = f32(np.zeros(8))
    cq = np.array([0, 100, 7, 3, 3, 3, 3, 3], dtype=np.int64)
    got = _shape(otrees.slot_tree(0, 8, zero, cq, 1))
    assert got[0][2] and got[1][:2] == (0, 2)
    # ... then [2, 8) (6 tokens, window of cuts 4..6, midpoint 5): all 3 -> midpoint 5
    j = got[0][2][1]
    assert got[j][:2] == (2, 6)
    assert got[got[j][2][0]][:2] == (2, 3)
    # ties away from the midpoint go to the nearest cut, then the lower one
    cq = np.array([0, 0, 0, 9, 0, 9, 0, 0], dtype=np.int64)
    got = _shape(otrees.slot_tree(0, 8, zero, cq, 1))
    assert got[1][:2] == (0, 3)
    cq = np.array([0, 0, 9, 0, 9, 0, 9, 0], dtype=np.int64)       # the midpoint 4 ties: it wins
    got = _shape(otrees.slot_tree(0, 8, zero, cq, 1))
    assert got[1][:2] == (0, 4)
    # D2: six tokens, window of cuts [2, 4] (ceil(6/4) = 2): a strong cut at 1 is ignored
    cq = np.array([0, 50, 0, 0, 0, 0], dtype=np.int64)
    got = _shape(otrees.slot_tree(0, 6, f32(np.zeros(6)), cq, 1))
    assert got[1][:2] == (0, 3)
    # the salient rule comes before the cut scores
    r = f32([.1, .1, .1, 5, .1, .1, .1, .1])
    cq = np.array([0, 0, 99, 0, 0, 0, 0, 0], dtype=np.int64)
    assert _shape(otrees.slot_tree(0, 8, r, cq, 1))[0] == (0, 8, (1, 6, 7))
    # sequence offsets: a slot starting at 5 uses r and cut scores at its own positions
    rr = np.concatenate([f32([9, 9, 9, 9, 9]), f32([.1, .1, .1, 5, .1, .1, .1, .1])])
    assert _shape(otrees.slot_tree(5, 8, rr, None, 1))[0] == (5, 8, (1, 6, 7))


def test_topology_by_hand():
    check_topology_by_hand()


def test_mode0_slot_tree_is_the_midpoint_tree():
    for n in list(range(1, 20)) + [64, 127, 128]:
        legacy = otrees.tree_nodes(3, n)
        got = otrees.slot_tree(3, n)
        for (a, m, lc, rc), (b, k, ch, _) in zip(legacy, got):
            assert (a, m) == (b, k)
            assert tuple(ch) == ((lc, rc) if lc >= 0 else ())
        assert len(legacy) == len(got)


# ================================================================ topology, invariants
def _depth_bound(n):
    d = 0
    while n > 1:
        n -= max(-(-n // 4), 1)
        d += 1
    return d


def test_topology_invariants_random():
    rng = np.random.default_rng(5)
    assert _depth_bound(128) == 14
    for trial in range(300):
        n = int(rng.integers(1, 129))
        kind = trial % 3
        if kind == 0:
            r = rng.random(n)
        elif kind == 1:
            r = rng.random(n) ** 8 * 10.0 ** rng.integers(-3, 3, n)   # heavy tails: salient tokens
        else:
            r = np.zeros(n)
            r[rng.integers(0, n)] = 1.0
        r = r.astype(np.float32)
        cq = rng.integers(0, 1 << 22, n).astype(np.int64) if trial % 2 else None
        nodes = otrees.slot_tree(0, n, r, cq, 1)
        assert len(nodes) <= 2 * n - 1
        depth = {0: 0}
        for j, (a, m, ch, p) in enumerate(nodes):
            if p >= 0:
                assert p < j and j in nodes[p][2]
                depth[j] = depth[p] + 1
            if ch:
                assert len(ch) in (2, 3)
                assert nodes[ch[0]][0] == a and ch[0] == j + 1
                assert sum(nodes[c][1] for c in ch) == m
                for x, y in zip(ch, ch[1:]):
                    assert nodes[x][0] + nodes[x][1] == nodes[y][0]
                if len(ch) == 3:
                    assert nodes[ch[1]][1] == 1
                assert max(nodes[c][1] for c in ch) <= m - max(-(-m // 4), 1)
            else:
                assert m == 1
        assert max(depth.values()) <= _depth_bound(n)
        leaves = sorted(a for a, m, ch, _ in nodes if not ch)
        assert leaves == list(range(n))
        rec = otrees.encode_topo(nodes, 0, n)
        assert rec.shape == (2 * n,) and np.all(rec[len(nodes):] == otrees.TOPO_NONE)
        assert _shape(otrees.decode_topo(rec, 0)) == _shape(nodes)


# ================================================================ utilities
def _build_split_trees(seed):
    """One sequence, one unit, slots of 8/13/5/16 tokens, with salient tokens
    and cut scores, so three-way and off-midpoint splits both occur."""
    cfg = _cfg(lens=[42], slot_len=0)
    rng = np.random.default_rng(seed)
    T, d = 42, 8
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    r = rng.random(T) * 0.1
    r[[3, 12, 23, 30, 37]] = [4.0, 2.0, 3.0, 5.0, 1.5]
    Qp = rng.standard_normal((1, 1, cfg.G, cfg.P, d))
    lse = np.log(T) + rng.random((1, 1, cfg.G, cfg.P))
    slots = [[(0, 8), (8, 13), (21, 5), (26, 16)]]
    cq = rng.integers(0, 1 << 20, T).astype(np.int64)
    sens = np.array([[[1.3]]], dtype=np.float32)
    out = otrees.build_trees(torch.from_numpy(K[None, None]), torch.from_numpy(V[None, None]),
                             torch.from_numpy(Qp), np.float32(lse), np.float32(r[None, None]), sens,
                             np.array([0, T]), slots, cfg, cut_q=cq)
    return cfg, slots, sens, out, r.astype(np.float32), cq


def check_split_utilities(seed):
    cfg, slots, sens, out, r, cq = _build_split_trees(seed)
    s = float(sens[0, 0, 0])
    n3 = 0
    for (st, n) in slots[0]:
        nodes = otrees.decode_topo(out["node_topo"][0, 0, 2 * st:2 * st + 2 * n], st)
        assert _shape(nodes) == _shape(otrees.slot_tree(st, n, r, cq, 1))
        m = len(nodes)
        rel = out["node_rel"][0, 0, 2 * st:2 * st + m].astype(np.float64)
        D = out["node_D"][0, 0, 2 * st:2 * st + m].astype(np.float64)
        util = out["op_util"][0, 0, 2 * st:2 * st + 2 * n]
        cost = out["op_cost"][0, 0, 2 * st:2 * st + 2 * n]

        def loss(fr):
            return s * rel[0] if fr is None else sum(s * rel[j] * D[j] for j in fr)

        def near(u, before, after, c):
            tol = 4e-7 * (abs(before) + abs(after)) + 1e-12
            return abs(float(u) * c - (before - after)) <= tol + abs(float(u)) * c * 2 ** -23

        assert cost[0] == 1 and near(util[0], loss(None), loss([0]), 1)
        assert int(cost.sum()) == n          # every op taken stores the n leaves
        for j, (_, _, ch, p) in enumerate(nodes):
            if not ch:
                assert cost[1 + j] == 0
                continue
            fr, a = [j], j
            while nodes[a][3] >= 0:
                q = nodes[a][3]
                fr += [c for c in nodes[q][2] if c != a]
                a = q
            after = [x for x in fr if x != j] + list(ch)
            assert cost[1 + j] == len(ch) - 1
            n3 += len(ch) == 3
            assert near(util[1 + j], loss(fr), loss(after), len(ch) - 1), (st, j)
    assert n3 >= 2
    return n3


def test_split_utilities_are_the_frontier_loss_decrease_per_entry():
    for seed in range(3):
        check_split_utilities(seed)


# ================================================================ auction with cost-2 operations
def _random_topology(rng, st, n):
    """Random pre-order nodes over [st, st+n): every internal node splits in
    two or three position-ordered parts (three only with a single-token middle)."""
    out = []

    def rec(a, m, p):
        j = len(out)
        out.append([a, m, [], p])
        if m > 1:
            if m >= 3 and rng.random() < 0.4:
                i = int(rng.integers(1, m - 1))
                parts = [(a, i), (a + i, 1), (a + i + 1, m - i - 1)]
            else:
                b = int(rng.integers(1, m))
                parts = [(a, b), (a + b, m - b)]
            for ca, cm in parts:
                out[j][2].append(rec(ca, cm, j))
        return j

    rec(st, n, -1)
    return out


def _forest(rng, n_slots, ties):
    lens = rng.integers(1, 10, n_slots).tolist()
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    T = int(sum(lens))
    util = np.zeros(2 * T, dtype=np.float32)
    cost = np.zeros(2 * T, dtype=np.uint8)
    topo = np.full((1, 1, 2 * T), otrees.TOPO_NONE, dtype=np.uint32)
    slots_ops = []
    draw = (lambda: rng.integers(0, 4)) if ties else (lambda: rng.standard_normal())
    for st, n in zip(starts, lens):
        nodes = _random_topology(rng, st, n)
        topo[0, 0, 2 * st:2 * st + 2 * n] = otrees.encode_topo(nodes, st, n)
        base = 2 * st
        slots_ops.append((base, nodes))
        util[base], cost[base] = draw(), 1
        for j, nd in enumerate(nodes):
            if nd[2]:
                util[base + 1 + j], cost[base + 1 + j] = draw(), len(nd[2]) - 1
    return lens, starts, T, util, cost, topo, slots_ops


def _creator(base, nodes, o):
    if o == base:
        return None
    j = o - base - 1
    return base if j == 0 else base + 1 + nodes[j][3]


def _ops(base, nodes):
    return [base] + [base + 1 + j for j, nd in enumerate(nodes) if nd[2]]


def _greedy_enumerated(util, cost, taken0, slots_ops, rem):
    """The page's greedy stated literally: each round enumerates the exposed
    ops and takes the highest-utility one that still fits (lower id on ties);
    it stops when nothing exposed fits."""
    taken = taken0.copy()
    while rem > 0:
        best = None
        for base, nodes in slots_ops:
            for o in _ops(base, nodes):
                c = _creator(base, nodes, o)
                if taken[o] or (c is not None and not taken[c]) or cost[o] > rem:
                    continue
                u = float(util[o])
                key = (-np.inf if u != u else u, -o)
                if best is None or key > best[0]:
                    best = (key, o)
        if best is None:
            break
        # an op that does not fit now never will: the page's queue drops it,
        # which the literal enumeration matches by never exposing its subtree
        taken[best[1]] = 1
        rem -= int(cost[best[1]])
    return taken


def _greedy_dropping(util, cost, taken0, slots_ops, rem):
    """The same greedy with the drop made explicit: an exposed op that does not
    fit when it is the best exposed one is discarded for good."""
    taken = taken0.copy()
    dropped = set()
    while rem > 0:
        best = None
        for base, nodes in slots_ops:
            for o in _ops(base, nodes):
                c = _creator(base, nodes, o)
                if taken[o] or o in dropped or (c is not None and not taken[c]):
                    continue
                u = float(util[o])
                key = (-np.inf if u != u else u, -o)
                if best is None or key > best[0]:
                    best = (key, o)
        if best is None:
            break
        o = best[1]
        if cost[o] > rem:
            dropped.add(o)
            continue
        taken[o] = 1
        rem -= int(cost[o])
    return taken


def _threshold_form(util, cost, taken0, slots_ops, rem):
    """What the GPU library computes, restated: beta(op) = the smallest key
    (u, -id) over the untaken part of its root path; ops are ranked by beta and
    the first rank whose cumulative cost passes the budget is the threshold;
    ops above it are taken; the tied group (beta equal to the threshold) is
    walked best-first by key, an op that does not fit is discarded with its
    subtree; then, while budget is left, the best-keyed exposed op that fits
    is taken."""
    keys, beta, creator = {}, {}, {}
    for base, nodes in slots_ops:
        for o in _ops(base, nodes):
            creator[o] = _creator(base, nodes, o)
            u = float(util[o])
            keys[o] = (-np.inf if u != u else u, -o)
        for o in _ops(base, nodes):          # creators first (pre-order ids)
            p = creator[o]
            inh = (np.inf, 0) if p is None or taken0[p] else beta[p]
            beta[o] = (np.inf, 0) if taken0[o] else min(keys[o], inh)
    cand = sorted([o for o in beta if not taken0[o]], key=lambda o: beta[o], reverse=True)
    taken = taken0.copy()
    cum, T = 0, None
    for o in cand:
        if cum + int(cost[o]) > rem:
            T = beta[o]
            break
        cum += int(cost[o])
    if T is None:
        for o in cand:
            taken[o] = 1
        return taken
    k = rem
    for o in cand:
        if beta[o] > T:
            taken[o] = 1
            k -= int(cost[o])
    group = [o for o in cand if beta[o] == T]
    dropped = set()
    while True:
        ex = [o for o in group if not taken[o] and o not in dropped and (creator[o] is None or taken[creator[o]])]
        if not ex:
            break
        o = max(ex, key=lambda o: keys[o])
        if cost[o] > k:
            dropped.add(o)
            continue
        taken[o] = 1
        k -= int(cost[o])
    while k > 0:
        ex = [o for o in cand if not taken[o] and o not in dropped and cost[o] <= k
              and (creator[o] is None or taken[creator[o]])]
        if not ex:
            break
        o = max(ex, key=lambda o: keys[o])
        taken[o] = 1
        k -= int(cost[o])
    return taken


@pytest.mark.parametrize("ties", [False, True])
def test_auction_with_three_way_splits_matches_the_greedy(ties):
    rng = np.random.default_rng(21 if ties else 22)
    n_drop_cases = 0
    for trial in range(80):
        lens, starts, T, util, cost, topo, slots_ops = _forest(rng, int(rng.integers(1, 5)), ties)
        total = int(cost.sum())
        slots = [[(st, n) for st, n in zip(starts, lens)]]
        taken0 = np.zeros(2 * T, dtype=np.uint8)
        if trial % 3 == 0:                       # a floor-like path taken up front
            base, nodes = slots_ops[0]
            i = int(rng.integers(nodes[0][0], nodes[0][0] + nodes[0][1]))
            for o in [base] + [base + 1 + j for j in osel._leaf_path(nodes, i)]:
                taken0[o] = 1
        pre = int(cost[taken0 == 1].sum())
        for B in sorted({pre + 1, pre + 2, pre + 3, total // 2, total - 1, total, total + 3}):
            if B <= pre:
                continue
            cfg = _cfg(lens=[T], slot_len=0, budget_ratio=0.0, budget_min=B)
            got, spent = osel.auction(util.reshape(1, 1, -1), cost.reshape(1, 1, -1), taken0.reshape(1, 1, -1),
                                      np.array([pre]), np.array([0, T]), slots, cfg, topo=topo)
            want = _greedy_dropping(util, cost, taken0, slots_ops, B - pre)
            assert np.array_equal(got.reshape(-1), want), (trial, B)
            assert spent[0] == pre + int(cost[(want == 1) & (taken0 == 0)].sum())
            assert spent[0] <= B
            alt = _threshold_form(util, cost, taken0, slots_ops, B - pre)
            assert np.array_equal(alt, want), (trial, B)
            if spent[0] < min(B, total):
                n_drop_cases += 1
    assert n_drop_cases > 0          # budgets a cost-2 op could not fill occurred


def test_skipping_and_dropping_are_the_same_greedy():
    # the budget left only shrinks, so an op that does not fit when it is the
    # best exposed one never fits later: skipping it (the literal statement)
    # and dropping it for good (the page's queue) take the same ops
    rng = np.random.default_rng(3)
    for trial in range(60):
        lens, starts, T, util, cost, topo, slots_ops = _forest(rng, 3, trial % 2 == 0)
        B = int(rng.integers(1, int(cost.sum()) + 2))
        a = _greedy_enumerated(util, cost, np.zeros(2 * T, np.uint8), slots_ops, B)
        b = _greedy_dropping(util, cost, np.zeros(2 * T, np.uint8), slots_ops, B)
        assert np.array_equal(a, b)


# ================================================================ floor and pack
def test_floor_pays_a_three_way_split_once():
    # tree of check_topology_by_hand case A over 8 tokens: the salient token 3
    # is a child of the three-way root, so its path is Add (1) + Split(root) (2)
    cfg = _cfg(lens=[8], slot_len=8, floor_frac=1.0, budget_ratio=0.0, budget_min=8)
    r = np.array([.1, .1, .1, 5, .1, .1, .1, .1], dtype=np.float32)
    nodes = otrees.slot_tree(0, 8, r, None, 1)
    topo = otrees.encode_topo(nodes, 0, 8).reshape(1, 1, -1)
    cost = np.zeros((1, 1, 16), dtype=np.uint8)
    cost[0, 0, 0] = 1
    for j, nd in enumerate(nodes):
        if nd[2]:
            cost[0, 0, 1 + j] = len(nd[2]) - 1
    rel = r.reshape(1, 1, -1)
    sens = np.ones((1, 1, 1), dtype=np.float32)
    tr = []
    ft, fs = osel.floor_select(rel, sens, cost, np.array([0, 8]), [[(0, 8)]], cfg, trace=tr, topo=topo)
    assert tr[0] == (3, 3)                          # token 3: Add + the root's three-way split
    # token 0 next (0.1, lowest id): Split([0,3)) and Split([0,2)) on top of the paid ones
    assert tr[1] == (0, 2)
    # the floor cap is alloc = 8: 3 + 2 + ... stays a hard maximum
    assert fs[0] <= 8 and fs[0] == sum(c for _, c in tr)


def test_pack_frontier_of_three_way_trees():
    rng = np.random.default_rng(9)
    for trial in range(12):
        n = int(rng.integers(3, 9))
        nodes = _random_topology(rng, 0, n)
        ops = _ops(0, nodes)
        cost = {0: 1}
        for j, nd in enumerate(nodes):
            if nd[2]:
                cost[1 + j] = len(nd[2]) - 1
        for mask in range(1 << len(ops)):
            taken = np.zeros(2 * n, dtype=np.uint8)
            for b, o in enumerate(ops):
                taken[o] = (mask >> b) & 1
            if any(taken[o] and _creator(0, nodes, o) is not None and not taken[_creator(0, nodes, o)]
                   for o in ops):
                continue
            fr = _frontier(nodes, taken, 0)
            assert len(fr) == sum(cost[o] for o in ops if taken[o])
            assert [nodes[j][0] for j in fr] == sorted(nodes[j][0] for j in fr)
            if fr:
                assert sum(nodes[j][1] for j in fr) == n


# ================================================================ end to end
@pytest.mark.parametrize("name", ["tiny", "fulldepth", "ragged"])
def test_split_mode_pipeline_spends_the_budget_and_full_budget_is_the_identity(name):
    cfg = small_config(name).replace(split_mode=1)
    inp = make_inputs(cfg)
    o = oracle.run_pipeline(inp, cfg)
    cu = inp["cu_seqlens"].numpy()
    bud = oracle.budgets([int(cu[s + 1] - cu[s]) for s in range(cfg.S)], cfg)
    assert [int(x) for x in o["spent"]] == [b["alloc"] for b in bud]
    if name != "ragged":     # single evidence tokens / planted spans with DP slots: some three-way splits
        assert int((o["trees"]["op_cost"] == 2).sum()) > 0
    full = oracle.run_pipeline(inp, cfg.replace(budget_ratio=1.0))
    assert np.all(full["kl"] == 0.0)
    assert np.array_equal(full["x_full"], full["x_comp"])


# ================================================================ planted slips
def _slipped_split(kind):
    orig = otrees.split_children

    def f(st, n, r, cut_q=None, mode=0):
        if mode == 0:
            return orig(st, n, r, cut_q, mode)
        b = (n + 1) // 2
        if n >= 3:
            seg = np.asarray(r[st:st + n], dtype=np.float32)
            i = int(np.argmax(seg))
            S = otrees.seq_sum(seg)
            q = -(-n // 4) if kind == "window_ceil" else max(n // 4, 1)
            half = 2.0 * float(seg[i]) >= S if kind == "at_least_half" else 2.0 * float(seg[i]) > S
            if S > 0 and half and q <= i <= n - 1 - q:
                return [(st, i), (st + i, 1), (st + i + 1, n - i - 1)]
        if cut_q is not None:
            m4 = n // 4 if kind == "cut_window_floor" else -(-n // 4)
            lo, hi = max(1, m4), min(n - 1, n - m4)
            best, bv = b, int(cut_q[st + b])
            for c in range(lo, hi + 1):
                v = int(cut_q[st + c])
                tie = (abs(c - b), -c) < (abs(best - b), -best) if kind == "tie_higher" else \
                    (abs(c - b), c) < (abs(best - b), best)
                if v > bv or (v == bv and tie):
                    best, bv = c, v
            b = best
        return [(st, b), (st + b, n - b)]
    return f


@pytest.mark.parametrize("kind", ["at_least_half", "window_ceil", "cut_window_floor", "tie_higher"])
def test_topology_slips_fail_the_pin(monkeypatch, kind):
    monkeypatch.setattr(otrees, "split_children", _slipped_split(kind))
    with pytest.raises(AssertionError):
        check_topology_by_hand()


def test_three_way_cost_slip_fails_the_pin(monkeypatch):
    orig = otrees.op_utilities

    def cost_one(nodes, rel, D, sens):
        util, cost = orig(nodes, rel, D, sens)
        for j, (_, _, ch, _) in enumerate(nodes):
            if len(ch) == 3:
                cost[1 + j] = 1
                util[1 + j] = np.float32(util[1 + j] * 2)
        return util, cost

    monkeypatch.setattr(otrees, "op_utilities", cost_one)
    with pytest.raises(AssertionError):
        check_split_utilities(0)
