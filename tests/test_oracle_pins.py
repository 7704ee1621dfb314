"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the pin it checks. A pin is a worked value the pages print
(tests/golden/*.json), a closed form, an invariant, a special case that
reduces to a library routine, or brute force on tiny inputs; each is chosen
so that a plausible slip in the oracle (a dropped term, a wrong sign, index or
scale, a transposed operand) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
from oracle import common, trees as otrees, select as osel, partition as opart
from oracle.pack import _frontier
from workload import small_config, make_inputs, Config

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(**kw):
    base = dict(name="t", S=1, Ly=1, H=1, G=2, d=8, lens=[16], dtype="f32", rope_base=1e4,
                P=4, slot_len=8, T_dec=1, vocab=64, w_dtype="f32", plant="evidence", n_plant=0)
    base.update(kw)
    return Config(**base)


# ---------------------------------------------------------------- budgets (P16)
def test_budget_formula_golden():
    g = json.load(open(os.path.join(GOLD, "budget_formula.json")))
    for c in g["cases"]:
        cfg = _cfg(budget_ratio=c["r"], budget_min=c["B_min"])
        assert common.budgets([c["L"]], cfg)[0]["B"] == c["B"]


def test_budget_regions_and_floor():
    cfg = small_config("ragged")
    for L in (10, 300, 1100):
        pe, c0, c1, ss = common.regions(L, cfg)
        assert 0 <= pe == c0 <= c1 <= ss <= L
    b = common.budgets([1100], cfg)[0]
    pe, c0, c1, ss = common.regions(1100, cfg)
    assert b["recent"] == (ss - c1) * cfg.Ly * cfg.H
    assert b["alloc"] == b["B"] - b["recent"]
    assert b["floor"] == math.floor(np.float32(cfg.floor_frac) * b["alloc"])


# ---------------------------------------------------------------- RoPE (P2)
def test_rope_inverse_and_complex_form():
    rng = np.random.default_rng(0)
    d, base = 16, 1e4
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 1000, 32767])
    y = common.rope(x, pos, base)
    assert np.allclose(common.rope_inv(y, pos, base), x, atol=1e-12)
    # independent form: pair (x_j, x_{j+d/2}) as a complex number times e^{i theta_j}
    j = np.arange(d // 2)
    theta = np.outer(pos, base ** (-2.0 * j / d))
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * theta)
    assert np.allclose(y[:, : d // 2], z.real, atol=1e-12)
    assert np.allclose(y[:, d // 2:], z.imag, atol=1e-12)
    # relative-position property: <R_m q, R_n k> depends on m - n only
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = common.rope(q, 40, base) @ common.rope(k, 33, base)
    b = common.rope(q, 1007, base) @ common.rope(k, 1000, base)
    assert abs(a - b) < 1e-9


# ---------------------------------------------------------------- scores (P8, P9)
def test_scores_against_library_softmax():
    cfg = small_config("tiny")
    inp = make_inputs(cfg)
    cu = inp["cu_seqlens"].numpy()
    sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    K = common.to64(inp["K"][0, 0])
    Q = common.to64(inp["Qp"][0, 0]).reshape(cfg.G * cfg.P, cfg.d)
    A = scipy.special.softmax(Q @ K.T / math.sqrt(cfg.d), axis=1)
    assert np.allclose(sc["r0"][0, 0], A.sum(0), rtol=1e-6)
    # P8: the summed mass of every unit is exactly G*P
    assert abs(float(A.sum()) - cfg.G * cfg.P) < 1e-9
    assert abs(float(sc["r0"][0, 0].astype(np.float64).sum()) - cfg.G * cfg.P) < 1e-3
    ent = scipy.stats.entropy(A, axis=1)
    assert np.allclose(sc["ent"][0, 0].reshape(-1), ent, rtol=1e-5)
    assert np.allclose(sc["lse"][0, 0].reshape(-1),
                       scipy.special.logsumexp(Q @ K.T / math.sqrt(cfg.d), axis=1), rtol=1e-6)
    Hi = (A * ent[:, None]).sum(0) / A.sum(0)
    assert np.allclose(sc["feats"][3, 0, 0], Hi, rtol=1e-5)
    mg = A.reshape(cfg.G, cfg.P, -1).sum(1)
    assert np.allclose(sc["feats"][2, 0, 0], np.var(mg, axis=0), rtol=1e-4, atol=1e-9)
    V = common.to64(inp["V"][0, 0])
    assert np.allclose(sc["feats"][1, 0, 0], np.linalg.norm(V, axis=1), rtol=1e-6)
    assert sc["feats"][4, 0, 0, 0] == 0 and sc["feats"][4, 0, 0, -1] == 1
    vn = np.linalg.norm(V, axis=1)
    assert np.isclose(sc["head_sens"][0, 0, 0], (A.sum(0) * vn).sum() / A.sum(), rtol=1e-6)


def test_entropy_closed_forms():
    cfg = _cfg(lens=[50])
    L, d = 50, cfg.d
    Kc = np.tile(np.linspace(-1, 1, d), (L, 1))
    K = torch.tensor(Kc.reshape(1, 1, L, d), dtype=torch.float32)
    V = torch.randn(1, 1, L, d)
    Qp = torch.randn(1, 1, cfg.G, cfg.P, d)
    sc = oracle.probe_scores(K, V, Qp, np.array([0, L]), cfg)
    # P9: all keys equal -> uniform rows -> H = ln L for every row and token
    assert np.allclose(sc["ent"], math.log(L), rtol=1e-6)
    assert np.allclose(sc["feats"][3], math.log(L), rtol=1e-6)
    assert np.allclose(sc["feats"][2], 0.0, atol=1e-12)
    # one dominant key -> entropy -> 0, mass concentrates on that key
    K2 = np.random.default_rng(1).standard_normal((L, d)) * 0.01
    q = np.ones(d)
    K2[17] = 400.0 * q
    Qp2 = torch.tensor(np.tile(q, (1, 1, cfg.G, cfg.P, 1)), dtype=torch.float32)
    sc2 = oracle.probe_scores(torch.tensor(K2.reshape(1, 1, L, d), dtype=torch.float32),
                              V, Qp2, np.array([0, L]), cfg)
    assert sc2["ent"].max() < 1e-6
    assert abs(sc2["r0"][0, 0, 17] - cfg.G * cfg.P) < 1e-3


# ---------------------------------------------------------------- propagation (P8, P19)
def test_propagation_conservation_and_dense_rollout():
    rng = np.random.default_rng(3)
    L, d, G = 40, 8, 2
    K = rng.standard_normal((L, d))
    Qc = rng.standard_normal((G, L, d))
    r0 = rng.random(L)
    w = 0.3
    # P19: with M >= L every token is a seed; one hop is w * A_hat^T r0 where
    # A_hat is the GQA-mean causal attention matrix of the prefill queries.
    cfg = _cfg(G=G, d=d, lens=[L], n_seeds=L, n_hops=1, hop_weight=w)
    out = oracle.propagate(torch.tensor(K.reshape(1, 1, L, d)), torch.tensor(Qc.reshape(1, G, L, d)),
                           r0.reshape(1, 1, L).astype(np.float32), np.array([0, L]), cfg)
    logits = np.einsum("gjd,id->gji", Qc, K) / math.sqrt(d)
    logits = np.where(np.tril(np.ones((L, L)))[None] > 0, logits, -np.inf)
    Ahat = scipy.special.softmax(logits, axis=2).mean(0)          # [j, i]
    r32 = r0.astype(np.float32).astype(np.float64)
    expect = r32 + w * Ahat.T @ r32
    assert np.allclose(out["rel"][0, 0], expect, rtol=1e-6)
    # P8: each hop hands on exactly w times the seeds' mass, and the seeds are
    # the top-M tokens of the previous increment
    from oracle.propagate import _unit
    wf = float(np.float32(w))
    tot, seeds = _unit(Qc, K, r32, G, 2, 5, wf)
    prev = r32
    total_check = r32.copy()
    for sd in seeds:
        inc = np.zeros(L)
        for j in sd:
            b = scipy.special.softmax((Qc[:, j] @ K[: j + 1].T) / math.sqrt(d), axis=1).mean(0)
            inc[: j + 1] += wf * prev[j] * b
        assert abs(inc.sum() - wf * prev[sd].sum()) < 1e-10
        order = np.argsort(-prev, kind="stable")[:5]
        assert set(order.tolist()) == set(sd.tolist())
        total_check += inc
        prev = inc
    assert np.allclose(tot, total_check, rtol=1e-12)


# ---------------------------------------------------------------- trees (P3, P4, P10)
def _tree_inputs(L, d, seed=0, P=4, G=2):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((L, d)), rng.standard_normal((L, d)), rng.random(L)


def test_tree_value_flow_and_topology():
    cfg = _cfg(d=8)
    ktil, V, r = _tree_inputs(37, 8)
    kn = np.linalg.norm(ktil, axis=1)
    Ad = np.random.default_rng(1).random((4, 37))
    Qd = np.random.default_rng(2).standard_normal((4, 8))
    lse = np.zeros(4)
    nodes, rel, D, mu, kh, vh = otrees._slot(ktil, kn, V, r, Ad, Qd, lse, 0, 37, 0, cfg, 1e4)
    assert len(nodes) == 2 * 37 - 1
    for j, (st, n, lc, rc) in enumerate(nodes):
        # P4: parent value is exactly the sum of its children's values
        if lc >= 0:
            assert rel[j] == rel[lc] + rel[rc]
            assert nodes[lc][0] == st and nodes[lc][1] == (n + 1) // 2
            assert nodes[rc][0] == st + (n + 1) // 2 and nodes[rc][1] == n // 2
            assert lc == j + 1 and rc == j + 2 * ((n + 1) // 2)
        else:
            assert n == 1 and rel[j] == r[st] and D[j] == 0 and mu[j] == 1
        assert abs(rel[j] - r[st:st + n].sum()) < 1e-12
        assert 0 <= D[j] <= 1


def test_one_token_prototype_is_the_token():
    # P3: a 1-token node reproduces its key (unrotate then rerotate at the same
    # position) and value, with multiplicity 1.
    cfg = _cfg(d=8)
    rng = np.random.default_rng(5)
    K = rng.standard_normal((10, 8))
    pos = np.arange(10)
    kt = common.rope_inv(K, pos, 1e4)
    V = rng.standard_normal((10, 8))
    r = rng.random(10)
    nodes, rel, D, mu, kh, vh = otrees._slot(kt, np.linalg.norm(kt, axis=1), V, r,
                                             np.ones((4, 10)), np.zeros((4, 8)), np.zeros(4),
                                             6, 1, 0, cfg, 1e4)
    assert len(nodes) == 1 and mu[0] == 1.0
    assert np.allclose(kh[0], K[6], atol=1e-12)
    assert np.allclose(vh[0], V[6], atol=1e-15)


def test_multiplicity_closed_forms():
    # P10: identical unrotated keys -> mu = n; orthogonal equal-norm -> sqrt(n)
    cfg = _cfg(d=8)
    n = 4
    kt_same = np.tile(np.arange(1.0, 9.0), (n, 1))
    kt_orth = np.eye(8)[:n] * 2.5
    V = np.zeros((n, 8))
    r = np.ones(n)
    for kt, want in ((kt_same, n), (kt_orth, math.sqrt(n))):
        nodes, rel, D, mu, kh, vh = otrees._slot(kt, np.linalg.norm(kt, axis=1), V, r,
                                                 np.ones((4, n)), np.zeros((4, 8)), np.zeros(4),
                                                 0, n, 0, cfg, 1e4)
        assert abs(mu[0] - want) < 1e-12
        # the prototype key is the mean re-rotated at the lower midpoint
        assert np.allclose(kh[0], common.rope(kt.mean(0), (n - 1) // 2, 1e4), atol=1e-12)


def test_distortion_closed_forms():
    cfg = _cfg(d=8)
    n = 4
    kt = np.tile(np.arange(1.0, 9.0), (n, 1))      # identical unrotated keys: mu = n
    Vsame = np.tile(np.linspace(0, 1, 8), (n, 1))  # identical values
    r = np.array([1.0, 2.0, 3.0, 4.0])
    L = 10
    # zero query rows: every logit is 0, a_i = exp(-lse) = 1/L
    lse = np.full(4, math.log(L))
    Ad = np.full((4, n), 1.0 / L)
    nodes, rel, D, mu, kh, vh = otrees._slot(kt, np.linalg.norm(kt, axis=1), Vsame, r, Ad,
                                             np.zeros((4, 8)), lse, 0, n, 0, cfg, 1e4)
    # Z = n/L, Z_hat = mu/L = n/L -> e_A = 0; identical values -> e_V = 0
    assert D[0] == pytest.approx(0.0, abs=1e-12)
    # orthogonal keys: mu = sqrt(2) for a 2-token node, e_A = |sqrt2 - 2| / 2
    kt2 = np.eye(8)[:2] * 3.0
    Ad2 = np.full((4, 2), 1.0 / L)
    nodes, rel, D2, mu2, _, _ = otrees._slot(kt2, np.linalg.norm(kt2, axis=1), Vsame[:2], r[:2],
                                             Ad2, np.zeros((4, 8)), lse, 0, 2, 0, cfg, 1e4)
    assert D2[0] == pytest.approx(0.25 * abs(math.sqrt(2) - 2) / 2, rel=1e-12)
    # value weights: 0.9 relevance share + 0.1 uniform
    V = np.random.default_rng(0).standard_normal((n, 8))
    nodes, rel, D3, _, _, vh3 = otrees._slot(kt, np.linalg.norm(kt, axis=1), V, r, Ad,
                                             np.zeros((4, 8)), lse, 0, n, 0, cfg, 1e4)
    w = 0.9 * r / r.sum() + 0.1 / n
    assert np.allclose(vh3[0], w @ V, atol=1e-12)
    # e_V from its definition with o_rho = u / Z
    u = Ad @ V
    Z = Ad.sum(1)
    o = u / Z[:, None]
    eV = (Z * np.linalg.norm(o - vh3[0], axis=1)).sum() / (Z * np.linalg.norm(o, axis=1)).sum()
    assert D3[0] == pytest.approx(min(1.0, 0.75 * eV), rel=1e-12)


def test_frontier_sizes_golden():
    # P14: every frontier an 8-token binary slot can reach; the page's sizes are
    # among them and each taken op adds exactly one stored entry
    g = json.load(open(os.path.join(GOLD, "gracekv_frontier_sizes.json")))
    n = g["slot_tokens"]
    nodes = otrees.tree_nodes(0, n)
    internal = [j for j, nd in enumerate(nodes) if nd[2] >= 0]
    parent = {}
    for j, nd in enumerate(nodes):
        for c in nd[2:]:
            if c >= 0:
                parent[c] = j
    sizes = set()
    for mask in range(1 << (1 + len(internal))):
        taken = np.zeros(2 * n, dtype=np.uint8)
        taken[0] = mask & 1
        for b, j in enumerate(internal):
            taken[1 + j] = (mask >> (b + 1)) & 1
        ok = True
        for j in internal:   # an op needs its creator
            if taken[1 + j]:
                creator = 0 if j == 0 else 1 + parent[j]
                ok &= bool(taken[creator])
        if not ok:
            continue
        fr = _frontier(otrees.slot_tree(0, n), taken, 0)
        assert len(fr) == int(taken.sum())
        starts = sorted((nodes[j][0], nodes[j][1]) for j in fr)
        assert [nodes[j][0] for j in fr] == [s for s, _ in starts]   # position order
        if fr:
            assert sum(m for _, m in starts) == n                    # covers the slot
        sizes.add(len(fr))
    assert set(g["sizes"]) <= sizes
    assert sizes == set(range(0, n + 1))


# ---------------------------------------------------------------- auction (P6, P13)
def _greedy_by_enumeration(util, cost, taken0, slots_ops, rem):
    """The page's greedy stated literally: every round enumerates the exposed
    ops and takes the highest-utility affordable one (lower id on ties)."""
    taken = taken0.copy()
    order = []
    while rem > 0:
        best = None
        for (base, nodes) in slots_ops:
            ops = [(base, None)] + [(base + 1 + j, j) for j, nd in enumerate(nodes) if nd[2] >= 0]
            for o, j in ops:
                if taken[o] or cost[o] == 0:
                    continue
                if j is None:
                    exposed = True
                else:
                    par = [p for p, nd in enumerate(nodes) if j in nd[2:]]
                    exposed = bool(taken[base]) if j == 0 else bool(taken[base + 1 + par[0]])
                if not exposed or cost[o] > rem:
                    continue
                u = float(util[o])
                u = -np.inf if u != u else u
                if best is None or (u, -o) > best[0]:
                    best = ((u, -o), o)
        if best is None:
            break
        o = best[1]
        taken[o] = 1
        rem -= int(cost[o])
        order.append(o)
    return taken, order


def _random_forest(rng, n_slots, ties):
    lens = rng.integers(1, 9, n_slots).tolist()
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    T = int(sum(lens))
    util = np.zeros(2 * T, dtype=np.float32)
    cost = np.zeros(2 * T, dtype=np.uint8)
    slots_ops = []
    for st, n in zip(starts, lens):
        nodes = otrees.tree_nodes(st, n)
        base = 2 * st
        slots_ops.append((base, nodes))
        util[base] = rng.integers(0, 4) if ties else rng.standard_normal()
        cost[base] = 1
        for j, nd in enumerate(nodes):
            if nd[2] >= 0:
                util[base + 1 + j] = rng.integers(0, 4) if ties else rng.standard_normal()
                cost[base + 1 + j] = 1
    return lens, starts, T, util, cost, slots_ops


def _beta_threshold_auction(util, cost, taken0, slots_ops, rem):
    """The GPU library's formulation of the same greedy, restated on the CPU:
    beta(op) = min of (u, -id) over the untaken part of its root path; ops with
    beta above the rem-th largest are taken; the tied group below the binding
    op is finished by a best-first walk of that subtree."""
    keys, beta, parent_op = {}, {}, {}
    for base, nodes in slots_ops:
        par = {}
        for j, nd in enumerate(nodes):
            for c in nd[2:]:
                if c >= 0:
                    par[c] = j
        ops = [base] + [base + 1 + j for j, nd in enumerate(nodes) if nd[2] >= 0]
        for o in ops:
            j = None if o == base else o - base - 1
            parent_op[o] = None if o == base else (base if j == 0 else base + 1 + par[j])
        for o in ops:
            u = float(util[o])
            keys[o] = (-np.inf if u != u else u, -o)
        for o in ops:   # parents before children (pre-order ids)
            p = parent_op[o]
            inherited = (np.inf, 0) if p is None or taken0[p] else beta[p]
            beta[o] = (np.inf, 0) if taken0[o] else min(keys[o], inherited)
    cand = sorted([o for o in beta if not taken0[o]], key=lambda o: beta[o], reverse=True)
    taken = taken0.copy()
    if rem >= len(cand):
        for o in cand:
            taken[o] = 1
        return taken
    if rem <= 0:
        return taken
    bstar = beta[cand[rem - 1]]
    above = [o for o in cand if beta[o] > bstar]
    for o in above:
        taken[o] = 1
    k = rem - len(above)
    group = [o for o in cand if beta[o] == bstar]
    while k > 0:
        exposed = [o for o in group if not taken[o] and (parent_op[o] is None or taken[parent_op[o]])]
        o = max(exposed, key=lambda o: keys[o])
        taken[o] = 1
        k -= 1
    return taken


@pytest.mark.parametrize("ties", [False, True])
def test_auction_matches_brute_force_greedy(ties):
    rng = np.random.default_rng(11 if ties else 12)
    for trial in range(60):
        lens, starts, T, util, cost, slots_ops = _random_forest(rng, int(rng.integers(1, 5)), ties)
        total_ops = int(cost.sum())
        cfg = _cfg(lens=[T], slot_len=0)
        slots = [[(st, n) for st, n in zip(starts, lens)]]
        # optional floor-like pre-taken paths
        taken0 = np.zeros(2 * T, dtype=np.uint8)
        if trial % 3 == 0:
            base, nodes = slots_ops[0]
            i = int(rng.integers(nodes[0][0], nodes[0][0] + nodes[0][1]))
            for o in [base] + [base + 1 + j for j in osel._leaf_path(otrees.slot_tree(nodes[0][0], nodes[0][1]), i)]:
                taken0[o] = 1
        pre = int(taken0.sum())
        for B in sorted({1, 2, 3, total_ops // 2, total_ops - 1, total_ops, total_ops + 3}):
            if B <= pre:
                continue
            cfg = _cfg(lens=[T], slot_len=0, budget_ratio=0.0, budget_min=B)
            got, spent = osel.auction(util.reshape(1, 1, -1), cost.reshape(1, 1, -1),
                                      taken0.reshape(1, 1, -1), np.array([pre]),
                                      np.array([0, T]), slots, cfg)
            want, _ = _greedy_by_enumeration(util, cost, taken0, slots_ops, B - pre)
            assert np.array_equal(got.reshape(-1), want), (trial, B)
            assert spent[0] == min(B, total_ops)
            alt = _beta_threshold_auction(util, cost, taken0, slots_ops, B - pre)
            assert np.array_equal(alt, want), (trial, B)


def test_gracekv_toy_auction_golden():
    # P13: the six-entry illustration: a floor path of cost 3 (Add + two
    # Splits to reach one exact token), then a Split and two Adds of cost 1.
    g = json.load(open(os.path.join(GOLD, "gracekv_toy_auction.json")))
    n = 4
    T = 3 * n                                    # slots A, B, C of four tokens
    cfg = _cfg(lens=[T], slot_len=n, budget_ratio=0.0, budget_min=g["budget"], floor_frac=0.5)
    slots = [[(0, n), (n, n), (2 * n, n)]]
    rel = np.full((1, 1, T), 0.01, dtype=np.float32)
    rel[0, 0, n] = 1.0                           # the exact token sits first in slot B
    sens = np.ones((1, 1, 1), dtype=np.float32)
    nodes = otrees.tree_nodes(0, n)
    cost = np.zeros((1, 1, 2 * T), dtype=np.uint8)
    util = np.full((1, 1, 2 * T), 0.05, dtype=np.float32)
    for k in range(3):
        cost[0, 0, 2 * k * n] = 1
        for j, nd in enumerate(nodes):
            if nd[2] >= 0:
                cost[0, 0, 2 * k * n + 1 + j] = 1
    A, B, C = 0, 2 * n, 4 * n
    right_B = B + 1 + nodes[0][3]                # Split of slot B's right half
    util[0, 0, right_B] = 3.0                    # "expiry phrase" split
    util[0, 0, C] = 2.0                          # Add: troubleshooting notes
    util[0, 0, A] = 1.0                          # Add: meeting background
    util[0, 0, C + 1] = 0.5
    ftrace, atrace = [], []
    ftaken, fspent = osel.floor_select(rel, sens, cost, np.array([0, T]), slots, cfg, trace=ftrace)
    taken, spent = osel.auction(util, cost, ftaken, fspent, np.array([0, T]), slots, cfg,
                                trace=atrace)
    steps = g["steps"]
    assert ftrace[0][1] == steps[0]["cost"] and fspent[0] == steps[0]["cost"]
    assert [int(cost.reshape(-1)[o]) for o in atrace] == [s["cost"] for s in steps[1:]]
    assert atrace == [right_B, C, A]
    assert spent[0] == g["total"]
    # P13: a leaf at depth D costs D + 1 (Add plus D Splits)
    for depth_n, want in ((1, 1), (2, 2), (4, 3), (8, 4), (64, 7), (128, 8)):
        nd = otrees.slot_tree(0, depth_n)
        assert len(osel._leaf_path(nd, 0)) + 1 == want


def test_floor_is_a_hard_cap_and_pays_shared_ancestors_once():
    cfg = small_config("tiny").replace(floor_frac=0.25, budget_min=32, budget_ratio=0.0)
    L = 64
    slots = [[(0, 32), (32, 32)]]
    rel = np.zeros((1, 1, L), dtype=np.float32)
    rel[0, 0, [3, 4, 5, 40]] = [4.0, 3.0, 2.0, 1.0]
    cost = np.zeros((1, 1, 2 * L), dtype=np.uint8)
    for st in (0, 32):
        nodes = otrees.tree_nodes(st, 32)
        cost[0, 0, 2 * st] = 1
        for j, nd in enumerate(nodes):
            if nd[2] >= 0:
                cost[0, 0, 2 * st + 1 + j] = 1
    tr = []
    taken, spent = osel.floor_select(rel, np.ones((1, 1, 1), dtype=np.float32), cost,
                                     np.array([0, L]), slots, cfg.replace(lens=[L]), trace=tr)
    F = common.budgets([L], cfg.replace(lens=[L]))[0]["floor"]
    assert F == 8
    # token 3: Add + 5 splits = 6; token 4 shares the root, the 16- and 8-token
    # nodes: 2 new splits but only 2 entries left -> accepted (6 + 2 = 8)
    assert tr[0] == (3, 6) and tr[1] == (4, 2) and spent[0] == 8 <= F
    assert int(taken.sum()) == 8


# ---------------------------------------------------------------- token top-B (P5)
def test_token_topk_is_a_top_set():
    rng = np.random.default_rng(7)
    for trial in range(20):
        H, L = 3, int(rng.integers(5, 40))
        rel = rng.integers(0, 5, (1, H, L)).astype(np.float32)   # tie storm
        cfg = _cfg(H=H, lens=[L], token_mode=True, budget_min=1,
                   budget_ratio=float(rng.random()))
        taken, spent = osel.token_topk(rel, np.array([0, L]), cfg)
        B = common.budgets([L], cfg)[0]["alloc"]
        assert taken.sum() == min(B, H * L) == spent[0]
        keys = [(float(rel[0, h, i]), -(h * L + i)) for h in range(H) for i in range(L)]
        sel = [k for k, t in zip(keys, taken.reshape(-1)) if t]
        uns = [k for k, t in zip(keys, taken.reshape(-1)) if not t]
        if sel and uns:
            assert min(sel) > max(uns)


# ---------------------------------------------------------------- partition (P17)
def test_dp_matches_exhaustive_segmentation():
    rng = np.random.default_rng(9)
    for trial in range(6):
        L = int(rng.integers(8, 15))
        cfg = _cfg(lens=[L], slot_len=0, slot_min=2, slot_max=5, slot_target=3, d=8)
        hidden = torch.tensor(rng.standard_normal((L, 6)), dtype=torch.float32)
        cq, kq = opart.slot_costs(hidden, np.array([0, L]), cfg)
        got = opart.dp_slots(cq, kq, 0, 0, L, cfg)

        def score(seg):
            v, a = 0, 0
            for i, n in enumerate(seg):
                v += int(cq[a + n - 1, n - cfg.slot_min])
                if a > 0:
                    v -= int(kq[a])
                a += n
            return v

        best = None
        for k in range(1, L // 2 + 1):
            for seg in itertools.product(range(2, 6), repeat=k):
                if sum(seg) == L:
                    sc_ = score(seg)
                    best = sc_ if best is None or sc_ < best else best
        assert sum(n for _, n in got) == L
        assert all(2 <= n <= 5 for _, n in got)
        assert score([n for _, n in got]) == best
        # quantized cost is round-half-away of the fp64 cost times 2^20
        hn = opart.normalize(common.to64(hidden))
        assert cq[4, 3 - 2] == math.floor(opart.slot_cost(hn, 2, 3, cfg) * 2 ** 20 + 0.5)


def test_dp_finds_planted_turns():
    rng = np.random.default_rng(4)
    Dh, cuts = 64, [0, 40, 90, 130, 200]
    hs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        c = rng.standard_normal(Dh)
        c /= np.linalg.norm(c)
        u = rng.standard_normal(Dh)
        u /= np.linalg.norm(u)
        t = np.arange(b - a)[:, None] / (b - a)
        hs.append(c + 0.5 * t * u + rng.standard_normal((b - a, Dh)) * 1e-4)
    hidden = torch.tensor(np.concatenate(hs), dtype=torch.float32)
    L = cuts[-1]
    cfg = _cfg(lens=[L], slot_len=0, slot_min=16, slot_max=128, slot_target=64)
    cq, kq = opart.slot_costs(hidden, np.array([0, L]), cfg)
    got = opart.dp_slots(cq, kq, 0, 0, L, cfg)
    bounds = {a for a, _ in got[1:]}
    for c in cuts[1:-1]:
        assert any(abs(c - b) <= 1 for b in bounds), (c, sorted(bounds))


# ---------------------------------------------------------------- decode (P11, P12)
def test_decode_matches_library_attention():
    cfg = small_config("stress")
    inp = make_inputs(cfg)
    cu = inp["cu_seqlens"].numpy()
    cache = oracle.full_view(inp["K"], inp["V"], cu)
    t = 1
    x, o = oracle.decode_step(cache, inp["Kd"], inp["Vd"], inp["Qd"][t], t, cfg.G)
    for s in range(cfg.S):
        for l in range(cfg.Ly):
            for h in range(cfg.H):
                a, b = int(cu[s]), int(cu[s + 1])
                k = torch.cat([inp["K"][l, h, a:b].double(), inp["Kd"][l, h, s, : t + 1].double()])
                v = torch.cat([inp["V"][l, h, a:b].double(), inp["Vd"][l, h, s, : t + 1].double()])
                q = inp["Qd"][t, s, l, h * cfg.G:(h + 1) * cfg.G].double()
                ref = torch.nn.functional.scaled_dot_product_attention(
                    q[:, None, :], k[None].expand(cfg.G, -1, -1).contiguous(),
                    v[None].expand(cfg.G, -1, -1).contiguous())[:, 0]
                assert np.allclose(o[s, l, h * cfg.G:(h + 1) * cfg.G], ref.numpy(), atol=1e-12)
    assert np.allclose(x[0], o[0].sum(0).reshape(-1), atol=1e-12)


def test_multiplicity_bias_equals_repeated_entries():
    # P11 (lossless merge): an entry with ln(mu) = ln 3 attends exactly like
    # three identical copies of it.
    rng = np.random.default_rng(2)
    d, G = 8, 2
    K = rng.standard_normal((5, d))
    V = rng.standard_normal((5, d))
    Kd = torch.tensor(rng.standard_normal((1, 1, 1, 1, d)))
    Vd = torch.tensor(rng.standard_normal((1, 1, 1, 1, d)))
    q = torch.tensor(rng.standard_normal((1, 1, G, d)))
    merged = {"K": K, "V": V, "lnmu": np.array([0, 0, math.log(3.0), 0, 0]),
              "seg_off": np.zeros((1, 1, 1), np.int64), "seg_len": np.full((1, 1, 1), 5, np.int32)}
    Kr = np.concatenate([K[:2], K[2:3], K[2:3], K[2:3], K[3:]])
    Vr = np.concatenate([V[:2], V[2:3], V[2:3], V[2:3], V[3:]])
    rep = {"K": Kr, "V": Vr, "lnmu": np.zeros(7), "seg_off": np.zeros((1, 1, 1), np.int64),
           "seg_len": np.full((1, 1, 1), 7, np.int32)}
    xa, _ = oracle.decode_step(merged, Kd, Vd, q, 0, G)
    xb, _ = oracle.decode_step(rep, Kd, Vd, q, 0, G)
    assert np.allclose(xa, xb, atol=1e-13)


def test_token_mode_eviction_bound():
    # P12 (DistillCache Sec. 3.1.4): with renormalized eviction,
    # ||o - o_hat|| <= 2 * max||v|| * eps, eps the evicted attention mass.
    cfg = small_config("mistral1").replace(T_dec=2)
    inp = make_inputs(cfg)
    out = oracle.run_pipeline(inp, cfg, stages=("compress",))
    cu = inp["cu_seqlens"].numpy()
    full = oracle.full_view(inp["K"], inp["V"], cu)
    taken = out["taken"]
    for t in range(cfg.T_dec):
        _, of = oracle.decode_step(full, inp["Kd"], inp["Vd"], inp["Qd"][t], t, cfg.G)
        _, oc = oracle.decode_step(out["cache"], inp["Kd"], inp["Vd"], inp["Qd"][t], t, cfg.G)
        for h in range(cfg.H):
            K = common.to64(inp["K"][0, h])
            V = common.to64(inp["V"][0, h])
            Ke = np.concatenate([K, common.to64(inp["Kd"][0, h, 0, : t + 1])])
            Ve = np.concatenate([V, common.to64(inp["Vd"][0, h, 0, : t + 1])])
            keep = np.concatenate([taken[0, h].astype(bool), np.ones(t + 1, bool)])
            for g in range(cfg.G):
                q = common.to64(inp["Qd"][t, 0, 0, h * cfg.G + g])
                p = scipy.special.softmax(Ke @ q / math.sqrt(cfg.d))
                eps = p[~keep].sum()
                C = np.linalg.norm(Ve, axis=1).max()
                diff = np.linalg.norm(of[0, 0, h * cfg.G + g] - oc[0, 0, h * cfg.G + g])
                assert diff <= 2 * C * eps + 1e-9


# ---------------------------------------------------------------- KL (P15)
def test_kl_against_library():
    rng = np.random.default_rng(8)
    n, Dm, Vv = 5, 16, 50
    xf = rng.standard_normal((n, Dm)).astype(np.float32)
    xc = (xf + 0.3 * rng.standard_normal((n, Dm))).astype(np.float32)
    W = torch.tensor(rng.standard_normal((Vv, Dm)), dtype=torch.float32)
    kl = oracle.kl_rows(xf, xc, W, "f32")
    assert (kl >= 0).all()
    assert np.array_equal(oracle.kl_rows(xf, xf, W, "f32"), np.zeros(n, np.float32))
    from oracle.kl import rmsnorm_cast
    y = torch.tensor(rmsnorm_cast(xf, "f32") @ common.to64(W).T)
    yh = torch.tensor(rmsnorm_cast(xc, "f32") @ common.to64(W).T)
    ref = torch.nn.functional.kl_div(torch.log_softmax(yh, 1), torch.log_softmax(y, 1),
                                     log_target=True, reduction="none").sum(1)
    assert np.allclose(kl, ref.numpy(), rtol=1e-5, atol=1e-7)
    sp = scipy.stats.entropy(scipy.special.softmax(y.numpy(), 1), scipy.special.softmax(yh.numpy(), 1),
                             axis=1)
    assert np.allclose(kl, sp, rtol=1e-5, atol=1e-7)
    # RMSNorm: unit RMS before the cast
    xr = rmsnorm_cast(xf, "f32")
    assert np.allclose(np.sqrt((xr.astype(np.float64) ** 2).mean(1)), 1.0, atol=1e-5)


# ---------------------------------------------------------------- end to end (P1)
@pytest.mark.parametrize("name", ["tiny", "stress", "ragged", "mistral1"])
def test_full_budget_recovers_the_cache_and_kl_is_zero(name):
    # P1 (GraceKV page, '05 Physical cache packing'): with the budget at full
    # scale every tree expands to its leaves and the original entries return
    # exactly; decode and KL then match the full cache exactly.
    cfg = small_config(name).replace(budget_ratio=1.0, T_dec=1)
    if name != "tiny":
        cfg = cfg.replace(Ly=1, H=1)
    inp = make_inputs(cfg)
    out = oracle.run_pipeline(inp, cfg)
    cu = inp["cu_seqlens"].numpy()
    full = oracle.full_view(inp["K"], inp["V"], cu)
    c = out["cache"]
    assert np.array_equal(c["seg_len"], full["seg_len"])
    for s in range(cfg.S):
        for l in range(cfg.Ly):
            for h in range(cfg.H):
                a, n = int(c["seg_off"][s, l, h]), int(c["seg_len"][s, l, h])
                b = int(full["seg_off"][s, l, h])
                assert np.array_equal(c["K"][a:a + n], full["K"][b:b + n])
                assert np.array_equal(c["V"][a:a + n], full["V"][b:b + n])
                assert np.array_equal(c["pos"][a:a + n], np.arange(n))
    assert np.all(c["lnmu"] == 0)
    assert np.array_equal(out["x_comp"], out["x_full"])
    assert np.all(out["kl"] == 0.0)


# ---------------------------------------------------------------- head-level hybrid (NEXT 4)
def _hybrid_cfg(**kw):
    return _cfg(**kw).replace(hybrid_frac=kw.get("hybrid_frac", 0.34))


def test_hybrid_units_are_the_top_heads_under_the_budget_cap():
    # DistillCache Appendix E.3: the most important heads keep the full cache;
    # K = min(floor(f*U), floor(alloc / C)); ranking by s_lh desc, unit asc
    rng = np.random.default_rng(21)
    for trial in range(30):
        Ly, H, L = 2, 3, int(rng.integers(4, 30))
        sens = rng.integers(0, 3, (2, Ly, H)).astype(np.float32)   # ties
        r = float(rng.choice([0.05, 0.2, 0.5, 1.0]))
        cfg = _hybrid_cfg(Ly=Ly, H=H, lens=[L, L], budget_ratio=r, budget_min=1, hybrid_frac=0.34)
        cu = np.array([0, L, 2 * L])
        full = osel.hybrid_units(sens, cu, cfg)
        for s in range(2):
            b = common.budgets([L], cfg)[0]
            K = min(math.floor(np.float32(0.34) * Ly * H), b["alloc"] // L)
            assert b["full_units"] == K and b["rest"] == b["alloc"] - K * L
            order = np.lexsort((np.arange(Ly * H), -sens[s].reshape(-1)))
            want = np.zeros(Ly * H, dtype=bool)
            want[order[:K]] = True
            assert np.array_equal(full[s].reshape(-1), want), (trial, s)
    # f = 0 keeps nothing whole
    cfg0 = _cfg(Ly=2, H=3, lens=[8])
    assert not osel.hybrid_units(np.ones((1, 2, 3), np.float32), np.array([0, 8]), cfg0).any()


def test_hybrid_token_mode_keeps_whole_heads_and_tops_the_rest():
    rng = np.random.default_rng(22)
    for trial in range(20):
        Ly, H, L = 2, 3, int(rng.integers(5, 30))
        rel = rng.integers(0, 5, (Ly, H, L)).astype(np.float32)
        sens = rng.random((1, Ly, H)).astype(np.float32)
        cfg = _hybrid_cfg(Ly=Ly, H=H, lens=[L], token_mode=True, budget_min=1,
                          budget_ratio=float(rng.uniform(0.2, 0.9)), hybrid_frac=0.34)
        cu = np.array([0, L])
        full = osel.hybrid_units(sens, cu, cfg)
        taken, spent = osel.token_topk(rel, cu, cfg, full)
        b = common.budgets([L], cfg)[0]
        K = int(full.sum())
        assert K == b["full_units"]
        assert np.all(taken[full[0]] == 1)
        # the rest: a top set of (rel desc, flat id asc) over the other units
        ids = [(l * H + h) * L + i for l in range(Ly) for h in range(H) if not full[0, l, h] for i in range(L)]
        vals = np.array([rel.reshape(-1)[f] for f in ids])
        order = np.lexsort((np.array(ids), -vals))
        k = min(b["rest"], len(ids))
        want = np.zeros(Ly * H * L, dtype=np.uint8)
        want[np.array(ids)[order[:k]]] = 1
        want.reshape(Ly, H, L)[full[0]] = 1
        assert np.array_equal(taken.reshape(-1), want), trial
        assert spent[0] == K * L + k


def test_hybrid_auction_equals_the_greedy_over_the_other_heads():
    rng = np.random.default_rng(23)
    for trial in range(25):
        lens, starts, T, _, _, _ = _random_forest(rng, int(rng.integers(1, 4)), False)
        H = 3
        util = np.zeros((1, H, 2 * T), dtype=np.float32)
        cost = np.zeros((1, H, 2 * T), dtype=np.uint8)
        slots_ops_all = []
        for h in range(H):
            for st, n in zip(starts, lens):
                nodes = otrees.tree_nodes(st, n)
                base = h * 2 * T + 2 * st
                slots_ops_all.append((h, base, nodes))
                cost[0, h, 2 * st] = 1
                util[0, h, 2 * st] = rng.standard_normal()
                for j, nd in enumerate(nodes):
                    if nd[2] >= 0:
                        cost[0, h, 2 * st + 1 + j] = 1
                        util[0, h, 2 * st + 1 + j] = rng.standard_normal()
        sens = rng.random((1, 1, H)).astype(np.float32)
        for B in (T, T + 1, T + 4, 2 * T, 3 * T):
            cfg = _hybrid_cfg(H=H, lens=[T], slot_len=0, budget_ratio=0.0, budget_min=B,
                              floor_frac=0.0, hybrid_frac=0.34)
            slots = [[(st, n) for st, n in zip(starts, lens)]]
            cu = np.array([0, T])
            full = osel.hybrid_units(sens, cu, cfg)
            fh = int(np.argmax(full[0, 0]))
            assert full.sum() == 1 and full[0, 0, fh] == (sens[0, 0, fh] == sens[0, 0].max())
            ftaken, fspent = osel.floor_select(util * 0 + 1, sens, cost, cu, slots, cfg, full=full)
            assert fspent[0] == 0
            got, spent = osel.auction(util, cost, ftaken, fspent, cu, slots, cfg, full=full)
            # brute force: the whole head's real ops up front, then the literal
            # greedy over the other heads with what is left
            taken0 = np.zeros(H * 2 * T, dtype=np.uint8)
            taken0[fh * 2 * T:(fh + 1) * 2 * T] = cost[0, fh] > 0
            others = [(base, nodes) for h, base, nodes in slots_ops_all if h != fh]
            want, _ = _greedy_by_enumeration(util.reshape(-1), cost.reshape(-1), taken0, others, B - T)
            assert np.array_equal(got.reshape(-1), want), (trial, B)
            other_ops = int(cost.sum()) - T
            assert spent[0] == T + min(B - T, other_ops)


def test_hybrid_floor_skips_whole_heads_and_caps_on_the_rest():
    L = 32
    H = 3
    slots = [[(0, 16), (16, 16)]]
    cost = np.zeros((1, H, 2 * L), dtype=np.uint8)
    for h in range(H):
        for st in (0, 16):
            nodes = otrees.tree_nodes(st, 16)
            cost[0, h, 2 * st] = 1
            for j, nd in enumerate(nodes):
                if nd[2] >= 0:
                    cost[0, h, 2 * st + 1 + j] = 1
    rel = np.zeros((1, H, L), dtype=np.float32)
    rel[0, 0, 5] = 9.0          # the best leaf sits in the head kept whole
    rel[0, 1, 7] = 2.0
    rel[0, 2, 20] = 1.0
    sens = np.array([[[3.0, 1.0, 1.0]]], dtype=np.float32)
    cfg = _hybrid_cfg(H=H, lens=[L], slot_len=16, budget_ratio=0.0, budget_min=L + 20,
                      floor_frac=0.5, hybrid_frac=0.34)
    cu = np.array([0, L])
    full = osel.hybrid_units(sens, cu, cfg)
    assert full[0, 0, 0] and full.sum() == 1
    b = common.budgets([L], cfg)[0]
    assert b["rest"] == 20 and b["floor"] == 10
    tr = []
    ftaken, fspent = osel.floor_select(rel, sens, cost, cu, slots, cfg, trace=tr, full=full)
    assert not ftaken[0, 0].any()
    # head 1 token 7: Add + 4 splits = 5; head 2 token 20: 5 more -> 10 = F;
    # later candidates are only those whose path is already paid (token 6
    # shares token 7's last split)
    assert [t[0] for t in tr[:2]] == [1 * L + 7, 2 * L + 20] and fspent[0] == 10
    assert all(c == 0 for _, c in tr[2:]) and (1 * L + 6, 0) in tr[2:]


# ---------------------------------------------------------------- "A r" propagation (NEXT 3)
def test_ar_propagation_matrix_form_and_constant():
    from oracle.propagate import propagate_ar
    rng = np.random.default_rng(31)
    L, d, G = 30, 8, 2
    K = rng.standard_normal((L, d))
    Qc = rng.standard_normal((G, L, d))
    r0 = rng.random(L).astype(np.float32)
    w = 0.3
    cfg = _cfg(G=G, d=d, lens=[L], n_hops=2, hop_weight=w)
    out = propagate_ar(torch.tensor(K.reshape(1, 1, L, d)), torch.tensor(Qc.reshape(1, G, L, d)),
                       r0.reshape(1, 1, L), np.array([0, L]), cfg)
    # library softmax per query head, causal; rows are the attending tokens
    logits = np.einsum("gjd,id->gji", Qc, K) / math.sqrt(d)
    logits = np.where(np.tril(np.ones((L, L)))[None] > 0, logits, -np.inf)
    Ahat = scipy.special.softmax(logits, axis=2).mean(0)          # [i attending, j attended]
    wf = float(np.float32(w))
    r = r0.astype(np.float64)
    d1 = wf * Ahat @ r
    d2 = wf * Ahat @ d1
    assert np.allclose(out["rel"][0, 0], r + d1 + d2, rtol=1e-6)
    # every row is a convex average: a constant increment passes on as w * c,
    # and the first token can only take its own value
    outc = propagate_ar(torch.tensor(K.reshape(1, 1, L, d)), torch.tensor(Qc.reshape(1, G, L, d)),
                        np.full((1, 1, L), 2.0, np.float32), np.array([0, L]), cfg.replace(n_hops=1))
    assert np.allclose(outc["rel"][0, 0], 2.0 + wf * 2.0, rtol=1e-6)
    assert abs(d1[0] - wf * r[0]) < 1e-12


# ---------------------------------------------------------------- multi-depth turns and surprisal (NEXT 1)
def test_partition_depths_and_surprisal_compose():
    rng = np.random.default_rng(41)
    L, Dh = 96, 16
    cfg = _cfg(lens=[L], slot_len=0, slot_min=4, slot_max=12, slot_target=8, lambda_surp=1.0)
    cu = np.array([0, L])
    h1 = rng.standard_normal((L, Dh))
    h2 = rng.standard_normal((L, Dh))
    c1, k1 = opart.slot_costs(h1, cu, cfg)
    c2, k2 = opart.slot_costs(h2, cu, cfg)
    # identical depths reproduce the single trajectory (up to one quantum)
    cs, ks = opart.slot_costs(np.stack([h1, h1, h1]), cu, cfg)
    assert np.abs(cs - c1).max() <= 1 and np.abs(ks - k1).max() <= 1
    # two depths: the mean of the two dispersions (the length term once), and
    # where both windows are valid at both depths the mean of the two turns
    cm, km = opart.slot_costs(np.stack([h1, h2]), cu, cfg)
    valid = c1 != 0
    assert np.abs(cm[valid] - (c1[valid] + c2[valid]) / 2).max() <= 1
    inner = slice(8, L - 8)
    assert np.abs(km[inner] - (k1[inner] + k2[inner]) / 2).max() <= 1
    # surprisal: lambda_surp * s / max s on top of the turning bonus
    sur = rng.random(L) * 3.0
    cs2, ks2 = opart.slot_costs(h1, cu, cfg, surprisal=sur)
    assert np.array_equal(cs2, c1)
    want = np.array([opart._q(float(np.float32(cfg.lambda_surp)) * sur[b] / sur.max()) for b in range(L)])
    assert np.abs(ks2 - k1 - want).max() <= 1
    # a non-positive surprisal maximum adds nothing
    _, ks3 = opart.slot_costs(h1, cu, cfg, surprisal=np.zeros(L))
    assert np.array_equal(ks3, k1)
