"""Pins of oracle parts that the first pin set left open, each with the slips it
catches planted in the oracle (on the CPU, through monkeypatch) to show that
the pin fails when the slip is there.

Parts pinned here:
* the operations' utilities (GraceKV page, '04 Top-down budget flow': an
  operation's utility is the relevance-weighted fidelity it adds per new
  entry; dropping a slot counts as full distortion) against the decrease of
  the loss sum over the slot's whole frontier, evaluated frontier by frontier;
* the distortion's probe rows (every (G*P // P_d)-th probe row);
* pack's prototype rows (GraceKV page, 'Inside one cache entry' and '05
  Physical cache packing') against the tree stage's prototypes and against
  closed forms (coherent keys give ln mu = ln n and the re-rotated key; a
  single relevant token gets weight 0.9 + 0.1/n; a merged entry with
  multiplicity n decodes like n copies of itself);
* the token regions of a sequence (GraceKV page, 'Core idea' and
  'Exact-information safeguard': prompt and suffix exact outside the budget,
  a recent window exact inside it) as hand-computed tuples;
* the turning score of a cut (GraceKV page, '01 Curvature-guided partition':
  turns of the normalized trajectory are good boundaries) on a straight line,
  a right angle and a reversal.
"""
import math

import numpy as np
import pytest

import importlib

import oracle
from oracle import common, trees as otrees, partition as opart, decode as odec
from oracle.pack import _frontier

opack = importlib.import_module("oracle.pack")  # the package re-exports a function of the same name
from workload import Config


def _cfg(**kw):
    base = dict(name="t", S=1, Ly=1, H=1, G=2, d=8, lens=[40], dtype="f32", rope_base=1e4,
                P=4, slot_len=8, T_dec=1, vocab=64, w_dtype="f32", plant="evidence", n_plant=0)
    base.update(kw)
    return Config(**base)


def _rope_complex(k, p, d, base):
    """Rotate-half RoPE as complex multiplication: pair j = k_j + i k_{j+d/2}
    times e^{i p base^(-2j/d)} (written independently of the oracle's rope)."""
    h = d // 2
    z = (np.asarray(k[:h]) + 1j * np.asarray(k[h:])) * np.exp(1j * p * base ** (-2.0 * np.arange(h) / d))
    return np.concatenate([z.real, z.imag])


# ================================================================ utilities
def _small_trees(seed, zero_queries=False, identical=False):
    """One sequence, one (layer, KV head), slots of 8/13/5 tokens."""
    cfg = _cfg(lens=[26], slot_len=0)
    rng = np.random.default_rng(seed)
    T, d = 26, 8
    import torch
    if identical:
        k0, v0 = rng.standard_normal(d), rng.standard_normal(d)
        K = np.stack([_rope_complex(k0, i, d, cfg.rope_base) for i in range(T)])
        V = np.tile(v0, (T, 1))
        r = np.full(T, 0.25)
    else:
        K, V, r = rng.standard_normal((T, d)), rng.standard_normal((T, d)), rng.random(T)
    Qp = rng.standard_normal((1, 1, cfg.G, cfg.P, d))
    if zero_queries:
        Qp[:] = 0.0
    lse = np.log(T) + rng.random((1, 1, cfg.G, cfg.P)) * (0 if zero_queries else 1)
    slots = [[(0, 8), (8, 13), (21, 5)]]
    sens = np.array([[[1.7]]], dtype=np.float32)
    out = otrees.build_trees(torch.from_numpy(K[None, None]), torch.from_numpy(V[None, None]),
                             torch.from_numpy(Qp), np.float32(lse), np.float32(r[None, None]), sens,
                             np.array([0, T]), slots, cfg)
    return cfg, slots, sens, out


def _loss(nodes, rel, D, sens, frontier):
    """Sum over the slot of sens * rel * D, an absent slot counting as its root
    with D = 1."""
    if frontier is None:
        return sens * rel[0]
    return sum(sens * rel[j] * D[j] for j in frontier)


def check_utilities(seed=0):
    _, slots, sens, out = _small_trees(seed)
    s = float(sens[0, 0, 0])
    for (st, n) in slots[0]:
        nodes = otrees.tree_nodes(st, n)
        base = 2 * st
        rel = out["node_rel"][0, 0, base:base + len(nodes)].astype(np.float64)
        D = out["node_D"][0, 0, base:base + len(nodes)].astype(np.float64)
        util = out["op_util"][0, 0, base:base + 2 * n]
        cost = out["op_cost"][0, 0, base:base + 2 * n]
        parent = {}
        for j, nd in enumerate(nodes):
            for c in nd[2:]:
                if c >= 0:
                    parent[c] = j
        # Add: from "absent" to the root alone
        # node values are read back as fp32 while the oracle forms the gains in
        # fp64, so the bar scales with the terms of the difference, not with it
        def near(u, before, after):
            tol = 4e-7 * (abs(before) + abs(after)) + 1e-12
            return abs(float(u) - (before - after)) <= tol + abs(float(u)) * 2 ** -23

        b, a = _loss(nodes, rel, D, s, None), _loss(nodes, rel, D, s, [0])
        assert cost[0] == 1
        assert near(util[0], b, a), ("Add", util[0], b - a)
        for j, (_, _, lc, rc) in enumerate(nodes):
            if lc < 0:
                assert cost[1 + j] == 0
                continue
            # the frontier that exposes Split(j): every ancestor of j split
            fr, a = [j], j
            while a in parent:
                p = parent[a]
                sib = [c for c in nodes[p][2:] if c != a]
                fr += sib
                a = p
            after = [x for x in fr if x != j] + [lc, rc]
            b, a = _loss(nodes, rel, D, s, fr), _loss(nodes, rel, D, s, after)
            assert cost[1 + j] == 1
            assert near(util[1 + j], b, a), ("Split", j, util[1 + j], b - a)


def check_utilities_closed_form():
    # identical tokens and zero query rows: every node's distortion is 0, so
    # Add gains sens * rel_root and every Split gains nothing
    _, slots, sens, out = _small_trees(3, zero_queries=True, identical=True)
    s = float(sens[0, 0, 0])
    for (st, n) in slots[0]:
        base = 2 * st
        # (0 up to the fp64 round-off of the key means and exponentials)
        assert np.all(np.abs(out["node_D"][0, 0, base:base + 2 * n - 1]) <= 1e-12)
        assert out["op_util"][0, 0, base] == pytest.approx(s * 0.25 * n, rel=1e-6)
        assert np.all(np.abs(out["op_util"][0, 0, base + 1:base + 2 * n]) <= 1e-12)


def test_utilities_are_the_frontier_loss_decrease():
    for seed in range(4):
        check_utilities(seed)
    check_utilities_closed_form()


def _slipped_utilities(kind):
    def f(nodes, rel, D, sens):
        m = len(nodes)
        util = np.zeros(m + 1, dtype=np.float32)
        cost = np.zeros(m + 1, dtype=np.uint8)
        add = rel[0] * D[0] if kind == "add_uses_D" else rel[0] * (1.0 - D[0])
        util[0] = np.float32((1.0 if kind == "no_sens" else sens) * add)
        cost[0] = 1
        for j, (_, _, ch, _) in enumerate(nodes):
            if not ch:
                continue
            lc, rc = ch
            if kind == "split_sign":
                g = (rel[lc] * D[lc] + rel[rc] * D[rc]) - rel[j] * D[j]
            elif kind == "split_child_swap":
                g = rel[j] * D[j] - (rel[lc] * D[rc] + rel[rc] * D[lc])
            elif kind == "split_parent_D":
                g = rel[j] * D[j] - (rel[lc] + rel[rc]) * D[j] * 0.5
            else:
                g = rel[j] * D[j] - (rel[lc] * D[lc] + rel[rc] * D[rc])
            util[1 + j] = np.float32((1.0 if kind == "no_sens" else sens) * g)
            cost[1 + j] = 1
        return util, cost
    return f


@pytest.mark.parametrize("kind", ["add_uses_D", "no_sens", "split_sign", "split_child_swap", "split_parent_D"])
def test_utility_slips_fail_the_pin(monkeypatch, kind):
    monkeypatch.setattr(otrees, "op_utilities", _slipped_utilities(kind))
    with pytest.raises(AssertionError):
        check_utilities(0)
        check_utilities(1)
        check_utilities_closed_form()


# ================================================================ distortion rows
DPROBE_CASES = [
    # (G, P, n_dprobe) -> rows rho = g*P + p, written out
    ((4, 64, 64), list(range(0, 256, 4))),
    ((4, 64, 48), list(range(0, 240, 5))),
    ((4, 64, 20), list(range(0, 240, 12))),
    ((4, 64, 1), [0]),
    ((4, 16, 64), list(range(64))),
    ((2, 4, 64), list(range(8))),
    ((8, 32, 64), list(range(0, 256, 4))),
    ((1, 64, 16), list(range(0, 64, 4))),
]


def check_dprobe_rows():
    for (G, P, nd), want in DPROBE_CASES:
        got = [int(x) for x in otrees.dprobe_rows(_cfg(G=G, P=P, n_dprobe=nd))]
        assert got == want, ((G, P, nd), got[:8])


def test_distortion_rows_are_every_stride_th_probe_row():
    check_dprobe_rows()


@pytest.mark.parametrize("kind", ["stride_over_P", "start_at_one", "ceil_stride", "first_rows"])
def test_dprobe_slips_fail_the_pin(monkeypatch, kind):
    def slipped(cfg):
        R = cfg.G * cfg.P
        Pd = min(cfg.n_dprobe, R)
        if kind == "stride_over_P":
            st = max(1, cfg.P // Pd)
            return np.arange(0, R, st)[:Pd]
        if kind == "start_at_one":
            st = R // Pd
            return np.arange(1, R, st)[:Pd]
        if kind == "ceil_stride":
            st = -(-R // Pd)
            return np.arange(0, R, st)[:Pd]
        return np.arange(Pd)
    monkeypatch.setattr(otrees, "dprobe_rows", slipped)
    with pytest.raises(AssertionError):
        check_dprobe_rows()


# ================================================================ pack's prototypes
def _pack_setup(seed=0, coherent=False, one_relevant=False):
    """One (layer, KV head), fixed 8-token slots over 40 tokens; a taken set
    that leaves internal nodes of several sizes on the frontier."""
    import torch
    cfg = _cfg(lens=[40], slot_len=8, dtype="f32")
    rng = np.random.default_rng(seed)
    T, d = 40, 8
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    r = rng.random(T)
    k0 = rng.standard_normal(d)
    v0 = np.round(rng.standard_normal(d) * 8) / 8
    if coherent:
        K = np.stack([_rope_complex(k0, i, d, cfg.rope_base) for i in range(T)])
        V = np.tile(v0, (T, 1))
    if one_relevant:
        r = np.zeros(T)
        r[[1, 10, 19, 28, 37]] = 1.0
    Qp = rng.standard_normal((1, 1, cfg.G, cfg.P, d))
    lse = np.float32(np.log(T) + rng.random((1, 1, cfg.G, cfg.P)))
    slots = oracle.slots_for(np.array([0, T]), cfg)
    sens = np.array([[[1.0]]], dtype=np.float32)
    Kt, Vt = torch.from_numpy(K[None, None]), torch.from_numpy(V[None, None])
    rel = np.float32(r[None, None])
    tr = otrees.build_trees(Kt, Vt, torch.from_numpy(Qp), lse, rel, sens, np.array([0, T]), slots, cfg,
                            keep_protos=True)
    taken = np.zeros((1, 1, 2 * T), dtype=np.uint8)
    for k, (st, n) in enumerate(slots[0]):
        base = 2 * st
        nodes = otrees.tree_nodes(st, n)
        taken[0, 0, base] = 1                       # Add: the root
        if k % 3 == 1:
            taken[0, 0, base + 1] = 1               # split the root: two 4-token nodes
        if k % 3 == 2:
            taken[0, 0, base + 1] = 1
            taken[0, 0, base + 1 + nodes[0][2]] = 1  # and its left child: 2 + 2 + 4
    pk = opack.pack(Kt, Vt, rel, tr, taken, np.array([0, T]), slots, cfg)
    return cfg, slots, K, V, r, tr, taken, pk


def _internal_entries(slots, taken, tr, pk):
    """(entry index, node, slot start) of every internal frontier node, in
    pack's order (positions ascending)."""
    out = []
    e = 0
    for (st, n) in slots[0]:
        nodes = otrees.slot_tree(st, n)
        for j in _frontier(nodes, taken.reshape(-1), 2 * st):
            if nodes[j][1] > 1:
                out.append((e, j, st))
            e += 1
    return out


def check_pack_against_tree_prototypes(seed=0):
    cfg, slots, K, V, r, tr, taken, pk = _pack_setup(seed)
    ents = _internal_entries(slots, taken, tr, pk)
    assert len(ents) >= 8
    for e, j, st in ents:
        pr = tr["protos"][(0, 0, 0, st)]
        a, m = pr["nodes"][j][0], pr["nodes"][j][1]
        assert np.array_equal(pk["K"][e], common.round_to(pr["khat"][j], cfg.dtype)), ("k", st, j)
        # pack normalizes the value weights by the stored (fp32) node relevance,
        # the tree stage by its fp64 sum: two fp32 ulps apart at most
        vt = common.round_to(pr["vhat"][j], cfg.dtype)
        assert np.all(np.abs(pk["V"][e] - vt) <= 2.0 ** -22 * np.abs(vt) + 1e-12), ("v", st, j)
        lm = np.float32(math.log(pr["mu"][j]))   # pack logs the stored fp32 mu
        assert abs(float(pk["lnmu"][e]) - float(lm)) <= 2.0 ** -22 * abs(float(lm)) + 2.0 ** -24, ("lnmu", st, j)
        assert pk["pos"][e] == a + (m - 1) // 2, ("pos", st, j)


def check_pack_closed_forms(seed=0):
    # coherent keys K_i = RoPE(k0, i) and one value v0: each prototype is
    # RoPE(k0, p_rep) with ln mu = ln n and value v0
    cfg, slots, K, V, r, tr, taken, pk = _pack_setup(seed, coherent=True)
    k0 = None
    for e, j, st in _internal_entries(slots, taken, tr, pk):
        nodes = otrees.tree_nodes(st, dict(slots[0])[st])
        a, m = nodes[j][0], nodes[j][1]
        p = a + (m - 1) // 2
        # k0 recovered from token 0 by the inverse rotation (complex form)
        if k0 is None:
            k0 = _rope_complex(K[0], -0, 8, cfg.rope_base)
        want_k = _rope_complex(k0, p, 8, cfg.rope_base)
        # the packed key is rounded to the cache dtype (fp32 here)
        assert np.all(np.abs(pk["K"][e] - want_k) <= 2.0 ** -23 * np.abs(want_k) + 1e-12), ("k", st, j)
        # the weights are normalized by the stored fp32 node relevance, so they
        # sum to 1 within two fp32 ulps
        assert np.all(np.abs(pk["V"][e] - V[0]) <= 2.0 ** -22 * np.abs(V[0]) + 1e-13), ("v", st, j)
        assert abs(pk["lnmu"][e] - np.float32(math.log(m))) <= 2e-7 * math.log(m) + 1e-7, ("lnmu", m, pk["lnmu"][e])
        assert pk["pos"][e] == p
    # one relevant token per slot: its weight is 0.9 + 0.1/m, the others 0.1/m
    cfg, slots, K, V, r, tr, taken, pk = _pack_setup(seed, one_relevant=True)
    for e, j, st in _internal_entries(slots, taken, tr, pk):
        nodes = otrees.tree_nodes(st, dict(slots[0])[st])
        a, m = nodes[j][0], nodes[j][1]
        seg = slice(a, a + m)
        if r[seg].sum() > 0:
            want = 0.9 * (r[seg] / r[seg].sum()) @ V[seg] + 0.1 * V[seg].mean(0)
        else:
            want = V[seg].mean(0)
        assert np.all(np.abs(pk["V"][e] - want) <= 2.0 ** -22 * np.abs(want) + 1e-12), ("v weights", st, j)


def check_merged_entry_decodes_like_copies(seed=0):
    # a packed entry with multiplicity n counts for n identical tokens
    cfg, slots, K, V, r, tr, taken, pk = _pack_setup(seed, coherent=True)
    ents = _internal_entries(slots, taken, tr, pk)
    rng = np.random.default_rng(seed + 11)
    d = 8
    q = rng.standard_normal((1, 1, cfg.G, d))
    Kd = np.zeros((1, 1, 1, 1, d))
    Vd = np.zeros((1, 1, 1, 1, d))
    # expand every internal entry into mu copies with ln mu = 0
    Ks, Vs = [], []
    for e in range(pk["K"].shape[0]):
        reps = 1
        for (ee, j, st) in ents:
            if ee == e:
                reps = int(round(math.exp(float(pk["lnmu"][e]))))
        Ks += [pk["K"][e]] * reps
        Vs += [pk["V"][e]] * reps
    N = len(Ks)
    expanded = {"K": np.array(Ks), "V": np.array(Vs), "lnmu": np.zeros(N, dtype=np.float32),
                "seg_off": np.zeros((1, 1, 1), dtype=np.int64), "seg_len": np.full((1, 1, 1), N, dtype=np.int32)}
    import torch
    x1, _ = odec.decode_step(pk, torch.from_numpy(Kd), torch.from_numpy(Vd), torch.from_numpy(q), 0, cfg.G)
    x2, _ = odec.decode_step(expanded, torch.from_numpy(Kd), torch.from_numpy(Vd), torch.from_numpy(q), 0, cfg.G)
    # ln mu is stored as fp32: exp(lnmu) equals n to 1e-7 relative
    assert np.allclose(x1, x2, rtol=1e-6, atol=1e-9), np.abs(x1 - x2).max()


def test_pack_prototypes_match_the_tree_stage_and_closed_forms():
    for seed in range(3):
        check_pack_against_tree_prototypes(seed)
        check_pack_closed_forms(seed)
        check_merged_entry_decodes_like_copies(seed)


def _slipped_prototype(kind):
    from oracle.common import rope, rope_inv, round_to

    def f(Ku, Vu, r, a, m, rel, mu, cfg):
        beta = float(np.float32(cfg.value_base))
        pos = np.arange(a, a + m, dtype=np.float64)
        kt = (rope if kind == "rotate_not_unrotate" else rope_inv)(Ku[a:a + m], pos, cfg.rope_base).mean(axis=0)
        prep = a + (m // 2 if kind == "upper_midpoint" else (m - 1) // 2)
        kh = rope(kt, prep, cfg.rope_base)
        if kind == "beta_swapped":
            w = beta * r[a:a + m] / rel + (1.0 - beta) / m if rel > 0 else np.full(m, 1.0 / m)
        else:
            w = (1.0 - beta) * r[a:a + m] / rel + beta / m if rel > 0 else np.full(m, 1.0 / m)
        vh = w @ Vu[a:a + m]
        lm = float(np.float32(mu if kind == "mu_not_log" else np.log(mu)))
        return round_to(kh, cfg.dtype), round_to(vh, cfg.dtype), lm, prep
    return f


@pytest.mark.parametrize("kind", ["rotate_not_unrotate", "upper_midpoint", "beta_swapped", "mu_not_log"])
def test_pack_prototype_slips_fail_the_pin(monkeypatch, kind):
    monkeypatch.setattr(opack, "prototype_entry", _slipped_prototype(kind))
    with pytest.raises(AssertionError):
        check_pack_against_tree_prototypes(0)
        check_pack_closed_forms(0)


# ================================================================ regions
# (L, prompt, recent, suffix) -> (prompt_end, comp_start, comp_end, suffix_start),
# computed by hand from: prompt first, then the suffix (never into the prompt),
# then the recent window before the suffix (never into the prompt).
REGION_CASES = [
    ((2053, 256, 128, 256), (256, 256, 1669, 1797)),
    ((29761, 256, 128, 256), (256, 256, 29377, 29505)),
    ((641, 256, 128, 256), (256, 256, 257, 385)),
    ((640, 256, 128, 256), (256, 256, 256, 384)),
    ((600, 256, 128, 256), (256, 256, 256, 344)),
    ((512, 256, 128, 256), (256, 256, 256, 256)),
    ((300, 256, 128, 256), (256, 256, 256, 256)),
    ((100, 256, 128, 256), (100, 100, 100, 100)),
    ((0, 256, 128, 256), (0, 0, 0, 0)),
    ((1100, 64, 32, 48), (64, 64, 1020, 1052)),
    ((16384, 0, 0, 0), (0, 0, 16384, 16384)),
    ((40, 0, 32, 0), (0, 0, 8, 40)),
    ((20, 0, 32, 0), (0, 0, 0, 20)),
]


def check_regions():
    for (L, pe, rc, sf), want in REGION_CASES:
        cfg = _cfg(prompt_exact=pe, recent_exact=rc, suffix_exact=sf)
        assert tuple(common.regions(L, cfg)) == want, ((L, pe, rc, sf), common.regions(L, cfg), want)


def test_regions_hand_computed():
    check_regions()


@pytest.mark.parametrize("kind", ["recent_before_suffix", "suffix_into_prompt", "recent_unclamped"])
def test_region_slips_fail_the_pin(monkeypatch, kind):
    def slipped(L, cfg):
        pe = min(cfg.prompt_exact, L)
        if kind == "recent_before_suffix":
            rs = max(pe, L - cfg.recent_exact)
            ss = max(rs, L - cfg.suffix_exact)
            return pe, pe, min(rs, ss), ss
        if kind == "suffix_into_prompt":
            ss = max(0, L - cfg.suffix_exact)
            rs = max(pe, ss - cfg.recent_exact)
            return pe, pe, rs, ss
        ss = max(pe, L - cfg.suffix_exact)
        return pe, pe, ss - cfg.recent_exact, ss
    monkeypatch.setattr(common, "regions", slipped)
    with pytest.raises(AssertionError):
        check_regions()


# ================================================================ turning score
def _turn_path(L, b, kind, dim=3):
    """Points along x up to b, then along y (right angle), back along x
    (reversal), or on along x (straight line)."""
    P = np.zeros((L, dim))
    for i in range(L):
        if i <= b or kind == "straight":
            P[i, 0] = i
        elif kind == "right":
            P[i, 0], P[i, 1] = b, i - b
        elif kind == "reverse":
            P[i, 0] = 2 * b - i
    return P


def check_turning():
    L = 40
    for kind, want in (("straight", 0.0), ("right", 0.5), ("reverse", 1.0)):
        for b in (10, 20, 31):          # both windows valid (b - 8 >= 0, b + 8 <= L - 1)
            assert opart.turning_score(_turn_path(L, b, kind), b) == pytest.approx(want, abs=1e-15), (kind, b)
    # only the 2-token window is valid at b = 4 and at b = L - 1 - 7; it sees
    # the turn, so the mean over valid windows is its value alone
    for b in (4, L - 1 - 7):
        assert opart.turning_score(_turn_path(L, b, "right"), b) == pytest.approx(0.5, abs=1e-15), b
    # b = L - 1 - 8 is the last position where the 8-token window is valid:
    # a turn 2 tokens after b is seen by it (a quarter turn of the chord)
    b = L - 1 - 8
    P = _turn_path(L, b + 2, "right")
    u, v = P[b] - P[b - 8], P[b + 8] - P[b]
    w8 = (1 - u @ v / (np.linalg.norm(u) * np.linalg.norm(v))) / 2
    assert opart.turning_score(P, b) == pytest.approx((0.0 + w8) / 2, abs=1e-15)
    # no valid window: 0
    assert opart.turning_score(_turn_path(3, 1, "right"), 1) == 0.0
    # a repeated point (zero difference) drops that window
    P = _turn_path(L, 20, "right")
    P[18] = P[20]
    assert opart.turning_score(P, 20) == pytest.approx(0.5, abs=1e-15)


def test_turning_score_closed_forms():
    check_turning()


@pytest.mark.parametrize("kind", ["sign_flipped", "no_half", "window_bound", "sum_not_mean"])
def test_turning_slips_fail_the_pin(monkeypatch, kind):
    orig = opart.turning_values

    def slipped(hn, b):
        L = hn.shape[0]
        vals = []
        for w in opart.WINDOWS:
            hi = L if kind == "window_bound" else L - 1
            if b - w < 0 or b + w > hi:
                continue
            if b + w >= L:
                vals.append(0.0)
                continue
            u = hn[b] - hn[b - w]
            v = hn[b + w] - hn[b]
            nu, nv = np.linalg.norm(u), np.linalg.norm(v)
            if nu == 0 or nv == 0:
                continue
            c = float(u @ v) / (nu * nv)
            if kind == "sign_flipped":
                vals.append((1.0 + c) / 2.0)
            elif kind == "no_half":
                vals.append(1.0 - c)
            else:
                vals.append((1.0 - c) / 2.0)
        if kind == "sum_not_mean":
            return [sum(vals)] if vals else []
        return vals
    monkeypatch.setattr(opart, "turning_values", slipped)
    with pytest.raises(AssertionError):
        check_turning()
    monkeypatch.setattr(opart, "turning_values", orig)
    check_turning()
