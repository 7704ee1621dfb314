"""GPU stage parity: every integer stage is bit-exact when fed the oracle's
inputs to that stage (top-B, floor + auction, DP cuts, pack indices, order and
leaf copies); float stages (trees, prototypes, DP costs) within tolerance.
All calls go through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from oracle import partition as opart
from workload import small_config, make_inputs
from parity import (close, as_np, to_dev, inputs_to, slots_to_dev, slots_from_dev, trees_to_dev, topo_np)

pytestmark = pytest.mark.gpu


def _kvc():
    from eviction_probe_softmax_amd import kvc
    return kvc


def _oracle_front(cfg, inp):
    cu = inp["cu_seqlens"].numpy()
    sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    pr = oracle.propagate(inp["K"], inp["Qctx"], sc["r0"], cu, cfg)
    return cu, sc, pr


def _full(cfg, cu, sc):
    return oracle.select.hybrid_units(sc["head_sens"], cu, cfg) if cfg.hybrid_frac > 0 else None


@pytest.mark.parametrize("name,kw", [("mistral1", {}), ("ragged", {"token_mode": True, "slot_len": 0}),
                                     ("mistral1", {"budget_ratio": 0.9}),
                                     ("mistral1", {"hybrid_frac": 0.5, "budget_ratio": 0.6}),
                                     ("ragged", {"token_mode": True, "slot_len": 0, "hybrid_frac": 0.5})])
def test_token_topk_and_pack_bit_exact(name, kw):
    kvc = _kvc()
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    print(f"[token] {name} {kw}", flush=True)
    cu, sc, pr = _oracle_front(cfg, inp)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    rel = to_dev(pr["rel"])
    g = kvc.auction(pb, rel=rel, head_sens=to_dev(sc["head_sens"]))
    full = _full(cfg, cu, sc)
    if cfg.hybrid_frac > 0:
        assert np.array_equal(as_np(kvc.hybrid_units(pb, to_dev(sc["head_sens"]))).astype(bool), full)
    otaken, ospent = oracle.token_topk(pr["rel"], cu, cfg, full)
    assert np.array_equal(as_np(g["taken"]), otaken)
    assert np.array_equal(as_np(g["spent"]), ospent)
    c = kvc.pack(pb, dinp["K"], dinp["V"], rel, None, g["taken"], None, None, None, None)
    oc = oracle.pack(inp["K"], inp["V"], pr["rel"], None, otaken, cu, [[]] * cfg.S, cfg)
    _compare_cache(c, oc, exact=True)


def _compare_cache(c, oc, exact):
    assert np.array_equal(as_np(c["seg_off"]), oc["seg_off"])
    assert np.array_equal(as_np(c["seg_len"]), oc["seg_len"])
    N = oc["K"].shape[0]
    assert np.array_equal(as_np(c["pos"])[:N], oc["pos"])
    gk, gv = as_np(c["K"])[:N].astype(np.float64), as_np(c["V"])[:N].astype(np.float64)
    lm = as_np(c["lnmu"])[:N]
    if exact:
        assert np.array_equal(gk, oc["K"]) and np.array_equal(gv, oc["V"])
        assert np.all(lm == 0)
        return
    leaf = oc["lnmu"] == 0
    # token leaves are bit copies of the cache
    assert np.array_equal(gk[leaf], oc["K"][leaf]) and np.array_equal(gv[leaf], oc["V"][leaf])
    close(gk, oc["K"], 2e-2, "packed K", floor=1e-2)
    close(gv, oc["V"], 2e-2, "packed V", floor=1e-2)
    close(lm, oc["lnmu"], 1e-3, "ln mu", floor=1e-3)




@pytest.mark.parametrize("name,kw", [("tiny", {}), ("stress", {}), ("ragged", {}), ("fulldepth", {}),
                                     ("stress", {"slot_len": 128}),
                                     ("fulldepth", {"slot_min": 64, "slot_max": 128, "slot_target": 120}),
                                     ("tiny", {"slot_len": 128}),
                                     ("fulldepth", {"slot_min": 8, "slot_max": 64, "slot_target": 40}),
                                     ("tiny", {"split_mode": 1}), ("fulldepth", {"split_mode": 1}),
                                     ("ragged", {"split_mode": 1}),
                                     ("fulldepth", {"split_mode": 1, "slot_min": 64, "slot_max": 128,
                                                    "slot_target": 120}),
                                     ("tiny", {"split_mode": 1, "slot_len": 128})])
def test_trees_match_oracle(name, kw):
    kvc = _kvc()
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    print(f"[trees] {name} {kw}", flush=True)
    cu, sc, pr = _oracle_front(cfg, inp)
    cq = kq = None
    if cfg.slot_len == 0:
        cq, kq = opart.slot_costs(inp["hidden"], cu, cfg)
    slots = oracle.slots_for(cu, cfg, cq, kq)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    ss, ns = slots_to_dev(slots, pb.slot_stride())
    rc, rs = kvc.rope_table(cfg.rope_base, cfg.d, max(cfg.lens))
    g = kvc.build_trees(pb, dinp["K"], dinp["V"], dinp["Qp"], to_dev(sc["lse"]), to_dev(pr["rel"]),
                        to_dev(sc["head_sens"]), rc, rs, ss, ns, cut_q=to_dev(kq) if cfg.split_mode else None)
    torch.cuda.synchronize()
    o = oracle.build_trees(inp["K"], inp["V"], inp["Qp"], sc["lse"], pr["rel"], sc["head_sens"], cu, slots, cfg,
                           cut_q=kq)
    if cfg.split_mode:   # the shapes: integer and fixed-order decisions on the same inputs, bit-exact
        gt = topo_np(g["node_topo"])
        print(f"  three-way splits {int((o['op_cost'] == 2).sum())}, nodes {int((o['node_topo'] != 0xFFFFFFFF).sum())}",
              flush=True)
        assert np.array_equal(gt, o["node_topo"])
    assert np.array_equal(as_np(g["op_cost"]), o["op_cost"])
    close(g["node_rel"], o["node_rel"], 1e-5, "node_rel")
    close(g["node_mu"], o["node_mu"], 1e-4, "node_mu")
    close(g["node_D"], o["node_D"], 1e-3, "node_D", floor=1e-3)
    close(g["op_util"], o["op_util"], 1e-3, "op_util", floor=1e-3)
    # P4 on the GPU output: parents are the exact fp32 sums of their children (left to right)
    nr = as_np(g["node_rel"])
    for s, lst in enumerate(slots):
        for (a, n) in lst[:3]:
            base = 2 * (int(cu[s]) + a)
            nodes = (oracle.trees.decode_topo(o["node_topo"][0, 0, base:base + 2 * n], a) if cfg.split_mode
                     else oracle.trees.slot_tree(a, n))
            for j, (_, _, ch, _) in enumerate(nodes):
                if ch:
                    acc = np.float32(nr[0, 0, base + ch[0]])
                    for c in ch[1:]:
                        acc = np.float32(acc + nr[0, 0, base + c])
                    assert nr[0, 0, base + j] == acc


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("stress", {}), ("ragged", {}), ("fulldepth", {}),
                                     ("stress", {"budget_ratio": 1.0 / 128, "floor_frac": 0.3}),
                                     ("ragged", {"floor_frac": 0.5}),
                                     ("fulldepth", {"hybrid_frac": 0.25, "budget_ratio": 0.4}),
                                     ("ragged", {"hybrid_frac": 0.5, "floor_frac": 0.3}),
                                     ("stress", {"hybrid_frac": 0.5}),
                                     ("tiny", {"hybrid_frac": 1.0, "budget_ratio": 1.0}),
                                     ("tiny", {"split_mode": 1}), ("tiny", {"split_mode": 1, "floor_frac": 0.3}),
                                     ("fulldepth", {"split_mode": 1}), ("ragged", {"split_mode": 1}),
                                     ("fulldepth", {"split_mode": 1, "hybrid_frac": 0.25, "budget_ratio": 0.4})])
def test_floor_and_auction_bit_exact(name, kw):
    kvc = _kvc()
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    print(f"[auction] {name} {kw}", flush=True)
    cu, sc, pr = _oracle_front(cfg, inp)
    cq = kq = None
    if cfg.slot_len == 0:
        cq, kq = opart.slot_costs(inp["hidden"], cu, cfg)
    slots = oracle.slots_for(cu, cfg, cq, kq)
    o = oracle.build_trees(inp["K"], inp["V"], inp["Qp"], sc["lse"], pr["rel"], sc["head_sens"], cu, slots, cfg,
                           cut_q=kq)
    full = _full(cfg, cu, sc)
    topo = o["node_topo"] if cfg.split_mode else None
    ft, fs = oracle.select.floor_select(pr["rel"], sc["head_sens"], o["op_cost"], cu, slots, cfg, full=full,
                                        topo=topo)
    taken, spent = oracle.select.auction(o["op_util"], o["op_cost"], ft, fs, cu, slots, cfg, full=full, topo=topo)
    if cfg.split_mode:
        print(f"  three-way splits {int((o['op_cost'] == 2).sum())}, taken {int(((o['op_cost'] == 2) & (taken > 0)).sum())}",
              flush=True)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    ss, ns = slots_to_dev(slots, pb.slot_stride())
    g = kvc.auction(pb, trees_to_dev(o), to_dev(pr["rel"]), to_dev(sc["head_sens"]), ss, ns)
    if full is not None:
        print(f"  units kept whole: {int(full.sum())}", flush=True)
    torch.cuda.synchronize()
    assert np.array_equal(as_np(g["spent_floor"]), fs), (as_np(g["spent_floor"]), fs)
    assert np.array_equal(as_np(g["spent"]), spent), (as_np(g["spent"]), spent)
    gt = as_np(g["taken"])
    assert np.array_equal(gt, taken), f"{int((gt != taken).sum())} ops differ"


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("stress", {}), ("ragged", {}), ("stress", {"slot_len": 128}),
                                     ("tiny", {"split_mode": 1}), ("tiny", {"split_mode": 1, "budget_ratio": 0.6}),
                                     ("ragged", {"split_mode": 1})])
def test_pack_tree_mode(name, kw):
    kvc = _kvc()
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    print(f"[pack] {name} {kw}", flush=True)
    cu, sc, pr = _oracle_front(cfg, inp)
    slots = oracle.slots_for(cu, cfg)
    o = oracle.build_trees(inp["K"], inp["V"], inp["Qp"], sc["lse"], pr["rel"], sc["head_sens"], cu, slots, cfg)
    topo = o["node_topo"] if cfg.split_mode else None
    ft, fs = oracle.select.floor_select(pr["rel"], sc["head_sens"], o["op_cost"], cu, slots, cfg, topo=topo)
    taken, spent = oracle.select.auction(o["op_util"], o["op_cost"], ft, fs, cu, slots, cfg, topo=topo)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    ss, ns = slots_to_dev(slots, pb.slot_stride())
    rc, rs = kvc.rope_table(cfg.rope_base, cfg.d, max(cfg.lens))
    c = kvc.pack(pb, dinp["K"], dinp["V"], to_dev(pr["rel"]), trees_to_dev(o), to_dev(taken), ss, ns, rc, rs)
    torch.cuda.synchronize()
    oc = oracle.pack(inp["K"], inp["V"], pr["rel"], o, taken, cu, slots, cfg)
    _compare_cache(c, oc, exact=False)


@pytest.mark.parametrize("name,kw", [("fulldepth", {}), ("fulldepth", {"lens": [300, 21, 517], "S": 3}),
                                     ("fulldepth", {"slot_min": 4, "slot_max": 12, "slot_target": 8}),
                                     ("fulldepth", {"n_depth": 3, "surprisal": True}),
                                     ("fulldepth", {"n_depth": 2, "surprisal": True, "lens": [300, 21, 517],
                                                    "S": 3, "lambda_surp": 0.5})])
def test_partition_dp(name, kw):
    kvc = _kvc()
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    print(f"[partition] {name} {kw}", flush=True)
    cu = inp["cu_seqlens"].numpy()
    cq, kq = opart.slot_costs(inp["hidden"], cu, cfg, inp.get("surprisal"))
    slots = oracle.slots_for(cu, cfg, cq, kq)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    # DP fed the oracle's quantized costs: identical cuts
    g = kvc.partition(pb, cost_q=to_dev(cq), cut_q=to_dev(kq), inject=True)
    assert slots_from_dev(g["slot_start"], g["n_slots"]) == slots
    # the GPU's own costs
    g2 = kvc.partition(pb, dinp["hidden"], cfg.hidden_dim, export=True, surprisal=dinp.get("surprisal"))
    torch.cuda.synchronize()
    gq = as_np(g2["dp_cost_q"]).astype(np.float64)
    valid = cq != 0
    err = np.abs(gq - cq)[valid]
    assert err.max() <= 1e-4 * np.abs(cq[valid]).max() + 64, err.max()
    gk = as_np(g2["dp_cut_q"]).astype(np.float64)
    assert np.abs(gk - kq).max() <= 1e-4 * (1 << 22) + 64
    # every region is covered by valid slots
    for s, lst in enumerate(slots_from_dev(g2["slot_start"], g2["n_slots"])):
        L = cfg.lens[s]
        pe, c0, c1, _ = oracle.regions(L, cfg)
        if c1 > c0:
            assert lst[0][0] == c0 and lst[-1][0] + lst[-1][1] == c1
            if c1 - c0 >= cfg.slot_min:
                assert all(cfg.slot_min <= n <= cfg.slot_max for _, n in lst)


def test_auction_with_three_way_splits_on_random_forests():
    """Cost-2 operations where the budget runs out on them: random tree
    shapes (binary and three-way splits) and utilities, every budget from a
    single entry to past the total, with and without a floor path taken up
    front; the GPU's threshold form, tie walk and extension against the
    oracle's best-first queue, bit-exact."""
    import test_oracle_pins_splits as sp
    from oracle import trees as otrees
    kvc = _kvc()
    rng = np.random.default_rng(31)
    n_short = 0
    for trial in range(24):
        lens, starts, T, util, cost, topo, slots_ops = sp._forest(rng, int(rng.integers(2, 6)), trial % 2 == 1)
        total = int(cost.sum())
        slots = [[(st, n) for st, n in zip(starts, lens)]]
        trees = {"node_rel": np.zeros((1, 1, 2 * T), np.float32), "node_D": np.zeros((1, 1, 2 * T), np.float32),
                 "node_mu": np.ones((1, 1, 2 * T), np.float32), "op_util": util.reshape(1, 1, -1),
                 "op_cost": cost.reshape(1, 1, -1), "node_topo": topo}
        rel = rng.random((1, 1, T)).astype(np.float32)
        sens = np.ones((1, 1, 1), np.float32)
        for B in sorted({1, 2, 3, total // 2, total - 1, total, total + 2}):
            if B < 1:
                continue
            for ff in (0.0, 0.5):
                cfg = sp._cfg(lens=[T], slot_len=0, slot_min=1, slot_max=128, budget_ratio=0.0, budget_min=B,
                              floor_frac=ff, G=4, P=16, d=64)
                cu = np.array([0, T])
                ft, fs = oracle.select.floor_select(rel, sens, trees["op_cost"], cu, slots, cfg, topo=topo)
                want, spent = oracle.select.auction(trees["op_util"], trees["op_cost"], ft, fs, cu, slots, cfg,
                                                    topo=topo)
                pb = kvc.make_problem(cfg, torch.tensor([0, T]), torch.float32)
                ss, ns = slots_to_dev(slots, pb.slot_stride())
                g = kvc.auction(pb, trees_to_dev(trees), to_dev(rel), to_dev(sens), ss, ns)
                torch.cuda.synchronize()
                assert np.array_equal(as_np(g["spent_floor"]), fs), (trial, B, ff)
                assert np.array_equal(as_np(g["spent"]), spent), (trial, B, ff, as_np(g["spent"]), spent)
                assert np.array_equal(as_np(g["taken"]), want), (trial, B, ff)
                n_short += int(spent[0]) < min(B, total)
    print(f"  budgets left partly unspent by a three-way split: {n_short}", flush=True)
    assert n_short > 0
