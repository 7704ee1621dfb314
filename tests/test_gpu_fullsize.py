"""GPU parity at the full size of the full-depth workload (1 x 16384 tokens,
32 layers x 8 KV heads, head dim 128, bf16) in the launch configuration the
benchmark times, on outputs the oracle can compute one at a time: sampled
(layer, KV head) units for scores, propagation, trees and decode; sampled
windows for the DP costs. Integer stages are checked against their
definitions at full size: the auction's taken set must be exactly the top of
the capped-priority order, and the packed cache must be the frontier of the
taken ops in position order with leaves copied bit for bit.

Inputs come from the seeded generator on the GPU and are copied to the host
for the oracle; no expected value comes from the HIP path (the auction and
pack checks use the stage's own inputs only to state the definition)."""
import math

import numpy as np
import pytest
import torch

from oracle import partition as opart
from oracle import trees as otrees
from oracle.propagate import _unit as prop_unit
from oracle.score import _unit_scores
from oracle.common import to64, rope_inv, regions, budgets
from workload import get_config, make_inputs
from parity import close, as_np, slots_from_dev

pytestmark = pytest.mark.gpu

UNITS = [(0, 0), (13, 5), (31, 7)]   # sampled (layer, KV head)


def _kvc():
    from eviction_probe_softmax_amd import kvc
    return kvc


@pytest.fixture(scope="module")
def run():
    kvc = _kvc()
    from eviction_probe_softmax_amd.pipeline import Compressor
    cfg = get_config("fulldepth")
    print(f"[fullsize] generating {cfg.name} inputs on the GPU", flush=True)
    inp = make_inputs(cfg, device="cuda")
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    out = comp.compress(inp)
    costs = kvc.partition(comp.pb, inp["hidden"], cfg.hidden_dim, export=True)
    torch.cuda.synchronize()
    return {"cfg": cfg, "inp": inp, "comp": comp, "out": out, "costs": costs, "cache": {}}


def _unit_oracle(r, l, h):
    """Oracle scores and propagation of one unit from the raw inputs (cached)."""
    key = (l, h)
    if key in r["cache"]:
        return r["cache"][key]
    cfg, inp = r["cfg"], r["inp"]
    G, P, d = cfg.G, cfg.P, cfg.d
    K = to64(inp["K"][l, h].cpu())
    V = to64(inp["V"][l, h].cpu())
    Q = to64(inp["Qp"][0, l, h * G:(h + 1) * G].cpu()).reshape(G * P, d)
    r0, feats, lse, ent, sens = _unit_scores(Q, K, V, G, P)
    r0_32 = np.float32(r0).astype(np.float64)          # the stage output is fp32
    Qc = to64(inp["Qctx"][l, h * G:(h + 1) * G].cpu())
    rel, _ = prop_unit(Qc, K, r0_32, G, cfg.n_hops, cfg.n_seeds, float(np.float32(cfg.hop_weight)))
    res = {"K": K, "V": V, "Q": Q, "r0": r0, "feats": feats, "lse": lse, "ent": ent, "sens": sens,
           "rel": np.float32(rel)}
    r["cache"][key] = res
    return res


def test_fullsize_scores_and_propagation_sampled(run):
    cfg, out = run["cfg"], run["out"]
    G, P = cfg.G, cfg.P
    for (l, h) in UNITS:
        o = _unit_oracle(run, l, h)
        print(f"  unit l={l} h={h}", flush=True)
        close(out["r0"][l, h], o["r0"], 1e-3, "r0", floor=1e-3)
        close(out["feats"][:, l, h], o["feats"], 1e-3, "feats", floor=1e-3)
        close(out["lse"][0, l, h * G:(h + 1) * G].reshape(G * P), o["lse"], 1e-3, "lse")
        close(out["ent"][0, l, h * G:(h + 1) * G].reshape(G * P), o["ent"], 1e-3, "entropy", floor=1e-3)
        close(np.array([float(out["head_sens"][0, l, h])]), np.array([o["sens"]]), 1e-3, "head sensitivity")
        close(out["rel"][l, h], o["rel"], 1e-3, "rel", floor=1e-3)


def test_fullsize_dp_costs_sampled(run):
    cfg, inp, costs, out = run["cfg"], run["inp"], run["costs"], run["out"]
    L = cfg.lens[0]
    pe, c0, c1, _ = regions(L, cfg)
    hn = opart.normalize(to64(inp["hidden"].cpu()))
    gq = as_np(costs["dp_cost_q"])
    gk = as_np(costs["dp_cut_q"])
    rng = np.random.default_rng(7)
    worst = 0.0
    for _ in range(300):
        n = int(rng.integers(cfg.slot_min, cfg.slot_max + 1))
        e = int(rng.integers(c0 + n, c1 + 1))               # exclusive end
        want = opart._q(opart.slot_cost(hn, e - n, n, cfg))
        got = int(gq[e - 1, n - cfg.slot_min])
        worst = max(worst, abs(got - want) / max(abs(want), 1))
        assert abs(got - want) <= 1e-4 * abs(want) + 64, (e, n, got, want)
    lam = float(np.float32(cfg.lambda_curv))
    for c in rng.integers(c0, c1, size=300):
        want = opart._q(lam * opart.turning_score(hn, int(c)))
        assert abs(int(gk[int(c)]) - want) <= 1e-4 * (1 << 22) + 64, (int(c), int(gk[int(c)]), want)
    slots = slots_from_dev(out["slot_start"], out["n_slots"])[0]
    assert slots[0][0] == c0 and slots[-1][0] + slots[-1][1] == c1
    assert all(slots[k][0] + slots[k][1] == slots[k + 1][0] for k in range(len(slots) - 1))
    assert all(cfg.slot_min <= n <= cfg.slot_max for _, n in slots)
    print(f"  worst relative cost error {worst:.2e}, {len(slots)} slots", flush=True)


@pytest.mark.parametrize("slot_len", [64, 128])
def test_fullsize_trees_sampled(run, slot_len):
    """Fixed slots (their boundaries follow from a rule, not from the DP) at
    full size; the sampled units' relevance, lse and sensitivity are the
    oracle's."""
    kvc = _kvc()
    cfg0, inp, out = run["cfg"], run["inp"], run["out"]
    cfg = cfg0.replace(slot_len=slot_len)
    G, P, d = cfg.G, cfg.P, cfg.d
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    part = kvc.partition(pb)
    rel = out["rel"].clone()
    lse = out["lse"].clone()
    sens = out["head_sens"].clone()
    for (l, h) in UNITS:
        o = _unit_oracle(run, l, h)
        rel[l, h] = torch.from_numpy(o["rel"]).cuda()
        lse[0, l, h * G:(h + 1) * G] = torch.from_numpy(np.float32(o["lse"]).reshape(G, P)).cuda()
        sens[0, l, h] = float(np.float32(o["sens"]))
    rc, rs = kvc.rope_table(cfg.rope_base, d, cfg.lens[0])
    tr = kvc.build_trees(pb, inp["K"], inp["V"], inp["Qp"], lse, rel, sens, rc, rs, part["slot_start"],
                         part["n_slots"])
    torch.cuda.synchronize()
    slots = slots_from_dev(part["slot_start"], part["n_slots"])[0]
    rows = otrees.dprobe_rows(cfg)
    c = 1.0 / math.sqrt(d)
    pick = [0, 1, len(slots) // 2, len(slots) - 2, len(slots) - 1]
    g = {k: as_np(tr[k]) for k in ("node_rel", "node_D", "node_mu", "op_util", "op_cost")}
    for (l, h) in UNITS:
        o = _unit_oracle(run, l, h)
        K, V = o["K"], o["V"]
        pos = np.arange(K.shape[0], dtype=np.float64)
        ktil = rope_inv(K, pos, cfg.rope_base)
        knorm = np.sqrt((ktil * ktil).sum(axis=1))
        Qd = o["Q"][rows]
        ls = np.float32(o["lse"]).astype(np.float64)[rows]
        r = o["rel"].astype(np.float64)
        s32 = float(np.float32(o["sens"]))
        for k in pick:
            st, n = slots[k]
            Ad = np.exp(c * (Qd @ K[st:st + n].T) - ls[:, None])
            Afull = np.zeros((len(rows), K.shape[0]))
            Afull[:, st:st + n] = Ad
            nodes, nrel, D, mu, _, _ = otrees._slot(ktil, knorm, V, r, Afull, Qd, ls, st, n, 0, cfg, cfg.rope_base)
            b = 2 * st
            m = len(nodes)
            close(g["node_rel"][l, h, b:b + m], np.float32(nrel), 1e-5, "node_rel")
            close(g["node_mu"][l, h, b:b + m], np.float32(mu), 1e-4, "node_mu")
            close(g["node_D"][l, h, b:b + m], np.float32(D), 1e-3, "node_D", floor=1e-3)
            util = np.zeros(2 * n)
            util[0] = s32 * nrel[0] * (1.0 - D[0])
            for j, (_, _, lc, rc_) in enumerate(nodes):
                if lc >= 0:
                    util[1 + j] = s32 * (nrel[j] * D[j] - (nrel[lc] * D[lc] + nrel[rc_] * D[rc_]))
            close(g["op_util"][l, h, b:b + 2 * n], np.float32(util), 1e-3, "op_util", floor=1e-3)
    print(f"  slot_len {slot_len}: {len(UNITS)} units x {len(pick)} slots match", flush=True)


def _capped_priorities(util, cost, slots, T, cu0=0):
    """u'(Add) = u; u'(Split j) = min(u(Split j), u'(creator of j)), per slot.
    util, cost: [U][2T]. Returns float32 [U][2T] (-inf where there is no op)."""
    U = util.shape[0]
    cap = np.full(util.shape, -np.inf, dtype=np.float32)
    by_n = {}
    for (st, n) in slots:
        by_n.setdefault(n, []).append(st)
    for n, starts in by_n.items():
        nodes = otrees.tree_nodes(0, n)
        parent = np.full(len(nodes), -1)
        for j, (_, _, lc, rc) in enumerate(nodes):
            if lc >= 0:
                parent[lc] = j
                parent[rc] = j
        idx = 2 * (cu0 + np.asarray(starts))[:, None] + np.arange(2 * n)[None, :]   # [S_n][2n]
        u = util[:, idx]                                                            # [U][S_n][2n]
        cp = np.full(u.shape, -np.inf, dtype=np.float32)
        cp[..., 0] = u[..., 0]
        for j, (_, _, lc, _) in enumerate(nodes):
            if lc < 0:
                continue
            creator = 0 if j == 0 else 1 + parent[j]
            cp[..., 1 + j] = np.minimum(u[..., 1 + j], cp[..., creator])
        ok = cost[:, idx] > 0
        cap[:, idx] = np.where(ok, cp, -np.inf)
    return cap


def _check_capped_top(g, rest, util, slots, T, k_rest):
    """g: taken flags (flat); rest: capped priorities of the competing ops
    (-inf elsewhere). Above the threshold priority every op is taken, below
    none; the ops tied with it are completed best-first from the exposed ones
    of their slot (the greedy pops the highest utility among exposed ops),
    which a plain (priority, id) order does not state."""
    ids = np.nonzero(np.isfinite(rest))[0]
    order = np.lexsort((ids, -rest[ids]))
    thr = rest[ids[order[k_rest - 1]]] if k_rest > 0 else np.inf
    above = np.isfinite(rest) & (rest > thr)
    tied = np.nonzero(rest == thr)[0]
    k_tied = k_rest - int(above.sum())
    assert g[above].all()
    assert not g[np.isfinite(rest) & (rest < thr)].any()
    slot_of = {}
    for (st, n) in slots:
        for q in range(2 * n):
            slot_of[2 * st + q] = (st, n)
    groups = {(int(t) // (2 * T), slot_of[int(t) % (2 * T)]) for t in tied}
    if len(groups) == 1:
        (u, (st, n)), = groups
        nodes = otrees.tree_nodes(0, n)
        base = u * 2 * T + 2 * st
        kids, creator = {0: [1] if nodes[0][2] >= 0 else []}, {}
        for j, (_, _, lc, rc) in enumerate(nodes):
            if lc >= 0:
                kids[1 + j] = [1 + c for c in (lc, rc) if nodes[c][2] >= 0]
                for c in kids[1 + j]:
                    creator[c] = 1 + j
        if 1 in kids[0]:
            creator[1] = 0
        uflat = util.reshape(-1)
        tied_set = set(int(t) for t in tied)
        exposed = [q for q in range(2 * n) if base + q in tied_set and (q == 0 or above[base + creator[q]])]
        taken_tied = set()
        for _ in range(k_tied):
            q = max(exposed, key=lambda q: (float(uflat[base + q]), -(base + q)))
            exposed.remove(q)
            taken_tied.add(base + q)
            exposed += [c for c in kids.get(q, []) if base + c in tied_set]
        assert set(np.nonzero(g & (rest == thr))[0].tolist()) == taken_tied
    else:
        assert int((g & (rest == thr)).sum()) == k_tied
    return len(tied)


def test_fullsize_auction_is_the_capped_priority_top(run):
    """Without the floor, the greedy auction with unit costs takes every op
    above the allocatable budget's threshold capped priority, none below, and
    completes the ops tied with it best-first."""
    kvc = _kvc()
    cfg0, inp, out = run["cfg"], run["inp"], run["out"]
    cfg = cfg0.replace(floor_frac=0.0)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    tr = out["trees"]
    au = kvc.auction(pb, tr, out["rel"], out["head_sens"], out["slot_start"], out["n_slots"])
    torch.cuda.synchronize()
    Ly, H, T = cfg.Ly, cfg.H, cfg.T
    util = as_np(tr["op_util"]).reshape(Ly * H, 2 * T)
    cost = as_np(tr["op_cost"]).reshape(Ly * H, 2 * T)
    slots = slots_from_dev(out["slot_start"], out["n_slots"])[0]
    cap = _capped_priorities(util, cost, slots, T).reshape(-1)
    valid = np.isfinite(cap)
    B_alloc = budgets(cfg.lens, cfg)[0]["alloc"]
    got = as_np(au["taken"]).reshape(-1).astype(bool)
    k = min(B_alloc, int(valid.sum()))
    assert int(as_np(au["spent"])[0]) == k and int(got.sum()) == k
    ntied = _check_capped_top(got, cap, util, slots, T, k)
    print(f"  {int(got.sum())} ops taken of {int(valid.sum())}, {ntied} tied at the threshold", flush=True)


def test_fullsize_taken_set_and_pack_structure(run):
    """With the floor: the budget is filled, every taken Split's creator is
    taken, and the packed cache is each unit's frontier in position order
    (leaves bit-identical to the source rows, ln mu = 0)."""
    from oracle.pack import _frontier
    cfg, inp, out = run["cfg"], run["inp"], run["out"]
    Ly, H, T = cfg.Ly, cfg.H, cfg.T
    B_alloc = budgets(cfg.lens, cfg)[0]["alloc"]
    taken = as_np(out["taken"]).reshape(Ly * H, 2 * T).astype(bool)
    spent = int(as_np(out["spent"])[0])
    assert spent == B_alloc
    slots = slots_from_dev(out["slot_start"], out["n_slots"])[0]
    cache = out["cache"]
    seg_off = as_np(cache["seg_off"]).reshape(-1)
    seg_len = as_np(cache["seg_len"]).reshape(-1)
    assert int(seg_len.sum()) == spent
    assert np.array_equal(seg_off[1:], seg_off[:-1] + seg_len[:-1])
    # creators of taken Splits are taken (all units at once, slots grouped by length)
    by_n = {}
    for (st, n) in slots:
        by_n.setdefault(n, []).append(st)
    shapes = {}
    for n, starts in by_n.items():
        nodes = otrees.tree_nodes(0, n)
        shapes[n] = nodes
        idx = 2 * np.asarray(starts)[:, None] + np.arange(2 * n)[None, :]
        tk = taken[:, idx]                                             # [U][S_n][2n]
        for j, (_, _, lc, rc) in enumerate(nodes):
            if lc < 0:
                continue
            kids = (lc, rc)
            assert np.all(~tk[..., 1 + j] | tk[..., 0]), (n, j)          # any Split needs the Add
            for kid in kids:
                if nodes[kid][2] >= 0:
                    assert np.all(~tk[..., 1 + kid] | tk[..., 1 + j]), (n, kid)
    pos_all = as_np(cache["pos"])
    lnmu_all = as_np(cache["lnmu"])
    for u in (0, 77, Ly * H // 2, Ly * H - 1):
        l, h = divmod(u, H)
        fr = []
        for (st, n) in slots:
            nodes = otrees.slot_tree(st, n)
            for j in _frontier(nodes, taken[u], 2 * st):
                a, m = nodes[j][0], nodes[j][1]
                fr.append((a + (m - 1) // 2, m, a))
        assert len(fr) == int(seg_len[u]), (u, len(fr), int(seg_len[u]))
        off = int(seg_off[u])
        pos = pos_all[off:off + len(fr)]
        assert np.array_equal(pos, np.array([p for p, _, _ in fr], dtype=pos.dtype)), u
        leaves = [k for k, (_, m, _) in enumerate(fr) if m == 1]
        src = [fr[k][2] for k in leaves]
        li = torch.tensor(leaves, device="cuda", dtype=torch.int64) + off
        si = torch.tensor(src, device="cuda", dtype=torch.int64)
        assert torch.equal(cache["K"][li], inp["K"][l, h][si]), u
        assert torch.equal(cache["V"][li], inp["V"][l, h][si]), u
        assert np.all(lnmu_all[off + np.array(leaves, dtype=np.int64)] == 0.0)
        print(f"  unit {u}: {len(fr)} entries, {len(leaves)} leaves", flush=True)


def test_fullsize_decode_sampled(run):
    """Decode over the full cache at full size: sampled units against the
    definition (softmax over the unit's keys and the appended tokens)."""
    kvc = _kvc()
    cfg, inp, comp = run["cfg"], run["inp"], run["comp"]
    G, d, Td = cfg.G, cfg.d, cfg.T_dec
    full = kvc.full_view(comp.pb, inp["K"], inp["V"])
    dec = kvc.Decoder(full, G, Td)
    x = torch.empty((cfg.S, cfg.d_model), dtype=torch.float32, device="cuda")
    o = torch.empty((cfg.S, cfg.Ly, cfg.H * G, d), dtype=torch.float32, device="cuda")
    c = 1.0 / math.sqrt(d)
    for t in (0, Td // 2, Td - 1):
        dec.step(inp["Kd"], inp["Vd"], t + 1, inp["Qd"][t], x, cfg.d_model, o_out=o)
        torch.cuda.synchronize()
        go = as_np(o)
        for (l, h) in UNITS:
            Ke = np.concatenate([to64(inp["K"][l, h].cpu()), to64(inp["Kd"][l, h, 0, :t + 1].cpu())])
            Ve = np.concatenate([to64(inp["V"][l, h].cpu()), to64(inp["Vd"][l, h, 0, :t + 1].cpu())])
            q = to64(inp["Qd"][t, 0, l, h * G:(h + 1) * G].cpu())
            z = c * (q @ Ke.T)
            p = np.exp(z - z.max(axis=1, keepdims=True))
            want = (p / p.sum(axis=1, keepdims=True)) @ Ve
            close(go[0, l, h * G:(h + 1) * G], want, 2e-2, "decode o", floor=1e-2)
        # x is the layer sum of o, in layer order
        close(as_np(x)[0], go[0].sum(axis=0).reshape(-1), 1e-5, "x = sum over layers", floor=1e-5)


def test_fullsize_hybrid_auction(run):
    """Head-level hybrid at full size, floor off: the K units with the largest
    head sensitivity keep every real op; the rest of the allocatable budget
    buys exactly the top of the capped-priority order over the other units."""
    kvc = _kvc()
    cfg0, inp, out = run["cfg"], run["inp"], run["out"]
    cfg = cfg0.replace(floor_frac=0.0, hybrid_frac=0.2)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    tr = out["trees"]
    au = kvc.auction(pb, tr, out["rel"], out["head_sens"], out["slot_start"], out["n_slots"])
    full_g = as_np(kvc.hybrid_units(pb, out["head_sens"])).reshape(-1).astype(bool)
    torch.cuda.synchronize()
    Ly, H, T = cfg.Ly, cfg.H, cfg.T
    b = budgets(cfg.lens, cfg)[0]
    K, C = b["full_units"], b["comp_len"]
    sens = as_np(out["head_sens"]).reshape(-1)
    order_u = np.lexsort((np.arange(Ly * H), -sens))
    full = np.zeros(Ly * H, dtype=bool)
    full[order_u[:K]] = True
    assert np.array_equal(full_g, full) and K == int(0.2 * Ly * H)
    util = as_np(tr["op_util"]).reshape(Ly * H, 2 * T)
    cost = as_np(tr["op_cost"]).reshape(Ly * H, 2 * T)
    slots = slots_from_dev(out["slot_start"], out["n_slots"])[0]
    cap = _capped_priorities(util, cost, slots, T)
    want = np.zeros(cap.shape, dtype=bool)
    want[full] = cost[full] > 0
    rest = cap.copy()
    rest[full] = -np.inf
    rest = rest.reshape(-1)
    k_rest = min(b["rest"], int(np.isfinite(rest).sum()))
    got = as_np(au["taken"]).reshape(Ly * H, 2 * T).astype(bool)
    assert int(as_np(au["spent"])[0]) == K * C + k_rest
    assert np.array_equal(got[full], want[full])
    ntied = _check_capped_top(got.reshape(-1), rest, util, slots, T, k_rest)
    print(f"  {K} units whole, {int(got.sum())} ops taken, {ntied} tied at the threshold", flush=True)


def test_fullsize_stepwise_prunes(run):
    """Step-wise eviction at full size: feature invariants, the MLP against
    the oracle on the kernel's own features (sampled tokens), the kept set
    exactly the top-B of the scores, kept rows bit copies, lengths on the
    budget schedule over a few steps."""
    from oracle import stepwise as osw
    from workload import make_policy
    kvc = _kvc()
    cfg, inp = run["cfg"], run["inp"]
    L = cfg.lens[0]
    pol_h = make_policy(seed=11)
    pol = {k: v.cuda() for k, v in pol_h.items()}
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    sw = kvc.Stepwise(pb, pol, 4, inp["K"].dtype, cfg.G)
    feats = torch.zeros((5, L), dtype=torch.float32, device="cuda")
    scores = torch.zeros((L,), dtype=torch.float32, device="cuda")
    sw.init(inp["K"], inp["V"], inp["Qctx"], feats, scores)
    torch.cuda.synchronize()
    f, sc = as_np(feats), as_np(scores)
    assert abs(f[0].sum() - 1.0) < 1e-3 and f[2].min() >= 0.0
    assert f[3].min() >= 0.0 and f[3].max() <= math.log(L) + 1e-3
    assert np.allclose(f[4], np.arange(L) / (L - 1), atol=1e-6)
    pick = np.random.default_rng(0).choice(L, 2000, replace=False)
    close(sc[pick], osw.policy_scores(f[:, pick].T.astype(np.float64), pol_h), 1e-4, "policy", floor=1e-4)
    B = osw.step_budget(L, cfg)
    kept = np.sort(osw.keep_top(sc, np.arange(L), B))
    pos = as_np(sw.pos[:B]).astype(np.int64)
    assert sw.lengths[0] == B and np.array_equal(pos, kept)
    for (l, h) in UNITS:
        assert torch.equal(sw.K[l, h, :B].cpu(), inp["K"][l, h, kept].cpu())
        assert torch.equal(sw.V[l, h, :B].cpu(), inp["V"][l, h, kept].cpu())
    cap = sw.cap_total
    feats2 = torch.zeros((5, cap), dtype=torch.float32, device="cuda")
    scores2 = torch.zeros((cap,), dtype=torch.float32, device="cuda")
    for t in range(4):
        sw.append(inp["Kd"], inp["Vd"], inp["Qd"][t], t)
        n = sw.lengths[0]
        before = as_np(sw.pos[:n]).astype(np.int64)
        sw.prune(t, feats2, scores2)
        torch.cuda.synchronize()
        B = osw.step_budget(L + t + 1, cfg)
        assert sw.lengths[0] == min(B, n)
        keep = osw.keep_top(as_np(scores2[:n]), before, B)
        assert np.array_equal(np.sort(before[keep]), np.sort(as_np(sw.pos[:sw.lengths[0]]).astype(np.int64)))
    print(f"  first prune kept {len(kept)}, final length {sw.lengths[0]}", flush=True)
