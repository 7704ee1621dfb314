"""The C++ oracle (oracle/cpp) against the Python oracle, stage by stage, on
every reduced workload: integer outputs (slots, seeds, op costs, floor and
auction choices, token top-B, pack layout and positions) bit-exact, floating
outputs at fp64 round-off (both round fp64 results to fp32 at the same
points, so they agree to an fp32 ulp). The integer stages are also run on the
Python oracle's own fp32 inputs, so their agreement does not rest on the
float stages matching. The full-budget identity (GraceKV page, '05 Physical
cache packing': at full budget every tree expands to its leaves and the
original entries come back; the KL is then exactly 0) is checked on the C++
oracle directly."""
import numpy as np
import pytest
import torch

import oracle
from oracle import cpp_oracle as co
from workload import small_config, make_inputs

CASES = [("tiny", {}), ("mistral1", {}), ("fulldepth", {}), ("stress", {}), ("stress8", {}), ("ragged", {}),
         ("fulldepth", {"n_depth": 3, "surprisal": True}), ("ragged", {"budget_ratio": 0.6, "floor_frac": 0.3}),
         ("tiny", {"split_mode": 1}), ("fulldepth", {"split_mode": 1}),
         ("ragged", {"split_mode": 1, "floor_frac": 0.3})]


def _close(a, b, name, rtol=2.0 ** -22):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, name
    scale = np.abs(b).max() if b.size else 0.0
    bad = np.abs(a - b) > rtol * np.abs(b) + 1e-12 * scale
    assert not bad.any(), (name, int(bad.sum()), float(np.abs(a - b).max()))


@pytest.fixture(scope="module", params=CASES, ids=lambda c: c[0] + "".join(f"-{k}={v}" for k, v in c[1].items()))
def both(request):
    name, kw = request.param
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    return cfg, inp, oracle.run_pipeline(inp, cfg), co.run_pipeline(inp, cfg)


def test_scores_and_propagation(both):
    cfg, inp, a, b = both
    for k in ("r0", "lse", "ent", "head_sens", "rel", "feats"):
        _close(b[k], a[k], k)
    assert np.array_equal(a["seeds"], b["seeds"])


def test_slots_trees_and_selection(both):
    cfg, inp, a, b = both
    cu = inp["cu_seqlens"].numpy()
    assert a["slots"] == b["slots"]
    if cfg.slot_len == 0 and not cfg.token_mode:
        assert np.array_equal(a["dp_cost_q"], b["dp_cost_q"])
        assert np.array_equal(a["dp_cut_q"], b["dp_cut_q"])
        # the DP alone, on the Python oracle's quantized costs
        assert co.slots_for(cu, cfg, a["dp_cost_q"], a["dp_cut_q"]) == a["slots"]
    if not cfg.token_mode:
        for k in ("node_rel", "node_D", "node_mu", "op_util"):
            _close(b["trees"][k], a["trees"][k], k)
        assert np.array_equal(a["trees"]["op_cost"], b["trees"]["op_cost"])
        assert np.array_equal(a["trees"]["node_topo"], b["trees"]["node_topo"])
        # the tree shapes on the Python oracle's fp32 relevance: bit-exact
        tr = co.build_trees(inp["K"], inp["V"], inp["Qp"], a["lse"], a["rel"], a["head_sens"], cu, a["slots"], cfg,
                            cut_q=a.get("dp_cut_q"))
        assert np.array_equal(tr["node_topo"], a["trees"]["node_topo"])
        # given shapes: the same trees from the records alone
        tg = co.build_trees(inp["K"], inp["V"], inp["Qp"], a["lse"], a["rel"], a["head_sens"], cu, a["slots"], cfg,
                            topo=a["trees"]["node_topo"])
        for k in ("node_topo", "op_cost", "node_rel", "node_D", "node_mu", "op_util"):
            assert np.array_equal(tg[k], tr[k]), k
        # floor and auction on the Python oracle's fp32 inputs: bit-exact
        topo = a["trees"]["node_topo"]
        ft, fs = co.floor_select(a["rel"], a["head_sens"], a["trees"]["op_cost"], cu, a["slots"], cfg, topo=topo)
        assert np.array_equal(ft, a["floor_taken"]) and np.array_equal(fs, a["floor_spent"])
        tk, sp = co.auction(a["trees"]["op_util"], a["trees"]["op_cost"], a["floor_taken"], a["floor_spent"], cu,
                            a["slots"], cfg, topo=topo)
        assert np.array_equal(tk, a["taken"]) and np.array_equal(sp, a["spent"])
    else:
        tk, sp = co.token_topk(a["rel"], cu, cfg)
        assert np.array_equal(tk, a["taken"]) and np.array_equal(sp, a["spent"])
    assert np.array_equal(a["taken"], b["taken"])
    assert np.array_equal(a["spent"], b["spent"])


def test_pack_decode_kl(both):
    cfg, inp, a, b = both
    ca, cb = a["cache"], b["cache"]
    for k in ("seg_off", "seg_len", "pos"):
        assert np.array_equal(ca[k], cb[k]), k
    _close(cb["lnmu"], ca["lnmu"], "lnmu")
    # rows in the cache dtype: identical values (a rounding of the fp64
    # prototype may differ by one unit of the cache dtype at most)
    Kb, Vb = co.rows_as_float64(cb["K"]), co.rows_as_float64(cb["V"])
    ulp = 2.0 ** -7 if cfg.dtype == "bf16" else 2.0 ** -23
    for got, want, nm in ((Kb, ca["K"], "K"), (Vb, ca["V"], "V")):
        diff = np.abs(got - want)
        assert np.all(diff <= ulp * np.abs(want)), nm
        assert (diff > 0).mean() < 1e-3, nm
    _close(b["x_full"], a["x_full"], "x_full", rtol=2.0 ** -21)
    _close(b["x_comp"], a["x_comp"], "x_comp", rtol=1e-5)
    assert np.abs(b["kl"] - a["kl"]).max() <= 1e-5


@pytest.mark.parametrize("name,mode", [("tiny", 0), ("stress", 0), ("ragged", 0), ("mistral1", 0), ("tiny", 1),
                                       ("fulldepth", 1)])
def test_cpp_full_budget_is_the_identity(name, mode):
    cfg = small_config(name).replace(budget_ratio=1.0, split_mode=mode)
    inp = make_inputs(cfg)
    cu = inp["cu_seqlens"].numpy()
    o = co.run_pipeline(inp, cfg)
    c = o["cache"]

    def raw(t):   # stored bits of the cache dtype
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if cfg.dtype == "bf16" else t.numpy()

    Kraw, Vraw = raw(inp["K"]), raw(inp["V"])
    for s in range(cfg.S):
        for l in range(cfg.Ly):
            for h in range(cfg.H):
                a, n = int(c["seg_off"][s, l, h]), int(c["seg_len"][s, l, h])
                assert n == int(cu[s + 1] - cu[s])
                assert np.array_equal(c["K"][a:a + n], Kraw[l, h, cu[s]:cu[s + 1]])
                assert np.array_equal(c["V"][a:a + n], Vraw[l, h, cu[s]:cu[s + 1]])
    assert np.all(c["lnmu"] == 0)
    assert np.array_equal(o["x_full"], o["x_comp"])
    assert np.all(o["kl"] == 0)


def test_cpp_sampled_steps_equal_all_steps():
    # decode step t depends only on the appended tokens 0..t: sampling steps
    # gives the same rows as running all of them
    cfg = small_config("stress").replace(T_dec=4)
    inp = make_inputs(cfg)
    allr = co.run_pipeline(inp, cfg)
    some = co.run_pipeline(inp, cfg, steps=[1, 3])
    assert np.array_equal(some["x_full"], allr["x_full"][:, [1, 3]])
    assert np.array_equal(some["x_comp"], allr["x_comp"][:, [1, 3]])
    assert np.array_equal(some["kl"], allr["kl"][:, [1, 3]])
