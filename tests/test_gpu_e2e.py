"""GPU end-to-end parity: the whole compress -> decode -> KL path from raw
inputs against the oracle (selected-set Jaccard, per-step KL), and the full-
budget identity on the GPU (packed cache == original bits, KL == 0)."""
import numpy as np
import pytest
import torch

import oracle
from workload import small_config, make_inputs
from parity import as_np, inputs_to, jaccard, close, check_kl, oracle_on_taken, slots_from_dev, topo_np

pytestmark = pytest.mark.gpu


def _run_gpu(cfg, inp):
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor, decode_both
    dinp = inputs_to(inp)
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    out = comp.compress(dinp)
    full = kvc.full_view(comp.pb, dinp["K"], dinp["V"])
    xf, xc = decode_both(out["cache"], full, dinp, cfg)
    n = cfg.S * cfg.T_dec
    klv = kvc.kl(xf.reshape(n, -1), xc.reshape(n, -1), dinp["W"]).reshape(cfg.S, cfg.T_dec)
    torch.cuda.synchronize()
    return out, xf, xc, klv




@pytest.mark.parametrize("name,kw", [("tiny", {}), ("mistral1", {}),
                                     ("stress", {}),
                                     ("ragged", {}),
                                     ("fulldepth", {}), ("ragged", {"hybrid_frac": 0.5}),
                                     ("fulldepth", {"hybrid_frac": 0.25, "budget_ratio": 0.4}),
                                     ("mistral1", {"hybrid_frac": 0.5, "budget_ratio": 0.6}),
                                     ("fulldepth", {"n_depth": 3, "surprisal": True}),
                                     ("tiny", {"split_mode": 1}), ("fulldepth", {"split_mode": 1}),
                                     ("ragged", {"split_mode": 1}),
                                     ("fulldepth", {"split_mode": 1, "n_depth": 3, "surprisal": True})])
def test_end_to_end_matches_oracle(name, kw):
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    print(f"[e2e] {name} {kw} lens={cfg.lens}", flush=True)
    out, xf, xc, klv = _run_gpu(cfg, inp)
    o = oracle.run_pipeline(inp, cfg)
    _compare(cfg, inp, out, xf, xc, klv, o, name)


def _compare(cfg, inp, out, xf, xc, klv, o, name):
    """Selected set (Jaccard), spent, slots; then x_full, x_comp and the KL
    against the oracle's decode and KL of the GPU's own taken set (so every
    run checks them, whatever the Jaccard)."""
    j = jaccard(as_np(out["taken"]), o["taken"])
    assert j >= 0.99, j
    assert np.array_equal(as_np(out["spent"]), o["spent"])
    if not cfg.token_mode:
        assert slots_from_dev(out["slot_start"], out["n_slots"]) == o["slots"]
    close(xf, o["x_full"], 2e-2, "x_full", floor=1e-3)
    print(f"  jaccard={j:.4f} kl_oracle_mean={o['kl'].mean():.4f}", flush=True)
    topo = None
    if getattr(cfg, "split_mode", 0):
        topo = topo_np(out["trees"]["node_topo"])
        same = float((topo == o["trees"]["node_topo"]).mean())
        print(f"  tree shapes equal to the oracle's at {same:.5f} of the records; three-way splits taken "
              f"{int(((o['trees']['op_cost'] == 2) & (o['taken'] > 0)).sum())}", flush=True)
        assert same >= 0.99, same
    xc_o, kl_o = oracle_on_taken(inp, cfg, o, out["taken"], topo)
    if j == 1.0:
        assert np.array_equal(xc_o, o["x_comp"]) and np.array_equal(kl_o, o["kl"])
    # the packed prototypes are bf16 on the GPU and fp64 in the oracle, so
    # x_comp carries their rounding, scaled by the summands (not by x)
    close(xc, xc_o, 2e-2, "x_comp", floor=1e-2)
    check_kl(klv, xf, xc, inp["W"], kl_o, name, o["x_full"], xc_o)


@pytest.mark.parametrize("name,seed", [("stress", 2), ("stress", 5), ("ragged", 3), ("ragged", 6),
                                       ("fulldepth", 4), ("mistral1", 7)])
def test_end_to_end_other_seeds(name, seed):
    """The same end-to-end bar on inputs drawn from other seeds."""
    cfg = small_config(name)
    inp = make_inputs(cfg, seed=seed)
    print(f"[e2e-seed] {name} seed={seed}", flush=True)
    out, xf, xc, klv = _run_gpu(cfg, inp)
    o = oracle.run_pipeline(inp, cfg)
    _compare(cfg, inp, out, xf, xc, klv, o, name)


@pytest.mark.parametrize("name,mode", [("tiny", 0), ("stress", 0), ("ragged", 0), ("mistral1", 0), ("tiny", 1),
                                       ("fulldepth", 1)])
def test_full_budget_is_the_identity_on_gpu(name, mode):
    cfg = small_config(name).replace(budget_ratio=1.0, split_mode=mode)
    inp = make_inputs(cfg)
    print(f"[identity] {name}", flush=True)
    out, xf, xc, klv = _run_gpu(cfg, inp)
    c = out["cache"]
    cu = inp["cu_seqlens"].numpy()
    K = inp["K"]
    for s in range(cfg.S):
        for l in range(cfg.Ly):
            for h in range(cfg.H):
                a, n = int(c["seg_off"][s, l, h]), int(c["seg_len"][s, l, h])
                assert n == int(cu[s + 1] - cu[s])
                assert torch.equal(c["K"][a:a + n].cpu(), K[l, h, cu[s]:cu[s + 1]])
                assert torch.equal(c["V"][a:a + n].cpu(), inp["V"][l, h, cu[s]:cu[s + 1]])
    assert torch.all(c["lnmu"][: int(c["seg_len"].sum())] == 0)
    assert torch.equal(xf, xc)
    assert torch.all(klv == 0)


def test_whole_heads_at_full_budget_are_the_identity():
    # the head-level hybrid keeping every unit whole is the full cache again
    cfg = small_config("stress").replace(budget_ratio=1.0, hybrid_frac=1.0)
    inp = make_inputs(cfg)
    out, xf, xc, klv = _run_gpu(cfg, inp)
    assert int(as_np(out["spent"]).sum()) == sum(cfg.lens) * cfg.Ly * cfg.H
    assert torch.equal(xf, xc)
    assert torch.all(klv == 0)


def test_pipeline_repeatable():
    cfg = small_config("ragged")
    inp = make_inputs(cfg)
    a = _run_gpu(cfg, inp)
    b = _run_gpu(cfg, inp)
    assert torch.equal(a[0]["taken"], b[0]["taken"])
    assert torch.equal(a[3], b[3])
    assert torch.equal(a[0]["cache"]["K"], b[0]["cache"]["K"])
