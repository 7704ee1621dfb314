"""GPU parity: probe scores/features (kvc_score) and propagation (kvc_propagate)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from workload import small_config, make_inputs
from parity import close, as_np, to_dev, inputs_to

pytestmark = pytest.mark.gpu

CASES = ["tiny", "mistral1", "ragged", "stress"]


def _setup(name, **kw):
    from eviction_probe_softmax_amd import kvc
    cfg = small_config(name, **kw)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    return kvc, cfg, inp, dinp, pb


@pytest.mark.parametrize("name", CASES)
def test_score_matches_oracle(name):
    kvc, cfg, inp, dinp, pb = _setup(name)
    print(f"[score] {name} lens={cfg.lens} Ly={cfg.Ly} H={cfg.H} d={cfg.d} P={cfg.P}", flush=True)
    g = kvc.score(pb, dinp["K"], dinp["V"], dinp["Qp"])
    torch.cuda.synchronize()
    o = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], inp["cu_seqlens"].numpy(), cfg)
    close(g["r0"], o["r0"], 1e-3, "r0")
    close(g["lse"], o["lse"], 1e-3, "lse")
    close(g["ent"], o["ent"], 1e-3, "ent")
    close(g["head_sens"], o["head_sens"], 1e-3, "head_sens")
    names = ["mass", "vnorm", "sigma", "entropy", "pos"]
    for f in range(5):
        # the variance feature is a difference of nearly equal per-head masses
        tol = 1e-3 if f != 2 else 1e-2
        close(g["feats"][f], o["feats"][f], tol, names[f], floor=1e-4 if f == 2 else 1e-6)
    # invariant: each unit's mass sums to G*P
    r0 = as_np(g["r0"]).astype(np.float64)
    cu = inp["cu_seqlens"].numpy()
    for s in range(cfg.S):
        tot = r0[:, :, cu[s]:cu[s + 1]].sum(-1)
        assert np.allclose(tot, cfg.G * cfg.P, rtol=1e-4)


@pytest.mark.parametrize("name,P", [("stress", 40), ("ragged", 48), ("mistral1", 32), ("stress", 24)])
def test_score_head_masses_with_other_probe_counts(name, P):
    """Probe counts that are not multiples of 32 put rows of two query heads in
    one 32-row block: the per-head masses behind the variance feature must
    still follow the heads (DistillCache paper, Sec. 3.1.1)."""
    kvc, cfg, inp, dinp, pb = _setup(name, P=P)
    print(f"[score] {name} P={P} G={cfg.G}", flush=True)
    g = kvc.score(pb, dinp["K"], dinp["V"], dinp["Qp"])
    torch.cuda.synchronize()
    o = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], inp["cu_seqlens"].numpy(), cfg)
    close(g["r0"], o["r0"], 1e-3, "r0")
    close(g["lse"], o["lse"], 1e-3, "lse")
    close(g["feats"][2], o["feats"][2], 1e-2, "sigma", floor=1e-4)
    close(g["feats"][3], o["feats"][3], 1e-3, "entropy")


@pytest.mark.parametrize("name", CASES)
def test_propagate_matches_oracle(name):
    kvc, cfg, inp, dinp, pb = _setup(name)
    print(f"[propagate] {name} lens={cfg.lens}", flush=True)
    cu = inp["cu_seqlens"].numpy()
    o_sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    # feed the oracle's fp32 scores so the first hop's seeds must match exactly
    g = kvc.propagate(pb, dinp["K"], dinp["Qctx"], to_dev(o_sc["r0"]))
    torch.cuda.synchronize()
    o = oracle.propagate(inp["K"], inp["Qctx"], o_sc["r0"], cu, cfg)
    gs = as_np(g["seeds"])
    assert np.array_equal(gs[0], o["seeds"][0]), "hop-1 seeds differ"
    # later hops seed from float increments: compare the sets
    for hop in range(1, cfg.n_hops):
        a, b = gs[hop].reshape(-1, cfg.n_seeds), o["seeds"][hop].reshape(-1, cfg.n_seeds)
        inter = sum(len(set(x) & set(y)) for x, y in zip(a.tolist(), b.tolist()))
        union = sum(len(set(x) | set(y)) for x, y in zip(a.tolist(), b.tolist()))
        assert inter / union >= 0.95
    close(g["rel"], o["rel"], 1e-3, "rel")


def test_propagate_dense_limit():
    # every token a seed (M >= L): one hop equals the dense GQA-mean rollout
    kvc, cfg, inp, dinp, pb = _setup("tiny", lens=[60], n_seeds=64, n_hops=1)
    cu = inp["cu_seqlens"].numpy()
    o_sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    g = kvc.propagate(pb, dinp["K"], dinp["Qctx"], to_dev(o_sc["r0"]))
    o = oracle.propagate(inp["K"], inp["Qctx"], o_sc["r0"], cu, cfg)
    assert np.array_equal(as_np(g["seeds"])[0, 0, 0, 0, :60], np.arange(60))
    close(g["rel"], o["rel"], 1e-3, "rel")


def test_score_repeatable():
    kvc, cfg, inp, dinp, pb = _setup("ragged")
    a = kvc.score(pb, dinp["K"], dinp["V"], dinp["Qp"])
    b = kvc.score(pb, dinp["K"], dinp["V"], dinp["Qp"])
    for k in ("r0", "feats", "lse", "ent", "head_sens"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name,kw", [("tiny", {"n_hops": 1}), ("tiny", {}), ("stress", {}), ("ragged", {}),
                                     ("mistral1", {"n_hops": 1})])
def test_dense_rollout_matches_oracle(name, kw):
    """Every token a seed in every hop (the oracle with n_seeds >= L), over
    several row blocks per sequence and ragged lengths."""
    kvc, cfg, inp, dinp, pb = _setup(name, **kw)
    cu = inp["cu_seqlens"].numpy()
    print(f"[dense rollout] {name} {kw} lens={cfg.lens}", flush=True)
    o_sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    g = kvc.propagate_dense(pb, dinp["K"], dinp["Qctx"], to_dev(o_sc["r0"]))
    o = oracle.propagate(inp["K"], inp["Qctx"], o_sc["r0"], cu, cfg.replace(n_seeds=max(cfg.lens)))
    close(g["rel"], o["rel"], 1e-3, "rel")


@pytest.mark.parametrize("name,kw", [("tiny", {"n_hops": 1}), ("tiny", {}), ("stress", {}), ("ragged", {}),
                                     ("mistral1", {"n_hops": 1})])
def test_ar_direction_matches_oracle(name, kw):
    """Every token takes the causal softmax average of the previous
    increment, over several row blocks and ragged lengths."""
    from oracle.propagate import propagate_ar
    kvc, cfg, inp, dinp, pb = _setup(name, **kw)
    cu = inp["cu_seqlens"].numpy()
    print(f"[A r] {name} {kw} lens={cfg.lens}", flush=True)
    o_sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    g = kvc.propagate_ar(pb, dinp["K"], dinp["Qctx"], to_dev(o_sc["r0"]))
    o = propagate_ar(inp["K"], inp["Qctx"], o_sc["r0"], cu, cfg)
    close(g["rel"], o["rel"], 1e-3, "rel")
