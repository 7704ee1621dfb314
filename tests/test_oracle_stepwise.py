"""Pins of the step-wise eviction oracle (DistillCache paper, Sec. 3.1.1,
Sec. 3.1.4, Algorithm 1) against library routines, closed forms and
invariants."""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import stepwise as sw, common
from workload import small_config, make_inputs, make_policy


def test_policy_matches_library_modules():
    pol = make_policy(seed=3)
    net = torch.nn.Sequential(torch.nn.Linear(5, 128), torch.nn.LayerNorm(128, eps=1e-5), torch.nn.ReLU(),
                              torch.nn.Linear(128, 128), torch.nn.LayerNorm(128, eps=1e-5), torch.nn.ReLU(),
                              torch.nn.Linear(128, 1)).double()
    with torch.no_grad():
        net[0].weight.copy_(pol["w1"]); net[0].bias.copy_(pol["b1"])
        net[1].weight.copy_(pol["g1"]); net[1].bias.copy_(pol["be1"])
        net[3].weight.copy_(pol["w2"]); net[3].bias.copy_(pol["b2"])
        net[4].weight.copy_(pol["g2"]); net[4].bias.copy_(pol["be2"])
        net[6].weight.copy_(pol["w3"][None, :]); net[6].bias.copy_(pol["b3"])
    x = np.random.default_rng(0).standard_normal((50, 5)) * np.array([1e-3, 10.0, 1e-6, 5.0, 0.5])
    want = net(torch.from_numpy(x)).squeeze(1).detach().numpy()
    assert np.allclose(sw.policy_scores(x, pol), want, rtol=1e-12, atol=1e-12)


def _rand_cache(rng, Ly=2, H=2, G=3, n=7, w=5, d=8):
    K = rng.standard_normal((Ly, H, n, d))
    V = rng.standard_normal((Ly, H, n, d))
    Q = rng.standard_normal((Ly, H * G, w, d))
    return K, V, Q


def test_window_features_closed_forms():
    rng = np.random.default_rng(1)
    K, V, Q = _rand_cache(rng)
    Ly, H, n, d = K.shape
    # identical keys: every window query spreads evenly
    Ke = np.broadcast_to(K[:, :, :1], K.shape).copy()
    f = sw.window_features(Ke, V, np.arange(n), Q, n_seen=20)
    assert np.allclose(f[:, 0], 1.0 / n) and np.allclose(f[:, 2], 0.0, atol=1e-15)
    assert np.allclose(f[:, 3], math.log(n))
    assert np.allclose(f[:, 1], np.linalg.norm(V, axis=-1).mean(axis=(0, 1)))
    assert np.allclose(f[:, 4], np.arange(n) / 19.0)
    # one cached token: all mass on it, zero entropy
    f1 = sw.window_features(K[:, :, :1], V[:, :, :1], np.array([5]), Q, n_seen=1)
    assert np.allclose(f1[0, [0, 2, 3, 4]], [1.0, 0.0, 0.0, 5.0])
    # general case against library softmax per query head
    f = sw.window_features(K, V, np.arange(n), Q, n_seen=n)
    G = Q.shape[1] // H
    mass, hn, hd = [], np.zeros(n), np.zeros(n)
    for l in range(Ly):
        for qh in range(H * G):
            a = scipy.special.softmax(Q[l, qh] @ K[l, qh // G].T / math.sqrt(d), axis=1)
            ent = scipy.stats.entropy(a, axis=1)
            mass.append(a.mean(axis=0))
            hn += (a * ent[:, None]).sum(axis=0)
            hd += a.sum(axis=0)
    mass = np.array(mass)
    assert np.allclose(f[:, 0], mass.mean(axis=0)) and abs(f[:, 0].sum() - 1.0) < 1e-12
    assert np.allclose(f[:, 2], np.var(mass, axis=0))
    assert np.allclose(f[:, 3], hn / hd)


def test_stepwise_full_budget_keeps_everything():
    cfg = small_config("tiny").replace(T_dec=3, window=16, budget_ratio=1.0)
    inp = make_inputs(cfg)
    tr = []
    o = sw.run_stepwise(inp, cfg, make_policy(), trace=tr)
    assert all(len(k) == B for (_, _, _, B, k, _, _) in tr)
    assert np.array_equal(o["kept"][0], np.arange(cfg.lens[0] + cfg.T_dec))
    assert np.abs(o["x_comp"] - o["x_full"]).max() <= 1e-5 * np.abs(o["x_full"]).max()
    assert np.abs(o["kl"]).max() < 1e-6


@pytest.mark.parametrize("r", [0.25, 0.05])
def test_stepwise_budget_schedule_and_top_sets(r):
    cfg = small_config("tiny").replace(T_dec=6, window=16, budget_ratio=r)
    inp = make_inputs(cfg)
    tr = []
    sw.run_stepwise(inp, cfg, make_policy(seed=5), trace=tr)
    L = cfg.lens[0]
    prevB = None
    for (s, step, n_before, B, kept, sc, f) in tr:
        n_seen = L if step < 0 else L + step + 1
        assert B == max(math.floor(np.float32(r) * n_seen), cfg.budget_min)
        assert n_before == (L if step < 0 else prevB + 1)
        assert len(kept) == min(B, n_before)
        prevB = len(kept)
    # each prune keeps a top set by (score desc, position asc)
    prev = None
    for (s, step, n_before, B, kept, sc, f) in tr:
        cache_pos = np.arange(L) if step < 0 else np.append(prev, L + step)
        keep = np.isin(cache_pos, kept)
        assert keep.sum() == len(kept)
        if not keep.all():
            key = [(float(sc[i]), -int(cache_pos[i])) for i in range(len(cache_pos))]
            assert min(k for k, m in zip(key, keep) if m) > max(k for k, m in zip(key, keep) if not m)
        prev = kept


def test_stepwise_eviction_bound():
    # DistillCache Sec. 3.1.4: ||o - o_hat|| <= 2 max||v|| eps, with eps the
    # evicted mass of the full cache's attention; checked on the last step
    cfg = small_config("tiny").replace(T_dec=3, window=16, budget_ratio=0.25)
    inp = make_inputs(cfg)
    o = sw.run_stepwise(inp, cfg, make_policy(seed=9))
    L, d, G, t = cfg.lens[0], cfg.d, cfg.G, cfg.T_dec - 1
    K = np.concatenate([common.to64(inp["K"][0, 0]), common.to64(inp["Kd"][0, 0, 0, :t + 1])])
    V = np.concatenate([common.to64(inp["V"][0, 0]), common.to64(inp["Vd"][0, 0, 0, :t + 1])])
    # the student at step t held the final kept set plus anything evicted by the last prune
    tr = []
    sw.run_stepwise(inp, cfg, make_policy(seed=9), trace=tr)
    before_last = tr[-2][4].tolist() + [L + t]
    keep = np.zeros(L + t + 1, bool)
    keep[before_last] = True
    C = np.linalg.norm(V, axis=1).max()
    for g in range(G):
        q = common.to64(inp["Qd"][t, 0, 0, g])
        p = scipy.special.softmax(K @ q / math.sqrt(d))
        of = p @ V
        oc = (p[keep] / p[keep].sum()) @ V[keep]
        eps = p[~keep].sum()
        assert np.linalg.norm(of - oc) <= 2 * C * eps + 1e-9
        assert np.allclose(oc, o["x_comp"][0, t, g * d:(g + 1) * d], rtol=1e-5, atol=1e-5)
