"""Full-size end-to-end parity against the C++ oracle: the GPU path runs each
workload whole, at its real shape and in the launch configuration bench.py
times; the oracle (fp64, OpenMP on the host cores) recomputes whole
sequences of it from the same raw inputs. Sequences are independent (each
has its own budget, and nothing of the path crosses sequences), so a
sequence of the batch is an exact unit of comparison:

* mistral1 (8 KV heads x 4096 tokens, token-level top-B, 32 steps, vocab
  32768) and fulldepth (32 layers x 8 KV heads x 16384 tokens, DP slots, 64
  steps): the whole job;
* stress (4 x 32768 tokens): one sequence at a budget of 1/128 and another
  at 12.5%, on the same inputs;
* ragged (16 sequences of 2,053-29,761 tokens, exact regions): the longest,
  the shortest and two in between.

Checked per sequence: the slots, the budget spent (exact), the taken
operations (Jaccard >= 0.99), the packed rows of every segment whose layout
matches (keys and values at rel 2e-2 of bf16, ln mu), and at three sampled
decode steps (each step depends only on the appended tokens before it) the
decode outputs over both caches and the KL, the compressed side against the
oracle's pack and decode of the GPU's own taken set."""
import time

import numpy as np
import pytest
import torch

from oracle import cpp_oracle as co
from workload import get_config, make_inputs
from parity import as_np, close, jaccard, check_kl, slots_from_dev, topo_np

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[fullsize-e2e] {msg}", flush=True)


def _gpu_run(cfg, inp, steps):
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    out = comp.compress(inp)
    full = kvc.full_view(comp.pb, inp["K"], inp["V"])
    S, Dm = cfg.S, cfg.d_model
    xf = torch.empty((S, len(steps), Dm), dtype=torch.float32, device="cuda")
    xc = torch.empty_like(xf)
    row = torch.empty((S, Dm), dtype=torch.float32, device="cuda")
    for k, t in enumerate(steps):
        kvc.decode_attn(full, inp["Kd"], inp["Vd"], t + 1, cfg.T_dec, inp["Qd"][t], cfg.G, row, Dm)
        xf[:, k] = row
        kvc.decode_attn(out["cache"], inp["Kd"], inp["Vd"], t + 1, cfg.T_dec, inp["Qd"][t], cfg.G, row, Dm)
        xc[:, k] = row
    n = S * len(steps)
    klv = kvc.kl(xf.reshape(n, Dm), xc.reshape(n, Dm), inp["W"]).reshape(S, len(steps))
    torch.cuda.synchronize()
    return out, xf, xc, klv


def _sub(inp, cfg, s):
    """Sequence s of the batch as a one-sequence problem on the host."""
    cu = inp["cu_seqlens"]
    a, b = int(cu[s]), int(cu[s + 1])
    sub = {"cu_seqlens": torch.tensor([0, b - a], dtype=torch.int64),
           "K": inp["K"][:, :, a:b].cpu(), "V": inp["V"][:, :, a:b].cpu(), "Qp": inp["Qp"][s:s + 1].cpu(),
           "Qctx": inp["Qctx"][:, :, a:b].cpu(), "Qd": inp["Qd"][:, s:s + 1].cpu(),
           "Kd": inp["Kd"][:, :, s:s + 1].cpu(), "Vd": inp["Vd"][:, :, s:s + 1].cpu(), "W": inp["W"].cpu(),
           "hidden": None, "surprisal": None}
    if inp.get("hidden") is not None:
        h = inp["hidden"]
        sub["hidden"] = (h[:, a:b] if h.dim() == 3 else h[a:b]).cpu()
    if inp.get("surprisal") is not None:
        sub["surprisal"] = inp["surprisal"][a:b].cpu()
    return sub, cfg.replace(S=1, lens=[b - a]), a, b


def _oracle_select(sub, cfg_s, pre):
    """Floor + auction (or top-B) and pack on the oracle, given its scores,
    relevance, slots and trees (which do not depend on the budget)."""
    cu = np.array([0, cfg_s.lens[0]])
    if cfg_s.token_mode:
        taken, spent = co.token_topk(pre["rel"], cu, cfg_s)
    else:
        topo = pre["trees"]["node_topo"] if cfg_s.split_mode else None
        ft, fs = co.floor_select(pre["rel"], pre["head_sens"], pre["trees"]["op_cost"], cu, pre["slots"], cfg_s,
                                 topo=topo)
        taken, spent = co.auction(pre["trees"]["op_util"], pre["trees"]["op_cost"], ft, fs, cu, pre["slots"], cfg_s,
                                  topo=topo)
    cache = co.pack(sub["K"], sub["V"], pre["rel"], pre.get("trees"), taken, cu, pre["slots"], cfg_s)
    return taken, spent, cache


def _oracle_pre(sub, cfg_s):
    cu = np.array([0, cfg_s.lens[0]])
    t0 = time.perf_counter()
    pre = co.probe_scores(sub["K"], sub["V"], sub["Qp"], cu, cfg_s)
    pre.update(co.propagate(sub["K"], sub["Qctx"], pre["r0"], cu, cfg_s))
    t1 = time.perf_counter()
    pre["slots"], pre["trees"] = [[]], None
    if not cfg_s.token_mode:
        cq = kq = None
        if cfg_s.slot_len == 0:
            cq, kq = co.slot_costs(sub["hidden"], cu, cfg_s, sub.get("surprisal"))
        pre["slots"] = co.slots_for(cu, cfg_s, cq, kq)
        t2 = time.perf_counter()
        pre["cut_q"] = kq
        pre["trees"] = co.build_trees(sub["K"], sub["V"], sub["Qp"], pre["lse"], pre["rel"], pre["head_sens"], cu,
                                      pre["slots"], cfg_s, cut_q=kq)
        _log(f"  oracle: scores+propagation {t1 - t0:.1f}s, slots {t2 - t1:.1f}s, trees "
             f"{time.perf_counter() - t2:.1f}s ({co.threads()} threads)")
    return pre


def _check_sequence(cfg, inp, out, xf, xc, klv, steps, s, pre=None, tag=""):
    sub, cfg_s, a, b = _sub(inp, cfg, s)
    L = b - a
    _log(f"{tag} sequence {s}: {L} tokens")
    if pre is None:
        pre = _oracle_pre(sub, cfg_s)
    taken_o, spent_o, cache_o = _oracle_select(sub, cfg_s, pre)
    assert int(as_np(out["spent"])[s]) == int(spent_o[0]), (int(as_np(out["spent"])[s]), int(spent_o[0]))
    if cfg.token_mode:
        taken_g = as_np(out["taken"])[:, :, a:b]
    else:
        assert slots_from_dev(out["slot_start"], out["n_slots"])[s] == pre["slots"][0]
        taken_g = as_np(out["taken"])[:, :, 2 * a:2 * b]
    j = jaccard(taken_g, taken_o)
    # packed rows of every (l, h) segment whose layout matches the oracle's
    c = out["cache"]
    off_g, len_g = as_np(c["seg_off"])[s], as_np(c["seg_len"])[s]
    matched = rows = 0
    Kg = Vg = None
    worst = 0.0
    for l in range(cfg.Ly):
        for h in range(cfg.H):
            og, ng = int(off_g[l, h]), int(len_g[l, h])
            oo, no = int(cache_o["seg_off"][0, l, h]), int(cache_o["seg_len"][0, l, h])
            pg = as_np(c["pos"][og:og + ng])
            if ng != no or not np.array_equal(pg, cache_o["pos"][oo:oo + no]):
                continue
            matched += 1
            rows += ng
            Kg = c["K"][og:og + ng].float().cpu().numpy()
            Vg = c["V"][og:og + ng].float().cpu().numpy()
            Ko = co.rows_as_float64(cache_o["K"][oo:oo + no])
            Vo = co.rows_as_float64(cache_o["V"][oo:oo + no])
            close(Kg, Ko, 2e-2, f"packed K (l={l}, h={h})", floor=1e-2)
            close(Vg, Vo, 2e-2, f"packed V (l={l}, h={h})", floor=1e-2)
            lg = as_np(c["lnmu"][og:og + ng]).astype(np.float64)
            lo = cache_o["lnmu"][oo:oo + no].astype(np.float64)
            assert np.all(np.abs(lg - lo) <= 2e-2 * np.abs(lo) + 1e-3), (l, h)
            worst = max(worst, float(np.abs(lg - lo).max()) if ng else 0.0)
    units = cfg.Ly * cfg.H
    _log(f"  jaccard {j:.5f}, spent {int(spent_o[0])}, segments with the oracle's layout {matched}/{units} "
         f"({rows} rows compared), max |d ln mu| {worst:.2e}")
    assert j >= 0.99, j
    assert matched >= 0.9 * units, matched
    # the oracle's pack of the GPU's taken set (on the GPU's tree shapes), and
    # decode + KL at the steps
    trees_g = pre.get("trees")
    if cfg.split_mode:
        topo_g = topo_np(out["trees"]["node_topo"])[:, :, 2 * a:2 * b]
        same = float((topo_g == trees_g["node_topo"]).mean())
        _log(f"  tree shapes equal to the oracle's at {same:.6f} of the records; three-way splits "
             f"{int((trees_g['op_cost'] == 2).sum())}, taken {int(((trees_g['op_cost'] == 2) & (taken_o > 0)).sum())}")
        assert same >= 0.99, same
        if same < 1.0:
            trees_g = co.build_trees(sub["K"], sub["V"], sub["Qp"], pre["lse"], pre["rel"], pre["head_sens"],
                                     np.array([0, L]), pre["slots"], cfg_s, topo=topo_g)
    if np.array_equal(taken_g, taken_o) and trees_g is pre.get("trees"):
        cache_g = cache_o
    else:
        cu = np.array([0, L])
        cache_g = co.pack(sub["K"], sub["V"], pre["rel"], trees_g, taken_g, cu, pre["slots"], cfg_s)
    fv = co.full_view(sub["K"], sub["V"], np.array([0, L]))
    xf_o = np.stack([co.decode_step(fv, sub["Kd"], sub["Vd"], sub["Qd"][t], t, cfg.G)[0] for t in steps])
    xc_o = np.stack([co.decode_step(cache_g, sub["Kd"], sub["Vd"], sub["Qd"][t], t, cfg.G)[0] for t in steps])
    close(xf[s], xf_o, 2e-2, "x_full", floor=1e-3)
    close(xc[s], xc_o, 2e-2, "x_comp", floor=1e-2)
    kl_o = co.kl_rows(xf_o, xc_o, sub["W"])
    check_kl(klv[s], xf[s], xc[s], inp["W"], kl_o, f"{cfg.name} seq {s}", xf_o, xc_o)
    return pre


def _run(name, seqs, steps, extra=None, cfg_kw=None):
    cfg = get_config(name).replace(**(cfg_kw or {}))
    t0 = time.perf_counter()
    inp = make_inputs(cfg, device="cuda")
    torch.cuda.synchronize()
    _log(f"{name}: inputs in {time.perf_counter() - t0:.1f}s (S={cfg.S}, T={cfg.T}, Ly={cfg.Ly}, H={cfg.H})")
    out, xf, xc, klv = _gpu_run(cfg, inp, steps)
    _log(f"{name}: GPU path done")
    pres = {}
    for s in seqs:
        pres[s] = _check_sequence(cfg, inp, out, xf, xc, klv, steps, s, tag=name)
    if extra is not None:
        extra(inp, pres)
    del inp, out
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_fullsize_e2e_mistral1():
    _run("mistral1", [0], list(range(32)))


@pytest.mark.timeout(900)
def test_fullsize_e2e_fulldepth():
    _run("fulldepth", [0], [0, 31, 63])


@pytest.mark.timeout(900)
def test_fullsize_e2e_fulldepth_tree_splits():
    # curvature-candidate cuts and salient three-way splits (split_mode 1)
    _run("fulldepth", [0], [0, 63], cfg_kw={"split_mode": 1})


@pytest.mark.timeout(900)
def test_fullsize_e2e_stress_both_budgets():
    steps = [0, 63, 127]

    def at_eighth(inp, pres):
        # the same inputs at 12.5%: the scores, relevance, slots and trees do
        # not depend on the budget, so the oracle reuses them
        cfg8 = get_config("stress8")
        out, xf, xc, klv = _gpu_run(cfg8, inp, steps)
        _log("stress8: GPU path done")
        _check_sequence(cfg8, inp, out, xf, xc, klv, steps, 1, pre=pres[1], tag="stress8")
        _check_sequence(cfg8, inp, out, xf, xc, klv, steps, 2, tag="stress8")

    _run("stress", [1], steps, extra=at_eighth)


@pytest.mark.timeout(900)
def test_fullsize_e2e_ragged():
    _run("ragged", [15, 0, 7, 10], [0, 128, 255])
