"""GPU parity at the full size of the two batched workloads, in the launch
configuration of `bench.py --config stress|ragged`: stress (4 x 32768 tokens,
32 layers x 8 KV heads, fixed 64-token slots, budget 1/128) and ragged (16
sequences of 2048-32768 tokens with exact prompt / recent / suffix regions,
budget 1/4). At these sizes K holds more than 2^31 elements (4.3 and 4.7
billion), so every index into it must be 64-bit; the checks sample units of
the first, a middle and the last sequence:

* probe scores of sampled (sequence, layer, KV head) units against the oracle
  (softmax definition, fp64) from the raw inputs;
* the budget is spent exactly and every sequence's segments hold its spent
  entries plus its exact regions, segments contiguous in (layer, KV head,
  sequence) order, positions strictly increasing inside each segment;
* one decode step over the packed and over the full cache for sampled units
  against the definition (softmax over the segment's entries with their
  ln mu and the appended tokens).

Inputs come from the seeded generator on the GPU; no expected value comes from
the HIP path."""
import math

import numpy as np
import pytest
import torch

from oracle.common import to64, regions, budgets
from oracle.score import _unit_scores
from workload import get_config, make_inputs
from parity import close, as_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=["stress", "ragged"])
def run(request):
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor
    cfg = get_config(request.param)
    print(f"[fullsize-batch] generating {cfg.name} inputs on the GPU", flush=True)
    inp = make_inputs(cfg, device="cuda")
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    out = comp.compress(inp)
    torch.cuda.synchronize()
    print(f"[fullsize-batch] {cfg.name} compressed", flush=True)
    r = {"cfg": cfg, "inp": inp, "comp": comp, "out": out, "kvc": kvc}
    del inp, comp, out
    yield r
    r.clear()
    torch.cuda.empty_cache()


def _samples(cfg):
    S, Ly, H = cfg.S, cfg.Ly, cfg.H
    return [(0, 0, 0), (S // 2, Ly // 2 - 3, H // 2 + 1), (S - 1, Ly - 1, H - 1)]


def test_batch_scores_sampled(run):
    cfg, inp, out = run["cfg"], run["inp"], run["out"]
    G, P = cfg.G, cfg.P
    cu = [int(x) for x in inp["cu_seqlens"]]
    for (s, l, h) in _samples(cfg):
        a, b = cu[s], cu[s + 1]
        print(f"  {cfg.name} scores s={s} l={l} h={h} L={b - a}", flush=True)
        K = to64(inp["K"][l, h, a:b].cpu())
        V = to64(inp["V"][l, h, a:b].cpu())
        Q = to64(inp["Qp"][s, l, h * G:(h + 1) * G].cpu()).reshape(G * P, cfg.d)
        r0, feats, lse, ent, sens = _unit_scores(Q, K, V, G, P)
        close(out["r0"][l, h, a:b], r0, 1e-3, "r0", floor=1e-3)
        close(out["lse"][s, l, h * G:(h + 1) * G].reshape(G * P), lse, 1e-3, "lse")
        close(out["ent"][s, l, h * G:(h + 1) * G].reshape(G * P), ent, 1e-3, "entropy", floor=1e-3)
        close(np.array([float(out["head_sens"][s, l, h])]), np.array([sens]), 1e-3, "head sensitivity")


def test_batch_budget_and_segments(run):
    cfg, out = run["cfg"], run["out"]
    Ly, H = cfg.Ly, cfg.H
    cache = out["cache"]
    seg_off = as_np(cache["seg_off"])          # [S][Ly][H]
    seg_len = as_np(cache["seg_len"]).astype(np.int64)
    spent = as_np(out["spent"]).astype(np.int64)
    bud = budgets(cfg.lens, cfg)
    for s, L in enumerate(cfg.lens):
        pe, c0, c1, _ = regions(L, cfg)
        assert spent[s] == bud[s]["alloc"], (s, int(spent[s]), bud[s])
        assert int(seg_len[s].sum()) == spent[s] + Ly * H * (pe + L - c1), s
    off = np.transpose(seg_off, (1, 2, 0)).reshape(-1)
    ln = np.transpose(seg_len, (1, 2, 0)).reshape(-1)
    assert off[0] == 0 and np.array_equal(off[1:], off[:-1] + ln[:-1])
    pos = as_np(cache["pos"])
    for (s, l, h) in _samples(cfg):
        p = pos[seg_off[s, l, h]:seg_off[s, l, h] + seg_len[s, l, h]].astype(np.int64)
        assert np.all(np.diff(p) > 0) and p[0] >= 0 and p[-1] < cfg.lens[s], (s, l, h)


def test_batch_decode_sampled(run):
    cfg, inp, comp, out, kvc = run["cfg"], run["inp"], run["comp"], run["out"], run["kvc"]
    G, d, Td = cfg.G, cfg.d, cfg.T_dec
    c = 1.0 / math.sqrt(d)
    t = Td - 1
    cu = [int(x) for x in inp["cu_seqlens"]]
    full = kvc.full_view(comp.pb, inp["K"], inp["V"])
    for label, cache in (("packed", out["cache"]), ("full", full)):
        dec = kvc.Decoder(cache, G, Td)
        x = torch.empty((cfg.S, cfg.d_model), dtype=torch.float32, device="cuda")
        o = torch.empty((cfg.S, cfg.Ly, cfg.H * G, d), dtype=torch.float32, device="cuda")
        dec.step(inp["Kd"], inp["Vd"], t + 1, inp["Qd"][t], x, cfg.d_model, o_out=o)
        torch.cuda.synchronize()
        go = as_np(o)
        seg_off = as_np(cache["seg_off"])
        seg_len = as_np(cache["seg_len"])
        for (s, l, h) in _samples(cfg):
            a, n = int(seg_off[s, l, h]), int(seg_len[s, l, h])
            print(f"  {cfg.name} decode {label} s={s} l={l} h={h} entries={n}", flush=True)
            if label == "full":
                assert a == (l * cfg.H + h) * cfg.T + cu[s] and n == cu[s + 1] - cu[s]
            Ke = np.concatenate([to64(cache["K"][a:a + n].cpu()), to64(inp["Kd"][l, h, s, :t + 1].cpu())])
            Ve = np.concatenate([to64(cache["V"][a:a + n].cpu()), to64(inp["Vd"][l, h, s, :t + 1].cpu())])
            lm = np.zeros(n + t + 1)
            if cache.get("lnmu") is not None:
                lm[:n] = as_np(cache["lnmu"][a:a + n]).astype(np.float64)
            q = to64(inp["Qd"][t, s, l, h * G:(h + 1) * G].cpu())
            z = c * (q @ Ke.T) + lm[None, :]
            p = np.exp(z - z.max(axis=1, keepdims=True))
            want = (p / p.sum(axis=1, keepdims=True)) @ Ve
            close(go[s, l, h * G:(h + 1) * G], want, 2e-2, f"decode o ({label})", floor=1e-2)
        close(as_np(x), go.sum(axis=1).reshape(cfg.S, -1), 1e-5, "x = sum over layers", floor=1e-5)
