"""Comparison helpers shared by the GPU parity tests (no test functions here)."""
import numpy as np
import torch


def as_np(t):
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy()
    return np.asarray(t)


def close(got, want, rtol, name="", floor=1e-6):
    """|got - want| <= rtol * (|want| + floor * max|want|), element-wise."""
    g = as_np(got).astype(np.float64)
    w = as_np(want).astype(np.float64)
    assert g.shape == w.shape, f"{name}: shape {g.shape} vs {w.shape}"
    scale = np.abs(w).max() if w.size else 0.0
    err = np.abs(g - w)
    lim = rtol * (np.abs(w) + floor * scale)
    bad = err > lim
    if bad.any():
        i = np.argmax(err - lim)
        idx = np.unravel_index(i, g.shape)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} elements off; worst at {idx}: "
                             f"got {g[idx]!r} want {w[idx]!r} (rtol {rtol})")


def to_dev(x, dev="cuda"):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(dev).contiguous()


def inputs_to(inp, dev="cuda"):
    out = {}
    for k, v in inp.items():
        out[k] = v.to(dev).contiguous() if isinstance(v, torch.Tensor) and k != "cu_seqlens" else v
    return out


def slots_to_dev(slots, stride, dev="cuda"):
    """Oracle slot lists -> the C ABI's slot_start [S][stride+1] / n_slots [S]."""
    S = len(slots)
    ss = np.zeros((S, stride + 1), dtype=np.int32)
    ns = np.zeros((S,), dtype=np.int32)
    for s, lst in enumerate(slots):
        ns[s] = len(lst)
        for k, (a, n) in enumerate(lst):
            ss[s, k] = a
        if lst:
            ss[s, len(lst)] = lst[-1][0] + lst[-1][1]
    return torch.from_numpy(ss).to(dev), torch.from_numpy(ns).to(dev)


def slots_from_dev(slot_start, n_slots):
    ss = as_np(slot_start)
    ns = as_np(n_slots)
    return [[(int(ss[s, k]), int(ss[s, k + 1] - ss[s, k])) for k in range(int(ns[s]))] for s in range(len(ns))]


def trees_to_dev(tr, dev="cuda"):
    out = {k: torch.from_numpy(np.ascontiguousarray(tr[k])).to(dev)
           for k in ("node_rel", "node_D", "node_mu", "op_util", "op_cost")}
    if tr.get("node_topo") is not None:   # uint32 records as int32 bits
        out["node_topo"] = torch.from_numpy(np.ascontiguousarray(tr["node_topo"]).view(np.int32)).to(dev)
    return out


def topo_np(t):
    """A device node_topo (int32 bits) as uint32 numpy."""
    return as_np(t).view(np.uint32)


def jaccard(a, b):
    a = np.asarray(a).astype(bool)
    b = np.asarray(b).astype(bool)
    u = np.logical_or(a, b).sum()
    return 1.0 if u == 0 else np.logical_and(a, b).sum() / u


def xhat_rows(x, w_dtype):
    """The vocab projection's input rows: x / sqrt(mean x^2 + 1e-6) rounded to
    W's dtype (through fp32), as float64 - the oracle's arithmetic."""
    from oracle import kl as okl
    return okl.rmsnorm_cast(np.asarray(x, dtype=np.float64), w_dtype)


def kl_flip_bound(xf_g, xc_g, xf_o, xc_o, W):
    """Per row: the number of x-hat elements whose W-dtype rounding differs
    between the GPU's decode outputs (xf_g, xc_g) and the oracle's (xf_o,
    xc_o), and a bound on how far those flips alone can move the KL.

    The flips change the logits by exactly dy = (x^_gpu - x^_oracle) W^T
    (full row) and dyh (compressed row); everything else about the rounded
    rows is identical. With P = softmax(y), Q = softmax(y^), g = y - y^:
      dKL/dy^ = Q - P                       -> |dKL| <= sum |Q - P| |dyh|
      dKL/dy  = P (g - E_P g)               -> |dKL| <= sum P |g - E_P g| |dy|
    to first order; the remainder is bounded by (1 + max|g - E_P g|) times the
    square of the largest logit change."""
    import torch
    wd = "bf16" if (isinstance(W, torch.Tensor) and W.dtype == torch.bfloat16) else "f32"
    from oracle.common import to64, logsumexp
    Wm = to64(W)
    hfg, hcg = xhat_rows(xf_g, wd), xhat_rows(xc_g, wd)
    hfo, hco = xhat_rows(xf_o, wd), xhat_rows(xc_o, wd)
    flips = (hfg != hfo).sum(axis=1) + (hcg != hco).sum(axis=1)
    y, yh = hfo @ Wm.T, hco @ Wm.T
    P = np.exp(y - logsumexp(y, axis=1)[:, None])
    Q = np.exp(yh - logsumexp(yh, axis=1)[:, None])
    dy, dyh = (hfg - hfo) @ Wm.T, (hcg - hco) @ Wm.T
    g = y - yh
    dev = np.abs(g - (P * g).sum(axis=1, keepdims=True))
    first = (np.abs(Q - P) * np.abs(dyh)).sum(axis=1) + (P * dev * np.abs(dy)).sum(axis=1)
    big = np.maximum(np.abs(dy).max(axis=1), np.abs(dyh).max(axis=1))
    return flips, first + (1.0 + dev.max(axis=1)) * (2.0 * big) ** 2


def check_kl(klv, xf, xc, W, kl_oracle, name="", xf_oracle=None, xc_oracle=None, atol=1e-3):
    """Per-step KL against the oracle.

    * stage: the GPU's KL against the oracle's KL of the GPU's own decode
      outputs, within atol;
    * end to end: against kl_oracle (the oracle's KL of its own decode
      outputs xf_oracle, xc_oracle), within atol where every x-hat element
      rounds to the same W-dtype value on both sides, and within atol plus
      kl_flip_bound elsewhere (x from fp32 decode differs from the fp64 one by
      ~1e-6 relative, which can flip a rounding of x-hat to bf16)."""
    from oracle import kl as okl
    n = int(np.prod(as_np(klv).shape))
    wd = "bf16" if W.dtype == torch.bfloat16 else "f32"
    Wc = W.detach().cpu()
    got = as_np(klv).reshape(n)
    xfg = as_np(xf).reshape(n, -1).astype(np.float32)
    xcg = as_np(xc).reshape(n, -1).astype(np.float32)
    stage = okl.kl_rows(xfg, xcg, Wc, wd)
    e_stage = np.abs(got - stage).max()
    want = np.asarray(kl_oracle).reshape(n)
    err = np.abs(got - want)
    if xf_oracle is None:
        xf_oracle, xc_oracle = xfg, xcg
    flips, bound = kl_flip_bound(xfg, xcg, np.asarray(xf_oracle).reshape(n, -1),
                                 np.asarray(xc_oracle).reshape(n, -1), Wc)
    lim = atol + bound
    print(f"  {name} max|dKL| stage={e_stage:.2e} end-to-end={err.max():.2e}; rows with flipped x-hat "
          f"roundings {int((flips > 0).sum())}/{n} (flips {int(flips.sum())}), largest flip bound "
          f"{bound.max():.2e}", flush=True)
    assert e_stage <= atol, (name, e_stage)
    bad = err > lim
    assert not bad.any(), (name, int(np.argmax(err - lim)), float(err.max()), float(lim[np.argmax(err - lim)]))


def oracle_on_taken(inp, cfg, o, taken, topo=None):
    """The oracle's pack, decode and KL of a given taken set (the GPU's), with
    the oracle's own relevance, trees and slots: x_comp [S][T_dec][d_model]
    and kl [S][T_dec]. topo (uint32 node records, the GPU's): tree shapes the
    taken set refers to; where they differ from the oracle's, the oracle's
    trees are rebuilt on them."""
    import oracle
    cu = inp["cu_seqlens"].numpy()
    trees = o.get("trees")
    if topo is not None and trees is not None and not np.array_equal(topo, trees["node_topo"]):
        trees = oracle.build_trees(inp["K"], inp["V"], inp["Qp"], o["lse"], o["rel"], o["head_sens"], cu,
                                   o["slots"], cfg, topo=topo)
    cache = oracle.pack(inp["K"], inp["V"], o["rel"], trees, as_np(taken), cu, o["slots"], cfg)
    xc = oracle.decode_all(cache, inp["Kd"], inp["Vd"], inp["Qd"], cfg.G)
    n = xc.shape[0] * xc.shape[1]
    kl = oracle.kl_rows(o["x_full"].reshape(n, -1), xc.reshape(n, -1), inp["W"], cfg.w_dtype)
    return xc, kl.reshape(xc.shape[0], xc.shape[1])
