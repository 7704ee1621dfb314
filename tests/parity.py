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
    return {k: torch.from_numpy(np.ascontiguousarray(tr[k])).to(dev)
            for k in ("node_rel", "node_D", "node_mu", "op_util", "op_cost")}


def jaccard(a, b):
    a = np.asarray(a).astype(bool)
    b = np.asarray(b).astype(bool)
    u = np.logical_or(a, b).sum()
    return 1.0 if u == 0 else np.logical_and(a, b).sum() / u


def check_kl(klv, xf, xc, W, kl_oracle, name="", e2e_atol=2e-2):
    """Per-step KL: the GPU's KL against the oracle's KL of the GPU's own
    decode outputs within 1e-3 absolute (the KL stage on the same inputs), and
    against the oracle's end-to-end KL within e2e_atol. The end-to-end gap is
    wider than the stage's because x-hat is rounded to W's dtype: a relative
    change of 1e-5 in x (fp32 decode against fp64) flips a few bf16 roundings,
    and each flip moves a KL near 15 by about 2e-3."""
    from oracle import kl as okl
    n = int(np.prod(as_np(klv).shape))
    wd = "bf16" if W.dtype == torch.bfloat16 else "f32"
    Wc = W.detach().cpu()
    got = as_np(klv).reshape(n)
    stage = okl.kl_rows(as_np(xf).reshape(n, -1).astype(np.float32), as_np(xc).reshape(n, -1).astype(np.float32),
                        Wc, wd)
    e_stage = np.abs(got - stage).max()
    e_e2e = np.abs(got - np.asarray(kl_oracle).reshape(n)).max()
    print(f"  {name} max|dKL| stage={e_stage:.2e} end-to-end={e_e2e:.2e}", flush=True)
    assert e_stage <= 1e-3, (name, e_stage)
    assert e_e2e <= e2e_atol, (name, e_e2e)
