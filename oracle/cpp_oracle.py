"""ctypes binding of the C++ oracle (oracle/cpp/kvc_oracle.cpp).

TEST INFRASTRUCTURE ONLY (see the package docstring): the same stages as the
Python oracle, in C++17 with OpenMP over (sequence, layer, KV head) units and
fp64 arithmetic, for inputs the Python oracle cannot finish (full-size
workloads) and for the CPU baseline of bench.py. Function names and results
follow the Python oracle's; packed caches keep their rows in the cache dtype
(bf16 bits as uint16, or fp32).

The library is compiled on first use when it is missing (g++, -O3,
-march=x86-64-v3, OpenMP); OMP_NUM_THREADS sets its thread count.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "cpp", "kvc_oracle.cpp")
LIB = os.path.join(HERE, "cpp", "libkvc_oracle.so")
CXXFLAGS = ["-O3", "-march=x86-64-v3", "-fopenmp", "-std=c++17", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["g++"] + CXXFLAGS + ["-o", tmp, SRC], check=True)
        os.replace(tmp, LIB)
    return LIB


class Shape(C.Structure):
    _fields_ = [("S", C.c_int32), ("Ly", C.c_int32), ("H", C.c_int32), ("G", C.c_int32), ("d", C.c_int32),
                ("P", C.c_int32), ("dtype", C.c_int32), ("T", C.c_int64), ("cu", C.POINTER(C.c_int64))]


class Params(C.Structure):
    _fields_ = [("budget_ratio", C.c_float), ("budget_min", C.c_int32), ("prompt_exact", C.c_int32),
                ("recent_exact", C.c_int32), ("suffix_exact", C.c_int32), ("n_hops", C.c_int32),
                ("n_seeds", C.c_int32), ("hop_weight", C.c_float), ("n_dprobe", C.c_int32),
                ("w_attn", C.c_float), ("w_value", C.c_float), ("value_base", C.c_float),
                ("floor_frac", C.c_float), ("token_mode", C.c_int32), ("slot_len", C.c_int32),
                ("slot_min", C.c_int32), ("slot_max", C.c_int32), ("slot_target", C.c_int32),
                ("lambda_len", C.c_float), ("lambda_curv", C.c_float), ("lambda_surp", C.c_float),
                ("rope_base", C.c_double), ("split_mode", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        _lib.ko_threads.restype = C.c_int
        _lib.ko_pack_count.restype = C.c_int64
    return _lib


def threads() -> int:
    return int(lib().ko_threads())


_DT = {torch.bfloat16: 1, torch.float32: 0}


class _Keep:
    """Holds the contiguous host copies whose pointers were handed out."""

    def __init__(self):
        self.refs = []

    def ptr(self, x):
        if x is None:
            return None
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16)
            self.refs.append(x)
            return C.c_void_p(x.data_ptr())
        x = np.ascontiguousarray(x)
        self.refs.append(x)
        return C.c_void_p(x.ctypes.data)


def _cu(cu):
    return np.ascontiguousarray(np.asarray(cu, dtype=np.int64))


def _shape(cu, cfg, dtype):
    cu = _cu(cu)
    sh = Shape(S=len(cu) - 1, Ly=cfg.Ly, H=cfg.H, G=cfg.G, d=cfg.d, P=cfg.P, dtype=dtype, T=int(cu[-1]),
               cu=cu.ctypes.data_as(C.POINTER(C.c_int64)))
    sh._cu = cu
    return sh


def _params(cfg):
    return Params(budget_ratio=cfg.budget_ratio, budget_min=cfg.budget_min, prompt_exact=cfg.prompt_exact,
                  recent_exact=cfg.recent_exact, suffix_exact=cfg.suffix_exact, n_hops=cfg.n_hops,
                  n_seeds=cfg.n_seeds, hop_weight=cfg.hop_weight, n_dprobe=cfg.n_dprobe, w_attn=cfg.w_attn,
                  w_value=cfg.w_value, value_base=cfg.value_base, floor_frac=cfg.floor_frac,
                  token_mode=int(bool(cfg.token_mode)), slot_len=cfg.slot_len, slot_min=cfg.slot_min,
                  slot_max=cfg.slot_max, slot_target=cfg.slot_target, lambda_len=cfg.lambda_len,
                  lambda_curv=cfg.lambda_curv, lambda_surp=getattr(cfg, "lambda_surp", 0.0),
                  rope_base=float(cfg.rope_base), split_mode=int(getattr(cfg, "split_mode", 0)))


def _dtype_of(t):
    return _DT[t.dtype] if isinstance(t, torch.Tensor) else (1 if t.dtype == np.uint16 else 0)


def regions(L, cfg):
    out = np.zeros(4, dtype=np.int64)
    lib().ko_regions(C.c_int64(L), C.byref(_params(cfg)), out.ctypes.data_as(C.c_void_p))
    return tuple(int(v) for v in out)


def budgets(cu, cfg):
    sh = _shape(cu, cfg, 1)
    S = sh.S
    B, A, F = (np.zeros(S, dtype=np.int64) for _ in range(3))
    lib().ko_budgets(C.byref(sh), C.byref(_params(cfg)), B.ctypes.data_as(C.c_void_p),
                     A.ctypes.data_as(C.c_void_p), F.ctypes.data_as(C.c_void_p))
    return B, A, F


def probe_scores(K, V, Qp, cu, cfg):
    kp = _Keep()
    sh = _shape(cu, cfg, _DT[K.dtype])
    Ly, H, T = cfg.Ly, cfg.H, sh.T
    S = sh.S
    r0 = np.zeros((Ly, H, T), dtype=np.float32)
    feats = np.zeros((5, Ly, H, T), dtype=np.float32)
    lse = np.zeros((S, Ly, H * cfg.G, cfg.P), dtype=np.float32)
    ent = np.zeros_like(lse)
    sens = np.zeros((S, Ly, H), dtype=np.float32)
    lib().ko_probe_scores(C.byref(sh), kp.ptr(K), kp.ptr(V), kp.ptr(Qp), kp.ptr(r0), kp.ptr(feats), kp.ptr(lse),
                          kp.ptr(ent), kp.ptr(sens))
    return {"r0": r0, "feats": feats, "lse": lse, "ent": ent, "head_sens": sens}


def propagate(K, Qctx, r0, cu, cfg):
    kp = _Keep()
    sh = _shape(cu, cfg, _DT[K.dtype])
    rel = np.zeros((cfg.Ly, cfg.H, sh.T), dtype=np.float32)
    seeds = np.full((cfg.n_hops, sh.S, cfg.Ly, cfg.H, cfg.n_seeds), -1, dtype=np.int32)
    lib().ko_propagate(C.byref(sh), C.byref(_params(cfg)), kp.ptr(K), kp.ptr(Qctx),
                       kp.ptr(np.asarray(r0, dtype=np.float32)), kp.ptr(rel), kp.ptr(seeds))
    return {"rel": rel, "seeds": seeds}


def slot_costs(hidden, cu, cfg, surprisal=None):
    kp = _Keep()
    sh = _shape(cu, cfg, _DT[hidden.dtype])
    D = hidden.shape[0] if hidden.dim() == 3 else 1
    dim = hidden.shape[-1]
    NW = cfg.slot_max - cfg.slot_min + 1
    cost_q = np.zeros((sh.T, NW), dtype=np.int64)
    cut_q = np.zeros((sh.T,), dtype=np.int64)
    sur = None if surprisal is None else surprisal.detach().cpu().float()
    lib().ko_slot_costs(C.byref(sh), C.byref(_params(cfg)), kp.ptr(hidden), C.c_int32(dim), C.c_int32(D),
                        kp.ptr(sur), kp.ptr(cost_q), kp.ptr(cut_q))
    return cost_q, cut_q


def slot_stride(cu, cfg):
    cu = _cu(cu)
    m = int(max(cu[1:] - cu[:-1]))
    smin = cfg.slot_len if cfg.slot_len > 0 else cfg.slot_min
    return (m + max(smin, 1) - 1) // max(smin, 1) + 1


def slot_arrays(cu, cfg, cost_q=None, cut_q=None):
    """slot_start [S][stride+1] int32, n_slots [S] int32 (DP when slot_len == 0)."""
    kp = _Keep()
    sh = _shape(cu, cfg, 1)
    stride = slot_stride(cu, cfg)
    ss = np.zeros((sh.S, stride + 1), dtype=np.int32)
    ns = np.zeros((sh.S,), dtype=np.int32)
    lib().ko_slots(C.byref(sh), C.byref(_params(cfg)), kp.ptr(cost_q), kp.ptr(cut_q), C.c_int32(stride), kp.ptr(ss),
                   kp.ptr(ns))
    return ss, ns


def slots_from_arrays(ss, ns):
    return [[(int(ss[s, k]), int(ss[s, k + 1] - ss[s, k])) for k in range(int(ns[s]))] for s in range(len(ns))]


def slots_to_arrays(slots, stride):
    S = len(slots)
    ss = np.zeros((S, stride + 1), dtype=np.int32)
    ns = np.zeros((S,), dtype=np.int32)
    for s, lst in enumerate(slots):
        ns[s] = len(lst)
        for k, (a, n) in enumerate(lst):
            ss[s, k] = a
        if lst:
            ss[s, len(lst)] = lst[-1][0] + lst[-1][1]
    return ss, ns


def slots_for(cu, cfg, cost_q=None, cut_q=None):
    return slots_from_arrays(*slot_arrays(cu, cfg, cost_q, cut_q))


def _topo(topo):
    return None if topo is None else np.asarray(topo, dtype=np.uint32)


def build_trees(K, V, Qp, lse, rel, head_sens, cu, slots, cfg, cut_q=None, topo=None):
    """Tree arrays as the Python oracle's build_trees (node_topo included);
    cut_q: the partition's int64 [T] cut scores (split_mode 1) or None; topo:
    node records whose shapes are used instead of deciding them, or None."""
    kp = _Keep()
    sh = _shape(cu, cfg, _DT[K.dtype])
    stride = slot_stride(cu, cfg)
    ss, ns = slots_to_arrays(slots, stride)
    shp = (cfg.Ly, cfg.H, 2 * sh.T)
    out = {k: np.zeros(shp, dtype=np.float32) for k in ("node_rel", "node_D", "node_mu", "op_util")}
    out["op_cost"] = np.zeros(shp, dtype=np.uint8)
    out["node_topo"] = np.full(shp, 0xFFFFFFFF, dtype=np.uint32)
    cq = None if cut_q is None else np.asarray(cut_q, dtype=np.int64)
    lib().ko_build_trees(C.byref(sh), C.byref(_params(cfg)), kp.ptr(K), kp.ptr(V), kp.ptr(Qp),
                         kp.ptr(np.asarray(lse, dtype=np.float32)), kp.ptr(np.asarray(rel, dtype=np.float32)),
                         kp.ptr(np.asarray(head_sens, dtype=np.float32)), kp.ptr(ss), kp.ptr(ns), C.c_int32(stride),
                         kp.ptr(cq), kp.ptr(_topo(topo)), kp.ptr(out["node_rel"]), kp.ptr(out["node_D"]), kp.ptr(out["node_mu"]),
                         kp.ptr(out["op_util"]), kp.ptr(out["op_cost"]), kp.ptr(out["node_topo"]))
    return out


def floor_select(rel, head_sens, op_cost, cu, slots, cfg, topo=None):
    kp = _Keep()
    sh = _shape(cu, cfg, 1)
    stride = slot_stride(cu, cfg)
    ss, ns = slots_to_arrays(slots, stride)
    taken = np.zeros((cfg.Ly, cfg.H, 2 * sh.T), dtype=np.uint8)
    spent = np.zeros((sh.S,), dtype=np.int64)
    lib().ko_floor(C.byref(sh), C.byref(_params(cfg)), kp.ptr(np.asarray(rel, dtype=np.float32)),
                   kp.ptr(np.asarray(head_sens, dtype=np.float32)), kp.ptr(np.asarray(op_cost, dtype=np.uint8)),
                   kp.ptr(_topo(topo)), kp.ptr(ss), kp.ptr(ns), C.c_int32(stride), kp.ptr(taken), kp.ptr(spent))
    return taken, spent


def auction(op_util, op_cost, floor_taken, spent_floor, cu, slots, cfg, topo=None):
    kp = _Keep()
    sh = _shape(cu, cfg, 1)
    stride = slot_stride(cu, cfg)
    ss, ns = slots_to_arrays(slots, stride)
    taken = np.array(floor_taken, dtype=np.uint8, copy=True)
    spent = np.array(spent_floor, dtype=np.int64, copy=True)
    lib().ko_auction(C.byref(sh), C.byref(_params(cfg)), kp.ptr(np.asarray(op_util, dtype=np.float32)),
                     kp.ptr(np.asarray(op_cost, dtype=np.uint8)), kp.ptr(_topo(topo)), kp.ptr(ss), kp.ptr(ns),
                     C.c_int32(stride), kp.ptr(taken), kp.ptr(spent))
    return taken, spent


def token_topk(rel, cu, cfg):
    kp = _Keep()
    sh = _shape(cu, cfg, 1)
    taken = np.zeros((cfg.Ly, cfg.H, sh.T), dtype=np.uint8)
    spent = np.zeros((sh.S,), dtype=np.int64)
    lib().ko_token_topk(C.byref(sh), C.byref(_params(cfg)), kp.ptr(np.asarray(rel, dtype=np.float32)),
                        kp.ptr(taken), kp.ptr(spent))
    return taken, spent


def pack(K, V, rel, trees, taken, cu, slots, cfg):
    """Packed cache: K, V [N][d] in the cache dtype (uint16 bf16 bits or
    float32), lnmu f32, pos i32, seg_off/seg_len [S][Ly][H], dtype."""
    kp = _Keep()
    dt = _DT[K.dtype]
    sh = _shape(cu, cfg, dt)
    stride = slot_stride(cu, cfg)
    ss, ns = slots_to_arrays(slots, stride)
    tk = np.asarray(taken, dtype=np.uint8)
    topo = _topo(trees.get("node_topo")) if trees is not None else None
    N = int(lib().ko_pack_count(C.byref(sh), C.byref(_params(cfg)), kp.ptr(tk), kp.ptr(topo), kp.ptr(ss),
                                kp.ptr(ns), C.c_int32(stride)))
    rdt = np.uint16 if dt == 1 else np.float32
    out = {"K": np.zeros((N, cfg.d), dtype=rdt), "V": np.zeros((N, cfg.d), dtype=rdt),
           "lnmu": np.zeros(N, dtype=np.float32), "pos": np.zeros(N, dtype=np.int32),
           "seg_off": np.zeros((sh.S, cfg.Ly, cfg.H), dtype=np.int64),
           "seg_len": np.zeros((sh.S, cfg.Ly, cfg.H), dtype=np.int32), "dtype": dt}
    nr = trees["node_rel"] if trees is not None else np.zeros(1, dtype=np.float32)
    nm = trees["node_mu"] if trees is not None else np.zeros(1, dtype=np.float32)
    lib().ko_pack(C.byref(sh), C.byref(_params(cfg)), kp.ptr(K), kp.ptr(V), kp.ptr(np.asarray(rel, dtype=np.float32)),
                  kp.ptr(np.asarray(nr, dtype=np.float32)), kp.ptr(np.asarray(nm, dtype=np.float32)), kp.ptr(topo),
                  kp.ptr(tk),
                  kp.ptr(ss), kp.ptr(ns), C.c_int32(stride), kp.ptr(out["K"]), kp.ptr(out["V"]),
                  kp.ptr(out["lnmu"]), kp.ptr(out["pos"]), kp.ptr(out["seg_off"]), kp.ptr(out["seg_len"]))
    return out


def rows_as_float64(a):
    """Packed rows (uint16 bf16 bits or float32) as float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def full_view(K, V, cu):
    """The uncompressed cache as a ragged cache over K, V themselves."""
    cu = _cu(cu)
    Ly, H, T, d = K.shape
    S = len(cu) - 1
    seg_off = np.zeros((S, Ly, H), dtype=np.int64)
    seg_len = np.zeros((S, Ly, H), dtype=np.int32)
    for l in range(Ly):
        for h in range(H):
            seg_off[:, l, h] = (l * H + h) * T + cu[:-1]
            seg_len[:, l, h] = cu[1:] - cu[:-1]
    return {"K": K, "V": V, "lnmu": None, "pos": None, "seg_off": seg_off, "seg_len": seg_len,
            "dtype": _DT[K.dtype]}


def decode_step(cache, Kd, Vd, Qd_t, t, G):
    """x [S][H*G*d] float32 for decode step t (appended tokens 0..t)."""
    kp = _Keep()
    S, Ly, HG, d = Qd_t.shape
    H = HG // G
    dt = cache["dtype"]
    assert _DT[Kd.dtype] == dt and _DT[Qd_t.dtype] == dt
    x = np.zeros((S, HG * d), dtype=np.float32)
    lnmu = cache.get("lnmu")
    lib().ko_decode_step(C.c_int32(S), C.c_int32(Ly), C.c_int32(H), C.c_int32(G), C.c_int32(d), C.c_int32(dt),
                         kp.ptr(cache["K"]), kp.ptr(cache["V"]), kp.ptr(lnmu), kp.ptr(cache["seg_off"]),
                         kp.ptr(cache["seg_len"]), kp.ptr(Kd), kp.ptr(Vd), C.c_int32(Kd.shape[3]), C.c_int32(t),
                         kp.ptr(Qd_t), kp.ptr(x))
    return x


def decode_steps(cache, Kd, Vd, Qd, G, steps):
    """x [S][len(steps)][H*G*d] float32 for the listed decode steps."""
    return np.stack([decode_step(cache, Kd, Vd, Qd[t], t, G) for t in steps], axis=1)


def kl_rows(x_full, x_comp, W, w_dtype=None):
    kp = _Keep()
    xf = np.ascontiguousarray(x_full, dtype=np.float32)
    xc = np.ascontiguousarray(x_comp, dtype=np.float32)
    n, dm = xf.shape
    kl = np.zeros(n, dtype=np.float32)
    lib().ko_kl_rows(C.c_int64(n), C.c_int32(dm), C.c_int32(W.shape[0]), kp.ptr(xf), kp.ptr(xc), kp.ptr(W),
                     C.c_int32(_DT[W.dtype]), kp.ptr(kl))
    return kl


def compress(inp, cfg, timings=None):
    """Compression stages on the oracle (score, propagate, slots, trees,
    floor + auction or token top-B, pack). ``timings`` (a dict) receives the
    wall time of each stage in seconds."""
    import time
    cu = inp["cu_seqlens"].numpy() if isinstance(inp["cu_seqlens"], torch.Tensor) else inp["cu_seqlens"]
    out = {}

    def tick(name, t0):
        if timings is not None:
            timings[name] = timings.get(name, 0.0) + time.perf_counter() - t0
        return time.perf_counter()

    t = time.perf_counter()
    sc = probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    out.update(sc)
    t = tick("score", t)
    pr = propagate(inp["K"], inp["Qctx"], sc["r0"], cu, cfg)
    out.update(pr)
    rel = pr["rel"]
    t = tick("propagate", t)
    trees = None
    if cfg.token_mode:
        slots = [[] for _ in range(len(cu) - 1)]
        taken, spent = token_topk(rel, cu, cfg)
        t = tick("auction", t)
    else:
        cost_q = cut_q = None
        if cfg.slot_len == 0:
            cost_q, cut_q = slot_costs(inp["hidden"], cu, cfg, inp.get("surprisal"))
            out["dp_cost_q"], out["dp_cut_q"] = cost_q, cut_q
        slots = slots_for(cu, cfg, cost_q, cut_q)
        t = tick("partition", t)
        trees = build_trees(inp["K"], inp["V"], inp["Qp"], sc["lse"], rel, sc["head_sens"], cu, slots, cfg,
                            cut_q=cut_q)
        out["trees"] = trees
        t = tick("trees", t)
        topo = trees["node_topo"]
        ftaken, fspent = floor_select(rel, sc["head_sens"], trees["op_cost"], cu, slots, cfg, topo=topo)
        out["floor_taken"], out["floor_spent"] = ftaken, fspent
        taken, spent = auction(trees["op_util"], trees["op_cost"], ftaken, fspent, cu, slots, cfg, topo=topo)
        t = tick("auction", t)
    out["slots"], out["taken"], out["spent"] = slots, taken, spent
    out["cache"] = pack(inp["K"], inp["V"], rel, trees, taken, cu, slots, cfg)
    tick("pack", t)
    return out


def run_pipeline(inp, cfg, steps=None):
    """compress, then decode over both caches at the listed steps (all when
    None) and the KL of those rows; x_full/x_comp [S][len(steps)][d_model],
    kl [S][len(steps)]."""
    out = compress(inp, cfg)
    cu = inp["cu_seqlens"].numpy()
    steps = list(range(cfg.T_dec)) if steps is None else list(steps)
    G = cfg.G
    x_comp = decode_steps(out["cache"], inp["Kd"], inp["Vd"], inp["Qd"], G, steps)
    x_full = decode_steps(full_view(inp["K"], inp["V"], cu), inp["Kd"], inp["Vd"], inp["Qd"], G, steps)
    n = x_full.shape[0] * x_full.shape[1]
    out["steps"], out["x_comp"], out["x_full"] = steps, x_comp, x_full
    out["kl"] = kl_rows(x_full.reshape(n, -1), x_comp.reshape(n, -1), inp["W"]).reshape(x_full.shape[:2])
    return out
