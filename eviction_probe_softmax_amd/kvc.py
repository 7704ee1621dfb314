"""Python binding of libkvc (ctypes).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory and the current HIP stream. Importing
this module loads libkvc.so from the package directory and raises if it is
missing; there is no fallback implementation.

Function names follow the C ABI (include/kvc.h): score, propagate, partition,
build_trees, auction, pack, full_view, decode_attn, kl, rope_table.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libkvc.so not found at {LIB_PATH}: run eviction_probe_softmax_amd.build_lib "
                      "(or __graft_entry__.build()) first")
_lib = C.CDLL(LIB_PATH)

KVC_F32, KVC_BF16 = 0, 1
STAGE_SCORE, STAGE_PROPAGATE, STAGE_PARTITION, STAGE_TREES, STAGE_AUCTION, STAGE_PACK = range(6)

EXPORTS = ["kvc_strerror", "kvc_last_error", "kvc_params_default", "kvc_budgets", "kvc_pack_capacity",
           "kvc_slot_stride", "kvc_workspace_size", "kvc_rope_table", "kvc_score", "kvc_propagate",
           "kvc_partition", "kvc_partition_ex", "kvc_build_trees", "kvc_build_trees_ex", "kvc_auction", "kvc_hybrid_units", "kvc_pack", "kvc_full_view",
           "kvc_decode_workspace", "kvc_decode_plan", "kvc_decode_attn", "kvc_decode_attn_planned",
           "kvc_decode_static_limit", "kvc_decode_attn_static",
           "kvc_kl_workspace", "kvc_kl", "kvc_step_capacity",
           "kvc_step_workspace", "kvc_step_init", "kvc_step_append", "kvc_step_prune",
           "kvc_propagate_dense_workspace", "kvc_propagate_dense", "kvc_propagate_ar_workspace",
           "kvc_propagate_ar"]


class Shape(C.Structure):
    _fields_ = [("n_seq", C.c_int32), ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32),
                ("group", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32),
                ("total_tokens", C.c_int64), ("cu_seqlens", C.POINTER(C.c_int64)),
                ("cu_seqlens_d", C.c_void_p)]


class Params(C.Structure):
    _fields_ = [("budget_ratio", C.c_float), ("budget_min", C.c_int32), ("prompt_exact", C.c_int32),
                ("recent_exact", C.c_int32), ("suffix_exact", C.c_int32), ("n_probe", C.c_int32),
                ("n_hops", C.c_int32), ("n_seeds", C.c_int32), ("hop_weight", C.c_float),
                ("n_dprobe", C.c_int32), ("w_attn", C.c_float), ("w_value", C.c_float),
                ("value_base", C.c_float), ("floor_frac", C.c_float), ("token_mode", C.c_int32),
                ("slot_len", C.c_int32), ("slot_min", C.c_int32), ("slot_max", C.c_int32),
                ("slot_target", C.c_int32), ("lambda_len", C.c_float), ("lambda_curv", C.c_float),
                ("rope_base", C.c_float), ("hybrid_frac", C.c_float), ("window", C.c_int32),
                ("n_depth", C.c_int32), ("lambda_surp", C.c_float), ("split_mode", C.c_int32)]


class Trees(C.Structure):
    _fields_ = [("node_rel", C.c_void_p), ("node_D", C.c_void_p), ("node_mu", C.c_void_p),
                ("op_util", C.c_void_p), ("op_cost", C.c_void_p), ("node_topo", C.c_void_p)]


class Policy(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w1", "b1", "g1", "be1", "w2", "b2", "g2", "be2", "w3", "b3")]


class Student(C.Structure):
    _fields_ = [("K", C.c_void_p), ("V", C.c_void_p), ("pos", C.c_void_p), ("Qwin", C.c_void_p),
                ("seg_off", C.c_void_p), ("seg_len", C.c_void_p), ("seq_off", C.POINTER(C.c_int64)),
                ("seq_cap", C.POINTER(C.c_int32)), ("seq_len", C.POINTER(C.c_int32)), ("cap_total", C.c_int64)]


class Ragged(C.Structure):
    _fields_ = [("K", C.c_void_p), ("V", C.c_void_p), ("lnmu", C.c_void_p), ("pos", C.c_void_p),
                ("seg_off", C.c_void_p), ("seg_len", C.c_void_p), ("n_seq", C.c_int32),
                ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("dtype", C.c_int32), ("max_seg", C.c_int32), ("capacity", C.c_int64)]


_P = C.c_void_p
_sig = {
    "kvc_strerror": (C.c_char_p, [C.c_int]),
    "kvc_last_error": (C.c_char_p, []),
    "kvc_params_default": (None, [C.POINTER(Params)]),
    "kvc_budgets": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P]),
    "kvc_pack_capacity": (C.c_int64, [C.POINTER(Shape), C.POINTER(Params)]),
    "kvc_slot_stride": (C.c_int32, [C.POINTER(Shape), C.POINTER(Params)]),
    "kvc_workspace_size": (C.c_size_t, [C.POINTER(Shape), C.POINTER(Params), C.c_int32]),
    "kvc_rope_table": (C.c_int, [C.c_float, C.c_int32, C.c_int32, _P, _P, _P]),
    "kvc_score": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                            C.c_size_t, _P]),
    "kvc_propagate": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "kvc_partition": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, C.c_int32, C.c_int32, _P, _P, _P,
                                _P, _P, C.c_size_t, _P]),
    "kvc_partition_ex": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, C.c_int32, _P, C.c_int32, _P, _P, _P,
                                   _P, _P, C.c_size_t, _P]),
    "kvc_build_trees": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  _P, C.POINTER(Trees), _P, C.c_size_t, _P]),
    "kvc_build_trees_ex": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _P, C.POINTER(Trees), _P, C.c_size_t, _P]),
    "kvc_auction": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), C.POINTER(Trees), _P, _P, _P, _P, _P,
                              _P, _P, _P, C.c_size_t, _P]),
    "kvc_pack": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, C.POINTER(Trees), _P, _P, _P,
                           _P, _P, C.POINTER(Ragged), _P, C.c_size_t, _P]),
    "kvc_hybrid_units": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P]),
    "kvc_propagate_dense_workspace": (C.c_size_t, [C.POINTER(Shape), C.POINTER(Params)]),
    "kvc_propagate_dense": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "kvc_propagate_ar_workspace": (C.c_size_t, [C.POINTER(Shape), C.POINTER(Params)]),
    "kvc_propagate_ar": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "kvc_full_view": (C.c_int, [C.POINTER(Shape), _P, _P, _P]),
    "kvc_decode_workspace": (C.c_size_t, [C.POINTER(Ragged), C.c_int32, C.c_int32]),
    "kvc_decode_attn": (C.c_int, [C.POINTER(Ragged), _P, _P, C.c_int32, C.c_int32, _P, C.c_int32, _P,
                                  C.c_int64, _P, _P, C.c_size_t, _P]),
    "kvc_decode_attn_planned": (C.c_int, [C.POINTER(Ragged), _P, _P, C.c_int32, C.c_int32, _P, C.c_int32, _P,
                                  C.c_int64, _P, _P, C.c_size_t, _P]),
    "kvc_decode_plan": (C.c_int, [C.POINTER(Ragged), C.c_int32, C.c_int32, _P, C.c_size_t, _P]),
    "kvc_decode_static_limit": (C.c_size_t, []),
    "kvc_decode_attn_static": (C.c_int, [C.POINTER(Ragged), _P, _P, C.c_int32, C.c_int32, _P, C.c_int32, _P,
                                         C.c_int64, _P, _P]),
    "kvc_step_capacity": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), C.c_int32, _P]),
    "kvc_step_workspace": (C.c_size_t, [C.POINTER(Shape), C.POINTER(Params), C.c_int64]),
    "kvc_step_init": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), _P, _P, _P, C.POINTER(Policy),
                                C.POINTER(Student), _P, _P, _P, C.c_size_t, _P]),
    "kvc_step_append": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), C.POINTER(Student), _P, _P, _P, C.c_int32,
                                  C.c_int32, _P]),
    "kvc_step_prune": (C.c_int, [C.POINTER(Shape), C.POINTER(Params), C.POINTER(Student), C.c_int32,
                                 C.POINTER(Policy), _P, _P, _P, C.c_size_t, _P]),
    "kvc_kl_workspace": (C.c_size_t, [C.c_int64, C.c_int32, C.c_int32, C.c_int32]),
    "kvc_kl": (C.c_int, [C.c_int64, C.c_int32, C.c_int32, _P, _P, _P, C.c_int32, _P, _P, C.c_size_t, _P]),
}
# measurement helpers (include/kvc_peaks.h)
PEAK_EXPORTS = ["kvc_peak_read", "kvc_peak_mfma", "kvc_peak_exp"]
_sig["kvc_peak_read"] = (C.c_int, [_P, C.c_size_t, C.c_int32, _P, _P])
_sig["kvc_peak_mfma"] = (C.c_int, [C.c_int32, C.c_int32, _P, _P])
_sig["kvc_peak_exp"] = (C.c_int, [C.c_int32, C.c_int32, _P, _P])
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class KvcError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.kvc_last_error().decode()
        super().__init__(f"{fn} failed: {_lib.kvc_strerror(status).decode()} ({status}): {msg}")
        self.status = status


def _check(fn, st):
    if st != 0:
        raise KvcError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_contiguous(), "tensors passed to libkvc must be contiguous"
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


_DT = {torch.bfloat16: KVC_BF16, torch.float32: KVC_F32}


@dataclass
class Problem:
    """Shape + parameters of one compression call, with device offsets."""
    shape: Shape
    params: Params
    cu_host: object
    cu_dev: torch.Tensor
    device: torch.device

    @property
    def S(self):
        return self.shape.n_seq

    @property
    def Ly(self):
        return self.shape.n_layers

    @property
    def H(self):
        return self.shape.n_kv_heads

    @property
    def T(self):
        return self.shape.total_tokens

    def budgets(self):
        S = self.S
        B = (C.c_int64 * S)()
        A = (C.c_int64 * S)()
        F = (C.c_int64 * S)()
        st = _lib.kvc_budgets(C.byref(self.shape), C.byref(self.params), B, A, F)
        _check("kvc_budgets", st)
        return list(B), list(A), list(F)

    def pack_capacity(self):
        return int(_lib.kvc_pack_capacity(C.byref(self.shape), C.byref(self.params)))

    def slot_stride(self):
        return int(_lib.kvc_slot_stride(C.byref(self.shape), C.byref(self.params)))

    def ws(self, stage):
        n = int(_lib.kvc_workspace_size(C.byref(self.shape), C.byref(self.params), stage))
        return torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)


def make_problem(cfg, cu_seqlens: torch.Tensor, dtype: torch.dtype, device="cuda") -> Problem:
    """cfg: any object with the workload fields (workload.Config works)."""
    dev = torch.device(device)
    cu = cu_seqlens.to(torch.int64).cpu().contiguous()
    cu_host = (C.c_int64 * len(cu))(*cu.tolist())
    cu_dev = cu.to(dev)
    sh = Shape(n_seq=len(cu) - 1, n_layers=cfg.Ly, n_kv_heads=cfg.H, group=cfg.G, head_dim=cfg.d,
               dtype=_DT[dtype], total_tokens=int(cu[-1]), cu_seqlens=C.cast(cu_host, C.POINTER(C.c_int64)),
               cu_seqlens_d=C.c_void_p(cu_dev.data_ptr()))
    p = Params()
    _lib.kvc_params_default(C.byref(p))
    p.budget_ratio = cfg.budget_ratio
    p.budget_min = cfg.budget_min
    p.prompt_exact, p.recent_exact, p.suffix_exact = cfg.prompt_exact, cfg.recent_exact, cfg.suffix_exact
    p.n_probe = cfg.P
    p.n_hops, p.n_seeds, p.hop_weight = cfg.n_hops, cfg.n_seeds, cfg.hop_weight
    p.n_dprobe, p.w_attn, p.w_value, p.value_base = cfg.n_dprobe, cfg.w_attn, cfg.w_value, cfg.value_base
    p.floor_frac = cfg.floor_frac
    p.token_mode = 1 if cfg.token_mode else 0
    p.slot_len, p.slot_min, p.slot_max, p.slot_target = cfg.slot_len, cfg.slot_min, cfg.slot_max, cfg.slot_target
    p.lambda_len, p.lambda_curv = cfg.lambda_len, cfg.lambda_curv
    p.rope_base = cfg.rope_base
    p.hybrid_frac = getattr(cfg, "hybrid_frac", 0.0)
    p.window = getattr(cfg, "window", 64)
    p.n_depth = getattr(cfg, "n_depth", 1)
    p.lambda_surp = getattr(cfg, "lambda_surp", 1.0)
    p.split_mode = getattr(cfg, "split_mode", 0)
    return Problem(sh, p, cu_host, cu_dev, dev)


# ------------------------------------------------------------------ entry points
def rope_table(base: float, head_dim: int, n_pos: int, device="cuda"):
    cs = torch.empty((n_pos, head_dim // 2), dtype=torch.float32, device=device)
    sn = torch.empty_like(cs)
    _check("kvc_rope_table", _lib.kvc_rope_table(base, head_dim, n_pos, _ptr(cs), _ptr(sn), _stream()))
    return cs, sn


def score(pb: Problem, K, V, Qp, feats=True):
    dev = pb.device
    E = pb.Ly * pb.H * pb.T
    R = pb.shape.group * pb.params.n_probe
    rel0 = torch.empty((pb.Ly, pb.H, pb.T), dtype=torch.float32, device=dev)
    ft = torch.empty((5, pb.Ly, pb.H, pb.T), dtype=torch.float32, device=dev) if feats else None
    lse = torch.empty((pb.S, pb.Ly, pb.H * pb.shape.group, pb.params.n_probe), dtype=torch.float32, device=dev)
    ent = torch.empty_like(lse)
    sens = torch.empty((pb.S, pb.Ly, pb.H), dtype=torch.float32, device=dev)
    ws = pb.ws(STAGE_SCORE)
    st = _lib.kvc_score(C.byref(pb.shape), C.byref(pb.params), _ptr(K), _ptr(V), _ptr(Qp), _ptr(rel0), _ptr(ft),
                        _ptr(lse), _ptr(ent), _ptr(sens), _ptr(ws), ws.numel(), _stream())
    _check("kvc_score", st)
    del E, R
    return {"r0": rel0, "feats": ft, "lse": lse, "ent": ent, "head_sens": sens}


def propagate(pb: Problem, K, Qctx, rel0, want_seeds=True):
    dev = pb.device
    rel = torch.empty_like(rel0)
    seeds = None
    if want_seeds and pb.params.n_hops > 0:
        seeds = torch.empty((pb.params.n_hops, pb.S, pb.Ly, pb.H, pb.params.n_seeds), dtype=torch.int32,
                            device=dev)
    ws = pb.ws(STAGE_PROPAGATE)
    st = _lib.kvc_propagate(C.byref(pb.shape), C.byref(pb.params), _ptr(K), _ptr(Qctx), _ptr(rel0), _ptr(rel),
                            _ptr(seeds), _ptr(ws), ws.numel(), _stream())
    _check("kvc_propagate", st)
    return {"rel": rel, "seeds": seeds}


def partition(pb: Problem, hidden=None, hidden_dim=0, cost_q=None, cut_q=None, inject=False, export=False,
              surprisal=None):
    dev = pb.device
    stride = pb.slot_stride()
    slot_start = torch.empty((pb.S, stride + 1), dtype=torch.int32, device=dev)
    n_slots = torch.empty((pb.S,), dtype=torch.int32, device=dev)
    nmin, nmax = pb.params.slot_min, pb.params.slot_max
    if export and cost_q is None:
        cost_q = torch.zeros((pb.T, nmax - nmin + 1), dtype=torch.int64, device=dev)
        cut_q = torch.zeros((pb.T,), dtype=torch.int64, device=dev)
    ws = pb.ws(STAGE_PARTITION)
    st = _lib.kvc_partition_ex(C.byref(pb.shape), C.byref(pb.params), _ptr(hidden), hidden_dim, _ptr(surprisal),
                               1 if inject else 0, _ptr(cost_q), _ptr(cut_q), _ptr(slot_start), _ptr(n_slots),
                               _ptr(ws), ws.numel(), _stream())
    _check("kvc_partition", st)
    return {"slot_start": slot_start, "n_slots": n_slots, "dp_cost_q": cost_q, "dp_cut_q": cut_q}


def empty_trees(pb: Problem):
    dev = pb.device
    n = (pb.Ly, pb.H, 2 * pb.T)
    return {"node_rel": torch.zeros(n, dtype=torch.float32, device=dev),
            "node_D": torch.zeros(n, dtype=torch.float32, device=dev),
            "node_mu": torch.zeros(n, dtype=torch.float32, device=dev),
            "op_util": torch.zeros(n, dtype=torch.float32, device=dev),
            "op_cost": torch.zeros(n, dtype=torch.uint8, device=dev),
            "node_topo": (torch.full(n, -1, dtype=torch.int32, device=dev) if pb.params.split_mode else None)}


def _trees_struct(tr):
    if tr is None:
        return None
    return Trees(node_rel=_ptr(tr["node_rel"]), node_D=_ptr(tr["node_D"]), node_mu=_ptr(tr["node_mu"]),
                 op_util=_ptr(tr["op_util"]), op_cost=_ptr(tr["op_cost"]), node_topo=_ptr(tr.get("node_topo")))


def build_trees(pb: Problem, K, V, Qp, lse, rel, head_sens, rope_cos, rope_sin, slot_start, n_slots, out=None,
                cut_q=None):
    """kvc_build_trees_ex. cut_q: the partition's int64 [T] cut scores (DP
    slots) or None; node_topo (int32 view of the uint32 records) is allocated
    when split_mode is 1."""
    tr = out if out is not None else empty_trees(pb)
    ts = _trees_struct(tr)
    ws = pb.ws(STAGE_TREES)
    st = _lib.kvc_build_trees_ex(C.byref(pb.shape), C.byref(pb.params), _ptr(K), _ptr(V), _ptr(Qp), _ptr(lse),
                                 _ptr(rel), _ptr(head_sens), _ptr(rope_cos), _ptr(rope_sin), _ptr(slot_start),
                                 _ptr(n_slots), _ptr(cut_q), C.byref(ts), _ptr(ws), ws.numel(), _stream())
    _check("kvc_build_trees_ex", st)
    return tr


def auction(pb: Problem, trees=None, rel=None, head_sens=None, slot_start=None, n_slots=None):
    dev = pb.device
    if pb.params.token_mode:
        taken = torch.empty((pb.Ly, pb.H, pb.T), dtype=torch.uint8, device=dev)
    else:
        taken = torch.empty((pb.Ly, pb.H, 2 * pb.T), dtype=torch.uint8, device=dev)
    spent = torch.empty((pb.S,), dtype=torch.int64, device=dev)
    spent_floor = torch.empty((pb.S,), dtype=torch.int64, device=dev)
    ts = _trees_struct(trees)
    ws = pb.ws(STAGE_AUCTION)
    st = _lib.kvc_auction(C.byref(pb.shape), C.byref(pb.params), C.byref(ts) if ts is not None else None,
                          _ptr(rel), _ptr(head_sens), _ptr(slot_start), _ptr(n_slots), _ptr(taken), _ptr(spent),
                          _ptr(spent_floor), _ptr(ws), ws.numel(), _stream())
    _check("kvc_auction", st)
    return {"taken": taken, "spent": spent, "spent_floor": spent_floor}


def propagate_dense(pb: Problem, K, Qctx, rel0):
    """Dense rollout: every token a seed in every hop. Returns rel [Ly][H][T]."""
    rel = torch.empty_like(rel0)
    n = int(_lib.kvc_propagate_dense_workspace(C.byref(pb.shape), C.byref(pb.params)))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=pb.device)
    st = _lib.kvc_propagate_dense(C.byref(pb.shape), C.byref(pb.params), _ptr(K), _ptr(Qctx), _ptr(rel0),
                                  _ptr(rel), _ptr(ws), ws.numel(), _stream())
    _check("kvc_propagate_dense", st)
    return {"rel": rel}


def propagate_ar(pb: Problem, K, Qctx, rel0):
    """The "A r" direction over every token. Returns rel [Ly][H][T]."""
    rel = torch.empty_like(rel0)
    n = int(_lib.kvc_propagate_ar_workspace(C.byref(pb.shape), C.byref(pb.params)))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=pb.device)
    st = _lib.kvc_propagate_ar(C.byref(pb.shape), C.byref(pb.params), _ptr(K), _ptr(Qctx), _ptr(rel0), _ptr(rel),
                               _ptr(ws), ws.numel(), _stream())
    _check("kvc_propagate_ar", st)
    return {"rel": rel}


def hybrid_units(pb: Problem, head_sens):
    """Units kept whole by the head-level hybrid: uint8 [S][Ly][H]."""
    full = torch.empty((pb.S, pb.Ly, pb.H), dtype=torch.uint8, device=pb.device)
    st = _lib.kvc_hybrid_units(C.byref(pb.shape), C.byref(pb.params), _ptr(head_sens), _ptr(full), _stream())
    _check("kvc_hybrid_units", st)
    return full


def _ragged_struct(c):
    return Ragged(K=_ptr(c["K"]), V=_ptr(c["V"]), lnmu=_ptr(c.get("lnmu")), pos=_ptr(c.get("pos")),
                  seg_off=_ptr(c["seg_off"]), seg_len=_ptr(c["seg_len"]), n_seq=c["n_seq"],
                  n_layers=c["n_layers"], n_kv_heads=c["n_kv_heads"], head_dim=c["head_dim"],
                  dtype=_DT[c["K"].dtype], max_seg=c["max_seg"], capacity=c["K"].shape[0])


def pack(pb: Problem, K, V, rel, trees, taken, slot_start, n_slots, rope_cos, rope_sin, capacity=None):
    dev = pb.device
    cap = pb.pack_capacity() if capacity is None else capacity
    d = pb.shape.head_dim
    L = [pb.cu_host[i + 1] - pb.cu_host[i] for i in range(pb.S)]
    c = {"K": torch.empty((max(cap, 1), d), dtype=K.dtype, device=dev),
         "V": torch.empty((max(cap, 1), d), dtype=K.dtype, device=dev),
         "lnmu": torch.empty((max(cap, 1),), dtype=torch.float32, device=dev),
         "pos": torch.empty((max(cap, 1),), dtype=torch.int32, device=dev),
         "seg_off": torch.empty((pb.S, pb.Ly, pb.H), dtype=torch.int64, device=dev),
         "seg_len": torch.empty((pb.S, pb.Ly, pb.H), dtype=torch.int32, device=dev),
         "n_seq": pb.S, "n_layers": pb.Ly, "n_kv_heads": pb.H, "head_dim": d, "max_seg": int(max(L))}
    rs = _ragged_struct(c)
    rs.capacity = cap
    ts = _trees_struct(trees)
    ws = pb.ws(STAGE_PACK)
    st = _lib.kvc_pack(C.byref(pb.shape), C.byref(pb.params), _ptr(K), _ptr(V), _ptr(rel),
                       C.byref(ts) if ts is not None else None, _ptr(taken), _ptr(slot_start), _ptr(n_slots),
                       _ptr(rope_cos), _ptr(rope_sin), C.byref(rs), _ptr(ws), ws.numel(), _stream())
    _check("kvc_pack", st)
    return c


def full_view(pb: Problem, K, V):
    dev = pb.device
    seg_off = torch.empty((pb.S, pb.Ly, pb.H), dtype=torch.int64, device=dev)
    seg_len = torch.empty((pb.S, pb.Ly, pb.H), dtype=torch.int32, device=dev)
    _check("kvc_full_view", _lib.kvc_full_view(C.byref(pb.shape), _ptr(seg_off), _ptr(seg_len), _stream()))
    L = [pb.cu_host[i + 1] - pb.cu_host[i] for i in range(pb.S)]
    d = pb.shape.head_dim
    return {"K": K.reshape(-1, d), "V": V.reshape(-1, d), "lnmu": None, "pos": None, "seg_off": seg_off,
            "seg_len": seg_len, "n_seq": pb.S, "n_layers": pb.Ly, "n_kv_heads": pb.H, "head_dim": d,
            "max_seg": int(max(L))}


class Decoder:
    """Holds the marshalled cache description, a reusable workspace and the
    cache's decode plan (kvc_decode_plan, made here on the current stream)
    for repeated decode steps over one cache. Call plan() again after the
    cache's segments change."""

    def __init__(self, cache, group: int, t_cap: int):
        self.cache = cache
        self.rs = _ragged_struct(cache)
        self.group = group
        self.t_cap = t_cap
        n = int(_lib.kvc_decode_workspace(C.byref(self.rs), group, t_cap))
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=cache["K"].device)
        self.plan()

    def plan(self):
        st = _lib.kvc_decode_plan(C.byref(self.rs), self.group, self.t_cap, _ptr(self.ws), self.ws.numel(),
                                  _stream())
        _check("kvc_decode_plan", st)

    def step(self, K_tail, V_tail, t_valid, Q, x_out, x_stride, o_out=None):
        st = _lib.kvc_decode_attn_planned(C.byref(self.rs), _ptr(K_tail), _ptr(V_tail), t_valid, self.t_cap, _ptr(Q),
                                          self.group, _ptr(x_out), x_stride, _ptr(o_out), _ptr(self.ws),
                                          self.ws.numel(), _stream())
        _check("kvc_decode_attn_planned", st)


def decode_attn(cache, K_tail, V_tail, t_valid, t_cap, Q, group, x_out, x_stride, o_out=None):
    """One step through the single-call entry point (plan and step together)."""
    rs = _ragged_struct(cache)
    n = int(_lib.kvc_decode_workspace(C.byref(rs), group, t_cap))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=cache["K"].device)
    st = _lib.kvc_decode_attn(C.byref(rs), _ptr(K_tail), _ptr(V_tail), t_valid, t_cap, _ptr(Q), group, _ptr(x_out),
                              x_stride, _ptr(o_out), _ptr(ws), ws.numel(), _stream())
    _check("kvc_decode_attn", st)


def decode_static_limit() -> int:
    """Bytes of the per-GPU scratch array behind decode_attn_static."""
    return int(_lib.kvc_decode_static_limit())


def decode_attn_static(cache, K_tail, V_tail, t_valid, t_cap, Q, group, x_out, x_stride, o_out=None):
    """One step through the entry point that allocates nothing (its workspace
    is the library's per-GPU scratch array; calls on one GPU must not overlap)."""
    rs = _ragged_struct(cache)
    st = _lib.kvc_decode_attn_static(C.byref(rs), _ptr(K_tail), _ptr(V_tail), t_valid, t_cap, _ptr(Q), group,
                                     _ptr(x_out), x_stride, _ptr(o_out), _stream())
    _check("kvc_decode_attn_static", st)


class KL:
    def __init__(self, n_pairs, d_model, vocab, w_dtype, device="cuda"):
        self.n_pairs, self.d_model, self.vocab, self.w_dtype = n_pairs, d_model, vocab, _DT[w_dtype]
        n = int(_lib.kvc_kl_workspace(n_pairs, d_model, vocab, self.w_dtype))
        self.ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)

    def __call__(self, x_full, x_comp, W, out=None):
        out = torch.empty((self.n_pairs,), dtype=torch.float32, device=x_full.device) if out is None else out
        st = _lib.kvc_kl(self.n_pairs, self.d_model, self.vocab, _ptr(x_full), _ptr(x_comp), _ptr(W), self.w_dtype,
                         _ptr(out), _ptr(self.ws), self.ws.numel(), _stream())
        _check("kvc_kl", st)
        return out


def kl(x_full, x_comp, W):
    n, dm = x_full.shape
    return KL(n, dm, W.shape[0], W.dtype, device=x_full.device)(x_full, x_comp, W)


class Stepwise:
    """Step-wise eviction (kvc_step_*): a student cache with one slot region
    per sequence, sized for t_steps decode steps, and its window of recent
    queries. ``policy`` holds the scoring MLP's fp32 tensors on the device."""

    def __init__(self, pb: Problem, policy, t_steps: int, dtype, group: int):
        S, Ly, H, d = pb.S, pb.Ly, pb.H, pb.shape.head_dim
        dev = pb.device
        self.pb, self.t_steps, self.group = pb, t_steps, group
        caps = (C.c_int32 * S)()
        _check("kvc_step_capacity", _lib.kvc_step_capacity(C.byref(pb.shape), C.byref(pb.params), t_steps, caps))
        self.caps = [int(c) for c in caps]
        offs = [0]
        for c in self.caps[:-1]:
            offs.append(offs[-1] + c)
        self.cap_total = sum(self.caps)
        self._off = (C.c_int64 * S)(*offs)
        self._cap = (C.c_int32 * S)(*self.caps)
        self._len = (C.c_int32 * S)()
        self.K = torch.empty((Ly, H, self.cap_total, d), dtype=dtype, device=dev)
        self.V = torch.empty_like(self.K)
        self.pos = torch.zeros((self.cap_total,), dtype=torch.int32, device=dev)
        self.Qwin = torch.empty((S, Ly, H * group, pb.params.window, d), dtype=dtype, device=dev)
        self.seg_off = torch.empty((S, Ly, H), dtype=torch.int64, device=dev)
        self.seg_len = torch.empty((S, Ly, H), dtype=torch.int32, device=dev)
        self.st = Student(K=_ptr(self.K), V=_ptr(self.V), pos=_ptr(self.pos), Qwin=_ptr(self.Qwin),
                          seg_off=_ptr(self.seg_off), seg_len=_ptr(self.seg_len), seq_off=self._off,
                          seq_cap=self._cap, seq_len=self._len, cap_total=self.cap_total)
        self._pol_t = policy
        self.pol = Policy(**{k: _ptr(policy[k]) for k in ("w1", "b1", "g1", "be1", "w2", "b2", "g2", "be2",
                                                         "w3", "b3")})
        n = int(_lib.kvc_step_workspace(C.byref(pb.shape), C.byref(pb.params), self.cap_total))
        if n == 0:
            raise KvcError("kvc_step_workspace", -1)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.decoder = None

    @property
    def lengths(self):
        return [int(x) for x in self._len]

    def init(self, K, V, Qctx, feats=None, scores=None):
        st = _lib.kvc_step_init(C.byref(self.pb.shape), C.byref(self.pb.params), _ptr(K), _ptr(V), _ptr(Qctx),
                                C.byref(self.pol), C.byref(self.st), _ptr(feats), _ptr(scores), _ptr(self.ws),
                                self.ws.numel(), _stream())
        _check("kvc_step_init", st)

    def append(self, K_tail, V_tail, Q_t, t):
        st = _lib.kvc_step_append(C.byref(self.pb.shape), C.byref(self.pb.params), C.byref(self.st), _ptr(K_tail),
                                  _ptr(V_tail), _ptr(Q_t), t, self.t_steps, _stream())
        _check("kvc_step_append", st)

    def prune(self, t, feats=None, scores=None):
        st = _lib.kvc_step_prune(C.byref(self.pb.shape), C.byref(self.pb.params), C.byref(self.st), t,
                                 C.byref(self.pol), _ptr(feats), _ptr(scores), _ptr(self.ws), self.ws.numel(),
                                 _stream())
        _check("kvc_step_prune", st)

    def view(self):
        """The occupied slots as a ragged cache for kvc_decode_attn (no tail)."""
        d = self.pb.shape.head_dim
        return {"K": self.K.reshape(-1, d), "V": self.V.reshape(-1, d), "lnmu": None, "pos": self.pos,
                "seg_off": self.seg_off, "seg_len": self.seg_len, "n_seq": self.pb.S, "n_layers": self.pb.Ly,
                "n_kv_heads": self.pb.H, "head_dim": d, "max_seg": int(max(self.caps))}

    def decode(self, K_tail, V_tail, Q_t, x_out, x_stride):
        """Attention of Q_t over the occupied slots (the appended token included)."""
        if self.decoder is None:
            self.decoder = Decoder(self.view(), self.group, self.t_steps)
        else:
            self.decoder.plan()  # the student's segments change every step
        self.decoder.step(K_tail, V_tail, 0, Q_t, x_out, x_stride)


def _time_ms(launch, reps):
    launch()
    launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def peak_read_gbs(nbytes=2 << 30, grid=16384, reps=10):
    """Measured HBM read ceiling (kvc_peak_read over nbytes of device memory), GB/s."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def launch():
        _check("kvc_peak_read", _lib.kvc_peak_read(_ptr(buf), nbytes, grid, _ptr(sink), _stream()))
    ms = _time_ms(launch, reps)
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def peak_exp_gelems(grid=2048, iters=2048, reps=5):
    """Measured exponential-mix ceiling (kvc_peak_exp): elements (one exp2 and
    three VALU operations each) per second, in G/s."""
    sink = torch.zeros(grid, dtype=torch.float32, device="cuda")

    def launch():
        _check("kvc_peak_exp", _lib.kvc_peak_exp(grid, iters, _ptr(sink), _stream()))
    ms = _time_ms(launch, reps)
    return grid * 256 * iters * 8 / (ms * 1e-3) / 1e9


def peak_mfma_tflops(grid=2048, iters=4096, reps=5):
    """Measured dense bf16 MFMA ceiling (kvc_peak_mfma), TFLOP/s."""
    sink = torch.zeros(grid, dtype=torch.float32, device="cuda")

    def launch():
        _check("kvc_peak_mfma", _lib.kvc_peak_mfma(grid, iters, _ptr(sink), _stream()))
    ms = _time_ms(launch, reps)
    return grid * 4 * iters * 131072 / (ms * 1e-3) / 1e12
