"""The whole path as a sequence of libkvc calls on one stream.

Orchestration only: every step below is a C-ABI call into the HIP library;
this module allocates outputs (via the binding) and passes tensors along.
Order follows the GraceKV page ('Method': partition -> represent -> value ->
allocate -> pack) and the DistillCache paper (decode over the pruned cache,
per-step KL against the full cache).
"""
from __future__ import annotations

from typing import Dict, Optional

import torch

from . import kvc


class Compressor:
    """Holds the problem description, RoPE tables and reusable buffers for
    repeated compression of inputs with one shape."""

    def __init__(self, cfg, cu_seqlens: torch.Tensor, dtype: torch.dtype, device="cuda"):
        self.cfg = cfg
        self.pb = kvc.make_problem(cfg, cu_seqlens, dtype, device)
        self.device = torch.device(device)
        lens = [int(cu_seqlens[i + 1] - cu_seqlens[i]) for i in range(len(cu_seqlens) - 1)]
        self.max_len = max(lens)
        self.rope_cos = self.rope_sin = None
        if not cfg.token_mode:
            self.rope_cos, self.rope_sin = kvc.rope_table(cfg.rope_base, cfg.d, self.max_len, device=device)

    def compress(self, inp: Dict[str, torch.Tensor], stop_after: Optional[str] = None) -> Dict[str, object]:
        pb, cfg = self.pb, self.cfg
        out: Dict[str, object] = {}
        sc = kvc.score(pb, inp["K"], inp["V"], inp["Qp"])
        out.update(sc)
        pr = kvc.propagate(pb, inp["K"], inp["Qctx"], sc["r0"])
        out.update(pr)
        rel = pr["rel"]
        if stop_after == "propagate":
            return out
        if cfg.token_mode:
            au = kvc.auction(pb, rel=rel, head_sens=sc["head_sens"])
            out.update(au)
            out["cache"] = kvc.pack(pb, inp["K"], inp["V"], rel, None, au["taken"], None, None, None, None)
            return out
        split = getattr(cfg, "split_mode", 0) == 1
        if cfg.slot_len > 0:
            part = kvc.partition(pb)
        else:   # curvature-candidate splits read the partition's cut scores
            part = kvc.partition(pb, inp["hidden"], cfg.hidden_dim, surprisal=inp.get("surprisal"), export=split)
        out.update(part)
        tr = kvc.build_trees(pb, inp["K"], inp["V"], inp["Qp"], sc["lse"], rel, sc["head_sens"], self.rope_cos,
                             self.rope_sin, part["slot_start"], part["n_slots"],
                             cut_q=part["dp_cut_q"] if split else None)
        out["trees"] = tr
        au = kvc.auction(pb, tr, rel, sc["head_sens"], part["slot_start"], part["n_slots"])
        out.update(au)
        out["cache"] = kvc.pack(pb, inp["K"], inp["V"], rel, tr, au["taken"], part["slot_start"],
                                part["n_slots"], self.rope_cos, self.rope_sin)
        return out


def decode_both(comp_cache, full_cache, inp, cfg, x_full=None, x_comp=None):
    """All decode steps over both caches. Returns x_full, x_comp
    [S][T_dec][d_model] fp32."""
    S, Td, Dm = cfg.S, cfg.T_dec, cfg.d_model
    dev = inp["K"].device
    x_full = torch.empty((S, Td, Dm), dtype=torch.float32, device=dev) if x_full is None else x_full
    x_comp = torch.empty((S, Td, Dm), dtype=torch.float32, device=dev) if x_comp is None else x_comp
    df = kvc.Decoder(full_cache, cfg.G, Td)
    dc = kvc.Decoder(comp_cache, cfg.G, Td)
    for t in range(Td):
        q = inp["Qd"][t]
        # row (s, t) lives at x[s, t]: base pointer of x[0, t], stride T_dec * d_model
        df.step(inp["Kd"], inp["Vd"], t + 1, q, _row_view(x_full, t), Td * Dm)
        dc.step(inp["Kd"], inp["Vd"], t + 1, q, _row_view(x_comp, t), Td * Dm)
    return x_full, x_comp


class _RowView:
    """A strided output target: data_ptr of x[0, t] with the caller's stride."""

    def __init__(self, x, t):
        self._ptr = x[0, t].data_ptr()

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self._ptr


def _row_view(x, t):
    return _RowView(x, t)


def run_stepwise(cfg, inp, policy, record=None, kept_trace=None):
    """Step-wise eviction over the decode steps (DistillCache paper,
    Algorithm 1): prune the prefill cache once, then per step append the new
    pair, decode over the student, prune; the full cache is decoded beside it
    and the per-step KL compares the two. ``record`` (a list) receives HIP
    event pairs (init, per-step prune) on the library's stream;
    ``kept_trace`` (a list) receives (step, kept positions per sequence)
    after every prune (step -1: the prefill prune; this synchronizes)."""
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    sw = kvc.Stepwise(pb, policy, cfg.T_dec, inp["K"].dtype, cfg.G)
    stream = torch.cuda.current_stream()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    e0 = ev() if record is not None else None
    sw.init(inp["K"], inp["V"], inp["Qctx"])
    if record is not None:
        record.append(("init", e0, ev()))

    def trace_kept(step):
        pos = sw.pos.cpu()
        kept, off = [], 0
        for s in range(cfg.S):
            kept.append(pos[off:off + sw.lengths[s]].numpy().copy())
            off += sw.caps[s]
        kept_trace.append((step, kept))

    if kept_trace is not None:
        trace_kept(-1)
    full = kvc.full_view(pb, inp["K"], inp["V"])
    dfull = kvc.Decoder(full, cfg.G, cfg.T_dec)
    S, Td, Dm = cfg.S, cfg.T_dec, cfg.d_model
    x_full = torch.empty((S, Td, Dm), dtype=torch.float32, device=inp["K"].device)
    x_comp = torch.empty_like(x_full)
    for t in range(Td):
        q = inp["Qd"][t]
        dfull.step(inp["Kd"], inp["Vd"], t + 1, q, _row_view(x_full, t), Td * Dm)
        e0 = ev() if record is not None else None
        sw.append(inp["Kd"], inp["Vd"], q, t)
        sw.decode(inp["Kd"], inp["Vd"], q, _row_view(x_comp, t), Td * Dm)
        e1 = ev() if record is not None else None
        sw.prune(t)
        if record is not None:
            record.append(("step", e0, e1, ev()))
        if kept_trace is not None:
            trace_kept(t)
    klv = kvc.kl(x_full.reshape(S * Td, Dm), x_comp.reshape(S * Td, Dm), inp["W"]).reshape(S, Td)
    pos = sw.pos.cpu()
    kept, off = [], 0
    for s in range(S):
        kept.append(pos[off:off + sw.lengths[s]].numpy().copy())
        off += sw.caps[s]
    return {"x_full": x_full, "x_comp": x_comp, "kl": klv, "kept": kept, "stepwise": sw}
