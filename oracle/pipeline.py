"""The whole path, stage after stage, on the oracle.

Test infrastructure only (see the package docstring).

Order (GraceKV page, 'Method': partition -> represent -> value -> allocate ->
pack; decode over the packed cache; DistillCache paper, Sec. 3.1.4: per-step
KL between the full and the compressed cache's next-token distributions).
"""
from __future__ import annotations

import numpy as np

from .score import probe_scores
from .propagate import propagate
from .partition import slot_costs, slots_for
from .trees import build_trees
from .select import floor_select, auction, token_topk, hybrid_units
from .pack import pack
from .decode import decode_all, full_view
from .kl import kl_rows


def run_pipeline(inp, cfg, stages=("compress", "decode", "kl")):
    cu = inp["cu_seqlens"].numpy()
    out = {}
    sc = probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    out.update(sc)
    pr = propagate(inp["K"], inp["Qctx"], sc["r0"], cu, cfg)
    out.update(pr)
    rel = pr["rel"]
    full = hybrid_units(sc["head_sens"], cu, cfg) if getattr(cfg, "hybrid_frac", 0.0) > 0 else None
    out["full_units"] = full
    if cfg.token_mode:
        slots = [[] for _ in range(len(cu) - 1)]
        taken, spent = token_topk(rel, cu, cfg, full)
        trees = None
    else:
        cost_q = cut_q = None
        if cfg.slot_len == 0:
            cost_q, cut_q = slot_costs(inp["hidden"], cu, cfg, inp.get("surprisal"))
            out["dp_cost_q"], out["dp_cut_q"] = cost_q, cut_q
        slots = slots_for(cu, cfg, cost_q, cut_q)
        trees = build_trees(inp["K"], inp["V"], inp["Qp"], sc["lse"], rel, sc["head_sens"],
                            cu, slots, cfg, cut_q=cut_q)
        out["trees"] = trees
        topo = trees["node_topo"]
        ftaken, fspent = floor_select(rel, sc["head_sens"], trees["op_cost"], cu, slots, cfg, full=full, topo=topo)
        out["floor_taken"], out["floor_spent"] = ftaken, fspent
        taken, spent = auction(trees["op_util"], trees["op_cost"], ftaken, fspent, cu, slots, cfg, full=full,
                               topo=topo)
    out["slots"] = slots
    out["taken"], out["spent"] = taken, spent
    cache = pack(inp["K"], inp["V"], rel, trees, taken, cu, slots, cfg)
    out["cache"] = cache
    if "decode" in stages:
        G = cfg.G
        x_comp = decode_all(cache, inp["Kd"], inp["Vd"], inp["Qd"], G)
        x_full = decode_all(full_view(inp["K"], inp["V"], cu), inp["Kd"], inp["Vd"], inp["Qd"], G)
        out["x_comp"], out["x_full"] = x_comp, x_full
        if "kl" in stages:
            n = x_full.shape[0] * x_full.shape[1]
            out["kl"] = kl_rows(x_full.reshape(n, -1), x_comp.reshape(n, -1), inp["W"],
                                cfg.w_dtype).reshape(x_full.shape[0], x_full.shape[1])
    return out
