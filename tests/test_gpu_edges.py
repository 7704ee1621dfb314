"""GPU edge cases against the oracle, through the C ABI: degenerate sequence
lengths (empty, one and two tokens, a one-token last slot), an empty
budget, distortion-probe counts below one per lane, every supported GQA
group size in decode (including MHA), decode with no appended tokens, and
head dim 64 in bf16."""
import numpy as np
import pytest
import torch

import oracle
from workload import small_config, make_inputs
from parity import close, as_np, inputs_to, jaccard, to_dev, slots_to_dev, check_kl, oracle_on_taken

pytestmark = pytest.mark.gpu


def _kvc():
    from eviction_probe_softmax_amd import kvc
    return kvc


def _e2e(cfg, inp):
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor, decode_both
    dinp = inputs_to(inp)
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    out = comp.compress(dinp)
    full = kvc.full_view(comp.pb, dinp["K"], dinp["V"])
    xf, xc = decode_both(out["cache"], full, dinp, cfg)
    n = cfg.S * cfg.T_dec
    klv = kvc.kl(xf.reshape(n, -1), xc.reshape(n, -1), dinp["W"]).reshape(cfg.S, cfg.T_dec)
    torch.cuda.synchronize()
    return out, xf, xc, klv


@pytest.mark.parametrize("base,lens", [("ragged", [0, 1, 2, 700, 1100]), ("ragged", [300, 0]),
                                       ("stress", [65, 129, 64])])
def test_degenerate_lengths_end_to_end(base, lens):
    # ragged: prompt/suffix 256 and recent 128 exact, so short sequences are
    # all exact and 700 leaves a 60-token compressible region; stress: fixed
    # 64-token slots, 65 and 129 leave one-token last slots; an empty
    # sequence has no entries and decodes its appended tokens only
    cfg = small_config(base).replace(S=len(lens), lens=lens, n_plant=2)
    inp = make_inputs(cfg)
    print(f"[edge] {base} lens={lens}", flush=True)
    out, xf, xc, klv = _e2e(cfg, inp)
    o = oracle.run_pipeline(inp, cfg)
    assert np.array_equal(as_np(out["spent"]), o["spent"])
    j = jaccard(as_np(out["taken"]), o["taken"])
    assert j >= 0.99, j
    close(xf, o["x_full"], 2e-2, "x_full", floor=1e-3)
    # against the oracle's decode and KL of the GPU's own taken set
    xc_o, kl_o = oracle_on_taken(inp, cfg, o, out["taken"])
    close(xc, xc_o, 2e-2, "x_comp", floor=1e-3)
    check_kl(klv, xf, xc, inp["W"], kl_o, base, o["x_full"], xc_o)


def test_empty_budget_keeps_nothing():
    cfg = small_config("stress").replace(budget_ratio=0.0, budget_min=0)
    inp = make_inputs(cfg)
    out, xf, xc, klv = _e2e(cfg, inp)
    assert int(as_np(out["spent"]).sum()) == 0
    assert int(as_np(out["cache"]["seg_len"]).sum()) == 0
    assert not as_np(out["taken"]).any()
    o = oracle.run_pipeline(inp, cfg)
    close(xc, o["x_comp"], 2e-2, "x_comp (appended tokens only)", floor=1e-3)
    check_kl(klv, xf, xc, inp["W"], o["kl"], "empty budget", o["x_full"], o["x_comp"])


@pytest.mark.parametrize("n_dprobe", [48, 20, 1])
def test_trees_with_fewer_distortion_rows(n_dprobe):
    kvc = _kvc()
    cfg = small_config("stress").replace(n_dprobe=n_dprobe)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    cu = inp["cu_seqlens"].numpy()
    sc = oracle.probe_scores(inp["K"], inp["V"], inp["Qp"], cu, cfg)
    pr = oracle.propagate(inp["K"], inp["Qctx"], sc["r0"], cu, cfg)
    slots = oracle.slots_for(cu, cfg)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    ss, ns = slots_to_dev(slots, pb.slot_stride())
    rc, rs = kvc.rope_table(cfg.rope_base, cfg.d, max(cfg.lens))
    g = kvc.build_trees(pb, dinp["K"], dinp["V"], dinp["Qp"], to_dev(sc["lse"]), to_dev(pr["rel"]),
                        to_dev(sc["head_sens"]), rc, rs, ss, ns)
    torch.cuda.synchronize()
    o = oracle.build_trees(inp["K"], inp["V"], inp["Qp"], sc["lse"], pr["rel"], sc["head_sens"], cu, slots, cfg)
    close(g["node_D"], o["node_D"], 1e-3, "node_D", floor=1e-3)
    close(g["op_util"], o["op_util"], 1e-3, "op_util", floor=1e-3)


@pytest.mark.parametrize("G,d", [(1, 128), (2, 128), (8, 128), (4, 64)])
@pytest.mark.parametrize("t_valid", [0, 3])
def test_decode_group_sizes_and_tail(G, d, t_valid):
    """Full-cache decode for every supported group size (G = 1 is MHA) and
    head dim, with and without appended tokens."""
    kvc = _kvc()
    cfg = small_config("stress").replace(G=G, d=d, P=min(64, 256 // G), T_dec=4)
    inp = make_inputs(cfg, with_qctx=False)
    dinp = inputs_to(inp)
    print(f"[edge decode] G={G} d={d} t_valid={t_valid}", flush=True)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    cache = kvc.full_view(pb, dinp["K"], dinp["V"])
    dec = kvc.Decoder(cache, G, cfg.T_dec)
    x = torch.zeros((cfg.S, cfg.d_model), dtype=torch.float32, device="cuda")
    o = torch.zeros((cfg.S, cfg.Ly, cfg.H * G, d), dtype=torch.float32, device="cuda")
    q = dinp["Qd"][max(t_valid - 1, 0)].contiguous()
    dec.step(dinp["Kd"], dinp["Vd"], t_valid, q, x, cfg.d_model, o_out=o)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].numpy()
    full = oracle.full_view(inp["K"], inp["V"], cu)
    # t_valid appended tokens: the oracle's step t sees tokens 0..t
    Kd, Vd = inp["Kd"], inp["Vd"]
    if t_valid == 0:
        Kd = Kd[:, :, :, :0]
        Vd = Vd[:, :, :, :0]
        want_x, want_o = oracle.decode_step(full, Kd, Vd, inp["Qd"][0], -1, G)
    else:
        want_x, want_o = oracle.decode_step(full, Kd, Vd, inp["Qd"][t_valid - 1], t_valid - 1, G)
    close(o, want_o, 2e-2, "o", floor=1e-3)
    close(x, want_x, 2e-2, "x", floor=1e-3)
