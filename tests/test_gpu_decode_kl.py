"""GPU parity: decode attention over ragged caches (kvc_decode_attn) and the
vocab KL (kvc_kl) against the CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
from workload import small_config, make_inputs
from parity import close, as_np, to_dev, inputs_to

pytestmark = pytest.mark.gpu

# decode outputs are sums of attention outputs that can sit near zero; the
# relative bar applies above 1e-3 of the tensor's largest magnitude
DEC_RTOL, DEC_FLOOR = 2e-2, 1e-3


def _kvc():
    from eviction_probe_softmax_amd import kvc
    return kvc


def _run_decode(kvc, cache_dev, inp_dev, cfg, S):
    Td = cfg.T_dec
    d_model = cfg.d_model
    x = torch.zeros((S, Td, d_model), dtype=torch.float32, device="cuda")
    dec = kvc.Decoder(cache_dev, cfg.G, Td)
    row = torch.zeros((S, d_model), dtype=torch.float32, device="cuda")
    for t in range(Td):
        dec.step(inp_dev["Kd"], inp_dev["Vd"], t + 1, inp_dev["Qd"][t].contiguous(), row, d_model)
        x[:, t] = row
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name", ["tiny", "mistral1", "ragged", "stress"])
def test_decode_full_cache(name):
    kvc = _kvc()
    cfg = small_config(name)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    print(f"[decode-full] {name} lens={cfg.lens} T_dec={cfg.T_dec}", flush=True)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    cache = kvc.full_view(pb, dinp["K"], dinp["V"])
    x = _run_decode(kvc, cache, dinp, cfg, cfg.S)
    cu = inp["cu_seqlens"].numpy()
    want = oracle.decode_all(oracle.full_view(inp["K"], inp["V"], cu), inp["Kd"], inp["Vd"], inp["Qd"], cfg.G)
    close(x, want, DEC_RTOL, "x_full", floor=DEC_FLOOR)
    # the fp32 path is far tighter than the bar: keep an eye on it
    err = np.abs(as_np(x) - want).max() / np.abs(want).max()
    assert err < 1e-4, err


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_decode_ragged_cache_with_multiplicity(name):
    kvc = _kvc()
    cfg = small_config(name)
    inp = make_inputs(cfg)
    rng = np.random.default_rng(5)
    S, Ly, H, d = cfg.S, cfg.Ly, cfg.H, cfg.d
    # a ragged cache of random entries (lengths 0..700, crossing split chunks)
    lens = rng.integers(0, 700, (S, Ly, H))
    lens[0, 0, 0] = 0
    N = int(lens.sum())
    dt = inp["K"].dtype
    Kc = torch.randn((N, d)).to(dt)
    Vc = torch.randn((N, d)).to(dt)
    lnmu = torch.tensor(np.log(rng.uniform(1, 4, N)), dtype=torch.float32)
    seg_off = np.zeros((S, Ly, H), np.int64)
    off = 0
    for l in range(Ly):
        for h in range(H):
            for s in range(S):
                seg_off[s, l, h] = off
                off += lens[s, l, h]
    ocache = {"K": oracle.to64(Kc), "V": oracle.to64(Vc), "lnmu": lnmu.numpy(), "seg_off": seg_off,
              "seg_len": lens.astype(np.int32)}
    gcache = {"K": Kc.cuda(), "V": Vc.cuda(), "lnmu": lnmu.cuda(), "pos": None,
              "seg_off": torch.from_numpy(seg_off).cuda(), "seg_len": torch.from_numpy(lens.astype(np.int32)).cuda(),
              "n_seq": S, "n_layers": Ly, "n_kv_heads": H, "head_dim": d, "max_seg": int(lens.max())}
    dinp = inputs_to(inp)
    x = _run_decode(kvc, gcache, dinp, cfg, S)
    want = oracle.decode_all(ocache, inp["Kd"], inp["Vd"], inp["Qd"], cfg.G)
    close(x, want, DEC_RTOL, "x_ragged", floor=DEC_FLOOR)
    # per-layer outputs through o_out
    o = torch.zeros((S, Ly, H * cfg.G, d), dtype=torch.float32, device="cuda")
    xx = torch.zeros((S, cfg.d_model), dtype=torch.float32, device="cuda")
    kvc.decode_attn(gcache, dinp["Kd"], dinp["Vd"], 1, cfg.T_dec, dinp["Qd"][0].contiguous(), cfg.G, xx,
                    cfg.d_model, o)
    _, oo = oracle.decode_step(ocache, inp["Kd"], inp["Vd"], inp["Qd"][0], 0, cfg.G)
    close(o, oo, DEC_RTOL, "o_layers", floor=DEC_FLOOR)


@pytest.mark.parametrize("dtype,t_valid", [(torch.bfloat16, 1000), (torch.bfloat16, 769), (torch.float32, 600),
                                            (torch.float32, 0)])
def test_decode_long_tails_and_empty_segments(dtype, t_valid):
    """Tails longer than one piece (768 entries bf16, 256 fp32) split into
    several tail pieces; units whose segment is empty attend over the tail
    alone, or (no tail) give zeros; segments of 1, 767, 769 and 2000 entries
    cover one, two and three segment pieces."""
    kvc = _kvc()
    g = torch.Generator().manual_seed(17)
    S, Ly, H, G, d = 2, 2, 2, 4, 128
    lens = np.array([[[0, 1], [767, 769]], [[2000, 0], [5, 1536]]], dtype=np.int64)  # [S][Ly][H]
    N = int(lens.sum())
    Kc = torch.randn((N, d), generator=g).to(dtype)
    Vc = torch.randn((N, d), generator=g).to(dtype)
    lnmu = torch.log(1 + 3 * torch.rand((N,), generator=g)).float()
    seg_off = np.zeros((S, Ly, H), np.int64)
    off = 0
    for s in range(S):
        for l in range(Ly):
            for h in range(H):
                seg_off[s, l, h] = off
                off += lens[s, l, h]
    t_cap = max(t_valid, 1)
    Kd = torch.randn((Ly, H, S, t_cap, d), generator=g).to(dtype)
    Vd = torch.randn((Ly, H, S, t_cap, d), generator=g).to(dtype)
    Q = torch.randn((S, Ly, H * G, d), generator=g).to(dtype)
    print(f"[decode-tails] {dtype} t_valid={t_valid}", flush=True)
    gcache = {"K": Kc.cuda(), "V": Vc.cuda(), "lnmu": lnmu.cuda(), "pos": None,
              "seg_off": torch.from_numpy(seg_off).cuda(), "seg_len": torch.from_numpy(lens.astype(np.int32)).cuda(),
              "n_seq": S, "n_layers": Ly, "n_kv_heads": H, "head_dim": d, "max_seg": int(lens.max())}
    x = torch.full((S, H * G * d), float("nan"), dtype=torch.float32, device="cuda")
    o = torch.full((S, Ly, H * G, d), float("nan"), dtype=torch.float32, device="cuda")
    kvc.decode_attn(gcache, Kd.cuda(), Vd.cuda(), t_valid, t_cap, Q.cuda(), G, x, H * G * d, o)
    torch.cuda.synchronize()
    ocache = {"K": oracle.to64(Kc), "V": oracle.to64(Vc), "lnmu": lnmu.numpy(), "seg_off": seg_off,
              "seg_len": lens.astype(np.int32)}
    # the oracle's step t attends over tail tokens 0..t
    if t_valid > 0:
        want_x, want_o = oracle.decode_step(ocache, Kd, Vd, Q, t_valid - 1, G)
    else:
        want_o = np.zeros((S, Ly, H * G, d))
        for s in range(S):
            for l in range(Ly):
                for h in range(H):
                    a0, n = int(seg_off[s, l, h]), int(lens[s, l, h])
                    if n == 0:
                        continue
                    Ke, Ve = ocache["K"][a0:a0 + n], ocache["V"][a0:a0 + n]
                    z = (oracle.to64(Q)[s, l, h * G:(h + 1) * G] @ Ke.T) / math.sqrt(d) + ocache["lnmu"][a0:a0 + n]
                    p = np.exp(z - z.max(axis=1, keepdims=True))
                    want_o[s, l, h * G:(h + 1) * G] = (p / p.sum(axis=1, keepdims=True)) @ Ve
        want_x = want_o.sum(axis=1).reshape(S, -1)
    rt = DEC_RTOL if dtype == torch.bfloat16 else 1e-4
    close(o, want_o, rt, "o", floor=DEC_FLOOR)
    close(x, want_x, rt, "x", floor=DEC_FLOOR)


def test_decode_plan_over_many_units():
    """16,384 units (more than one round of the plan's scan), segments of 0..5
    entries, head dim 64, group 1: every unit's output against the definition."""
    kvc = _kvc()
    g = torch.Generator().manual_seed(23)
    S, Ly, H, G, d, t_cap, t_valid = 64, 16, 16, 1, 64, 3, 2
    lens = torch.randint(0, 6, (S, Ly, H), generator=g).numpy().astype(np.int64)
    N = int(lens.sum())
    Kc = torch.randn((N, d), generator=g).to(torch.bfloat16)
    Vc = torch.randn((N, d), generator=g).to(torch.bfloat16)
    seg_off = np.concatenate([[0], np.cumsum(lens.reshape(-1))[:-1]]).reshape(S, Ly, H).astype(np.int64)
    Kd = torch.randn((Ly, H, S, t_cap, d), generator=g).to(torch.bfloat16)
    Vd = torch.randn((Ly, H, S, t_cap, d), generator=g).to(torch.bfloat16)
    Q = torch.randn((S, Ly, H * G, d), generator=g).to(torch.bfloat16)
    print(f"[decode-units] {S * Ly * H} units, {N} entries", flush=True)
    gcache = {"K": Kc.cuda(), "V": Vc.cuda(), "lnmu": None, "pos": None,
              "seg_off": torch.from_numpy(seg_off).cuda(), "seg_len": torch.from_numpy(lens.astype(np.int32)).cuda(),
              "n_seq": S, "n_layers": Ly, "n_kv_heads": H, "head_dim": d, "max_seg": int(lens.max())}
    x = torch.full((S, H * G * d), float("nan"), dtype=torch.float32, device="cuda")
    o = torch.full((S, Ly, H * G, d), float("nan"), dtype=torch.float32, device="cuda")
    kvc.decode_attn(gcache, Kd.cuda(), Vd.cuda(), t_valid, t_cap, Q.cuda(), G, x, H * G * d, o)
    torch.cuda.synchronize()
    # the definition, vectorised over units: softmax over the segment and the tail
    K64, V64 = oracle.to64(Kc), oracle.to64(Vc)
    Kd64, Vd64, Q64 = oracle.to64(Kd), oracle.to64(Vd), oracle.to64(Q)
    want = np.zeros((S, Ly, H * G, d))
    for s in range(S):
        for l in range(Ly):
            for h in range(H):
                a0, n = int(seg_off[s, l, h]), int(lens[s, l, h])
                Ke = np.concatenate([K64[a0:a0 + n], Kd64[l, h, s, :t_valid]])
                Ve = np.concatenate([V64[a0:a0 + n], Vd64[l, h, s, :t_valid]])
                z = Ke @ Q64[s, l, h] / math.sqrt(d)
                p = np.exp(z - z.max())
                want[s, l, h] = (p / p.sum()) @ Ve
    close(o, want, DEC_RTOL, "o", floor=DEC_FLOOR)
    close(x, want.sum(axis=1).reshape(S, -1), DEC_RTOL, "x", floor=DEC_FLOOR)


@pytest.mark.parametrize("name", ["ragged", "mistral1"])
def test_decode_planned_steps_match_single_call_and_repeat(name):
    """The planned path (one plan, many steps) gives the single-call path's
    bits; 16 repeats of one step give identical bits (the pieces, the merge
    and the last-arriver layer sum are deterministic); o_out holds the layers
    whose sum, in layer order, is x."""
    kvc = _kvc()
    cfg = small_config(name)
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    pb = kvc.make_problem(cfg, inp["cu_seqlens"], inp["K"].dtype)
    cache = kvc.full_view(pb, dinp["K"], dinp["V"])
    S, Td, Dm = cfg.S, cfg.T_dec, cfg.d_model
    dec = kvc.Decoder(cache, cfg.G, Td)
    for t in (0, Td // 2, Td - 1):
        print(f"[decode-planned] {name} t={t}", flush=True)
        q = dinp["Qd"][t].contiguous()
        a = torch.zeros((S, Dm), dtype=torch.float32, device="cuda")
        b = torch.zeros((S, Dm), dtype=torch.float32, device="cuda")
        o = torch.zeros((S, cfg.Ly, cfg.H * cfg.G, cfg.d), dtype=torch.float32, device="cuda")
        dec.step(dinp["Kd"], dinp["Vd"], t + 1, q, a, Dm)
        kvc.decode_attn(cache, dinp["Kd"], dinp["Vd"], t + 1, Td, q, cfg.G, b, Dm, o)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        xs = torch.zeros_like(a)
        for l in range(cfg.Ly):
            xs += o[:, l].reshape(S, -1)
        assert torch.equal(xs, a)
        for _ in range(16):
            dec.step(dinp["Kd"], dinp["Vd"], t + 1, q, b, Dm)
            torch.cuda.synchronize()
            assert torch.equal(a, b)


@pytest.mark.parametrize("w_dtype,dm,vocab,n", [("f32", 256, 2048, 37), ("bf16", 1024, 1000, 37),
                                                 ("bf16", 4096, 32768, 37), ("bf16", 512, 1000, 100),
                                                 ("f32", 384, 300, 70), ("bf16", 128, 64, 1),
                                                 ("bf16", 256, 8192, 1024), ("bf16", 1024, 4096, 600),
                                                 ("bf16", 256, 1024, 1100)])
def test_kl_matches_oracle(w_dtype, dm, vocab, n):
    """n pairs give 2n rows: 37 leaves a partial last row block, 100 and 70
    span two 128-row tiles, vocab 1000 / 300 / 64 leave partial column tiles;
    from 1,024 rows on (bf16, vocab a multiple of 256) the 256 x 256-tiled
    kernel runs: 2,048 rows x 8,192 columns, and 1,200 and 2,200 rows with a
    padded last row tile."""
    kvc = _kvc()
    g = torch.Generator().manual_seed(3)
    xf = torch.randn((n, dm), generator=g)
    xc = xf + 0.5 * torch.randn((n, dm), generator=g)
    W = (torch.randn((vocab, dm), generator=g) * (4.0 / math.sqrt(dm))).to(
        torch.bfloat16 if w_dtype == "bf16" else torch.float32)
    print(f"[kl] {w_dtype} dm={dm} vocab={vocab} n={n}", flush=True)
    got = kvc.kl(xf.cuda(), xc.cuda(), W.cuda())
    torch.cuda.synchronize()
    want = oracle.kl_rows(xf.numpy(), xc.numpy(), W, w_dtype)
    err = np.abs(as_np(got) - want)
    assert err.max() <= 1e-3, (err.max(), want[:4], as_np(got)[:4])
    same = kvc.kl(xf.cuda(), xf.cuda(), W.cuda())
    assert torch.all(same == 0), same


def test_kl_at_the_ragged_batch_shape_on_sampled_pairs():
    """The bench's KL call: 4,096 pairs (8,192 rows) x d_model 4,096 x vocab
    32,768 in bf16; sampled pairs against the oracle, identical rows give 0."""
    kvc = _kvc()
    g = torch.Generator().manual_seed(5)
    n, dm, vocab = 4096, 4096, 32768
    xf = torch.randn((n, dm), generator=g)
    xc = xf + 0.3 * torch.randn((n, dm), generator=g)
    xc[7] = xf[7]
    W = (torch.randn((vocab, dm), generator=g) * (4.0 / math.sqrt(dm))).to(torch.bfloat16)
    got = as_np(kvc.kl(xf.cuda(), xc.cuda(), W.cuda()))
    torch.cuda.synchronize()
    idx = [0, 1, 7, 255, 256, 1023, 2048, 3333, 4095]
    want = oracle.kl_rows(xf[idx].numpy(), xc[idx].numpy(), W, "bf16")
    err = np.abs(got[idx] - want)
    print(f"[kl] ragged shape: max |dKL| {err.max():.2e} over {len(idx)} sampled pairs", flush=True)
    assert err.max() <= 1e-3, (err.max(), got[idx], want)
    assert got[7] == 0.0
