"""GPU check of kvc_decode_attn_static, the decode entry point that allocates
nothing (its workspace is the library's per-GPU scratch array): two calls in
a row through the C ABI, the second over a smaller cache, each against
kvc_decode_attn with a caller workspace on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
from workload import small_config, make_inputs
from parity import close, inputs_to

pytestmark = pytest.mark.gpu


def _step(kvc, fn, cache, dinp, cfg, t):
    Dm = cfg.d_model
    x = torch.full((cfg.S, Dm), float("nan"), dtype=torch.float32, device="cuda")
    o = torch.full((cfg.S, cfg.Ly, cfg.H * cfg.G, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    fn(cache, dinp["Kd"], dinp["Vd"], t + 1, cfg.T_dec, dinp["Qd"][t].contiguous(), cfg.G, x, Dm, o)
    torch.cuda.synchronize()
    return x, o


def test_static_decode_matches_workspace_decode_twice():
    from eviction_probe_softmax_amd import kvc
    from eviction_probe_softmax_amd.pipeline import Compressor
    cfg = small_config("ragged")
    inp = make_inputs(cfg)
    dinp = inputs_to(inp)
    print(f"[no-alloc] ragged lens={cfg.lens}", flush=True)
    comp = Compressor(cfg, inp["cu_seqlens"], inp["K"].dtype)
    packed = comp.compress(dinp)["cache"]
    full = kvc.full_view(comp.pb, dinp["K"], dinp["V"])
    n_full = int(full["seg_len"].to(torch.int64).sum())
    n_packed = int(packed["seg_len"].to(torch.int64).sum())
    assert n_packed < n_full
    cu = inp["cu_seqlens"].numpy()
    # first call over the full cache, the second over the smaller packed one
    for cache, t, ref in ((full, cfg.T_dec - 1, oracle.full_view(inp["K"], inp["V"], cu)), (packed, 0, None)):
        xs, os_ = _step(kvc, kvc.decode_attn_static, cache, dinp, cfg, t)
        xw, ow = _step(kvc, kvc.decode_attn, cache, dinp, cfg, t)
        assert torch.equal(xs, xw)
        assert torch.equal(os_, ow)
        if ref is not None:
            want, _ = oracle.decode_step(ref, inp["Kd"], inp["Vd"], inp["Qd"][t], t, cfg.G)
            close(xs, want, 2e-2, "x (static)", floor=1e-3)


def test_static_decode_rejects_a_cache_above_its_limit():
    import ctypes as C
    from eviction_probe_softmax_amd import kvc
    lim = kvc.decode_static_limit()
    assert lim == 64 << 20
    dev = torch.zeros(16, dtype=torch.uint8, device="cuda")
    seg_off = torch.zeros(1, dtype=torch.int64, device="cuda")
    seg_len = torch.zeros(1, dtype=torch.int32, device="cuda")
    x = torch.zeros(1024, dtype=torch.float32, device="cuda")
    # a capacity of 2^30 entries needs far more than the limit for the pieces'
    # partials; the call must refuse before launching anything
    rs = kvc.Ragged(K=dev.data_ptr(), V=dev.data_ptr(), lnmu=None, pos=None, seg_off=seg_off.data_ptr(),
                    seg_len=seg_len.data_ptr(), n_seq=1, n_layers=1, n_kv_heads=1, head_dim=128,
                    dtype=kvc.KVC_BF16, max_seg=0, capacity=1 << 30)
    need = int(kvc._lib.kvc_decode_workspace(C.byref(rs), 4, 0))
    assert need > lim
    st = kvc._lib.kvc_decode_attn_static(C.byref(rs), None, None, 0, 0, dev.data_ptr(), 4, x.data_ptr(), 512,
                                         None, None)
    assert st == -4
    assert "above" in kvc._lib.kvc_last_error().decode()
