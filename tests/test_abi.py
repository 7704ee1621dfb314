"""CPU checks of the C ABI: the library loads, exports every symbol the
header declares, and its host-side logic (validation, budgets, capacities,
workspace sizes) behaves as documented. Nothing here launches a kernel."""
import ctypes as C
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kvc.h")
PEAKS_HDR = os.path.join(ROOT, "include", "kvc_peaks.h")


def _declared(hdr=HDR):
    txt = open(hdr).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def kvc():
    from eviction_probe_softmax_amd import kvc as k
    return k


def test_every_declared_symbol_is_exported(kvc):
    names = _declared()
    assert len(names) >= 15
    lib = C.CDLL(kvc.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kvc.h but not exported"
    assert set(kvc.EXPORTS) == set(names)
    # every header under include/ is one of these two
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["kvc.h", "kvc_peaks.h"]
    peaks = _declared(PEAKS_HDR)
    for n in peaks:
        assert hasattr(lib, n), f"{n} declared in kvc_peaks.h but not exported"
    assert set(kvc.PEAK_EXPORTS) == set(peaks)


def test_peak_helpers_reject_bad_arguments(kvc):
    lib = kvc._lib
    dummy = C.c_void_p(16)
    assert lib.kvc_peak_read(None, 1024, 64, dummy, None) == -1
    assert lib.kvc_peak_read(dummy, 1000, 64, dummy, None) == -1   # not a multiple of 16
    assert lib.kvc_peak_read(dummy, 1024, 0, dummy, None) == -1
    assert lib.kvc_peak_mfma(0, 10, dummy, None) == -1
    assert lib.kvc_peak_mfma(8, 0, dummy, None) == -1
    assert lib.kvc_peak_mfma(8, 10, None, None) == -1
    assert lib.kvc_peak_exp(0, 10, dummy, None) == -1
    assert lib.kvc_peak_exp(8, 0, dummy, None) == -1
    assert lib.kvc_peak_exp(8, 10, None, None) == -1


def _problem(kvc, lens, **kw):
    from workload import Config
    base = dict(name="t", S=len(lens), Ly=2, H=2, G=4, d=128, lens=lens, P=64)
    base.update(kw)
    cfg = Config(**base)
    return kvc.make_problem(cfg, torch.tensor([0] + list(np.cumsum(lens))), torch.bfloat16, device="cpu"), cfg


def test_budgets_match_the_oracle(kvc):
    import oracle
    for kw in ({}, {"prompt_exact": 64, "recent_exact": 32, "suffix_exact": 48}, {"budget_ratio": 1 / 128},
               {"hybrid_frac": 0.2}, {"hybrid_frac": 0.75, "budget_ratio": 0.5, "floor_frac": 0.3},
               {"hybrid_frac": 1.0, "recent_exact": 32, "budget_ratio": 0.6}):
        pb, cfg = _problem(kvc, [1100, 777, 90], **kw)
        B, A, F = pb.budgets()
        ob = oracle.budgets(cfg.lens, cfg)
        assert B == [b["B"] for b in ob]
        assert A == [b["alloc"] for b in ob]
        assert F == [b["floor"] for b in ob]


def test_budget_error_when_recent_window_exceeds_budget(kvc):
    pb, cfg = _problem(kvc, [40], recent_exact=32, budget_ratio=0.01, budget_min=4)
    with pytest.raises(kvc.KvcError) as e:
        pb.budgets()
    assert e.value.status == -5


def test_capacity_and_strides(kvc):
    pb, cfg = _problem(kvc, [1100, 777], slot_len=64)
    cap = pb.pack_capacity()
    B, A, F = pb.budgets()
    assert cap == sum(A)               # no exact regions: the budget alone
    assert pb.slot_stride() == (1100 + 63) // 64 + 1
    pb2, _ = _problem(kvc, [1100, 777], slot_len=0, slot_min=16)
    assert pb2.slot_stride() == (1100 + 15) // 16 + 1


def test_invalid_arguments_are_rejected_on_the_host(kvc):
    lib = kvc._lib
    pb, cfg = _problem(kvc, [100])
    # NULL inputs: rejected before any launch
    st = lib.kvc_score(C.byref(pb.shape), C.byref(pb.params), None, None, None, None, None, None, None, None,
                       None, 0, None)
    assert st == -1
    # bad head dim
    sh = kvc.Shape.from_buffer_copy(pb.shape)
    sh.head_dim = 96
    st = lib.kvc_score(C.byref(sh), C.byref(pb.params), None, None, None, None, None, None, None, None, None, 0,
                       None)
    assert st == -2
    # workspace too small
    dummy = C.c_void_p(16)
    st = lib.kvc_score(C.byref(pb.shape), C.byref(pb.params), dummy, dummy, dummy, dummy, None, dummy, dummy,
                       dummy, dummy, 1, None)
    assert st == -4
    assert b"workspace" in lib.kvc_last_error()
    # group * probes beyond 256 rows
    p = kvc.Params.from_buffer_copy(pb.params)
    p.n_probe = 128
    st = lib.kvc_score(C.byref(pb.shape), C.byref(p), dummy, dummy, dummy, dummy, None, dummy, dummy, dummy,
                       dummy, 1 << 30, None)
    assert st == -2
    # decode: t_valid beyond t_cap
    rg = kvc.Ragged(K=dummy, V=dummy, seg_off=dummy, seg_len=dummy, n_seq=1, n_layers=1, n_kv_heads=1,
                    head_dim=128, dtype=1, max_seg=10, capacity=10)
    st = lib.kvc_decode_attn(C.byref(rg), dummy, dummy, 5, 4, dummy, 4, dummy, 512, None, dummy, 1 << 30, None)
    assert st == -1
    st = lib.kvc_decode_attn_planned(C.byref(rg), dummy, dummy, 5, 4, dummy, 4, dummy, 512, None, dummy, 1 << 30,
                                     None)
    assert st == -1
    # plan: workspace smaller than kvc_decode_workspace asks for
    need = lib.kvc_decode_workspace(C.byref(rg), 4, 4)
    assert need > 0
    st = lib.kvc_decode_plan(C.byref(rg), 4, 4, dummy, need - 1, None)
    assert st == -4
    # plan: group 3 is not supported
    st = lib.kvc_decode_plan(C.byref(rg), 3, 4, dummy, 1 << 30, None)
    assert st == -7
    # kl: d_model not a multiple of 128
    st = lib.kvc_kl(2, 100, 50, dummy, dummy, dummy, 1, dummy, dummy, 1 << 30, None)
    assert st == -2


def test_workspace_sizes_are_positive(kvc):
    pb, cfg = _problem(kvc, [1100, 777])
    for stage in range(6):
        assert kvc._lib.kvc_workspace_size(C.byref(pb.shape), C.byref(pb.params), stage) >= 0
    assert kvc._lib.kvc_workspace_size(C.byref(pb.shape), C.byref(pb.params), 0) > 0
    assert kvc._lib.kvc_kl_workspace(64, 4096, 32768, 1) > 64 * 2 * 4096 * 2
