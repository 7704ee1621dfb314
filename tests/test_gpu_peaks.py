"""The measurement helpers run on the GPU and give plausible ceilings (they
are checked only for sanity: the vendor's HBM peak is 8 TB/s and the dense
bf16 MFMA peak 2.5 PFLOP/s; the exponential mix is bounded by the VALU issue rate)."""
import pytest

pytestmark = pytest.mark.gpu


def test_peak_read_and_mfma():
    from eviction_probe_softmax_amd import kvc
    gbs = kvc.peak_read_gbs(nbytes=1 << 30, reps=5)
    tf = kvc.peak_mfma_tflops(grid=1024, iters=512, reps=3)
    print(f"[peaks] read {gbs:.0f} GB/s, bf16 MFMA {tf:.0f} TFLOP/s", flush=True)
    assert 1000 < gbs < 8500
    assert 200 < tf < 2600


def test_peak_exp_mix():
    # one v_exp_f32 and three VALU operations an element; 256 CUs at 2.4 GHz
    # issue at most 64 fp32 VALU lanes a CU a cycle, so the rate is well below
    # 256 * 2.4e9 * 64 / 4 elements a second
    from eviction_probe_softmax_amd import kvc
    ge = kvc.peak_exp_gelems(grid=1024, iters=512, reps=3)
    print(f"[peaks] exp mix {ge:.0f} G elements/s", flush=True)
    assert 100 < ge < 256 * 2.4 * 64 / 4
