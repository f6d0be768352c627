"""The device probe on the GPU: the matrix-core rate it measures is the 32x32x16 fp16 MFMA's
4096 FLOP per clock per compute unit (256 compute units x 4 SIMDs x 1024) at the clock the run held,
the clocks are plausible, and the LDS and HBM figures are positive and below their hardware bounds."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_probe_rates_are_consistent():
    import exact_long_context_cqsa_amd as m
    print("[gpu-case] probe_device", file=sys.stderr, flush=True)
    p = m.probe_device(copy_bytes=256 << 20, repeats=3)
    print("[gpu-case] probe:", {k: v for k, v in p.items() if not k.endswith("_seconds")}, file=sys.stderr, flush=True)
    assert p["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert 0.5 < p["mfma_clock_ghz"] < 3.0 and 0.5e9 < p["lds_clock_hz"] < 3.0e9
    # the loop adds a compare and a branch per four MFMAs; the clock is averaged over each wave's loop
    assert 3500.0 < p["mfma_flop_per_clk_per_cu"] < 4300.0, p["mfma_flop_per_clk_per_cu"]
    assert 32.0 < p["lds_bytes_per_clk_per_cu"] < 520.0, p["lds_bytes_per_clk_per_cu"]
    assert 100.0 < p["hbm_copy_gbs"] < 8200.0, p["hbm_copy_gbs"]
    assert p["mfma_seconds"] > 0 and p["lds_seconds"] > 0 and p["copy_seconds"] > 0


def test_probe_rejects_bad_arguments():
    import exact_long_context_cqsa_amd as m
    with pytest.raises(m.CqsaError):
        m.probe_device(copy_bytes=1000)
    with pytest.raises(m.CqsaError):
        m.probe_device(repeats=0)
