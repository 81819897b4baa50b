"""ft_moe_measure_rates on the device: every rate is measured and lies within what the part can do
(its published peaks: 8 TB/s of HBM, 2.5 / 5.0 / 10.1 PFLOP/s dense for bf16 / fp8 / fp6 and fp4
MFMA, PCIe 5.0 x16 at 63 GB/s per direction), and not absurdly far below it."""
from __future__ import annotations

import pytest
import torch

from gpu_util import log

pytestmark = pytest.mark.gpu


def test_measure_rates():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    r = ft.ft_moe_measure_rates(dev_bytes=512 << 20, host_bytes=128 << 20, reps=2)
    log(f"rates: {r}")
    assert r["compute_units"] >= 1 and r["stream_blocks"] >= r["compute_units"]
    assert 1000.0 < r["hbm_read_gbs"] < 8500.0
    assert 5.0 < r["host_read_gbs"] < 70.0
    assert 300.0 < r["mfma_bf16_tflops"] < 2600.0
    assert 600.0 < r["mfma_fp8_tflops"] < 5200.0
    assert 1200.0 < r["mfma_fp6_fp4_tflops"] < 10500.0
    assert 0.5 < r["mfma_clock_ghz"] < 2.6


def test_measure_rates_without_host_buffer():
    import routed_expert_ffn_wave_amd as ft
    r = ft.ft_moe_measure_rates(dev_bytes=64 << 20, host_bytes=0, reps=1)
    assert r["host_read_gbs"] == 0.0 and r["hbm_read_gbs"] > 0.0
