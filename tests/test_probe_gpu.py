"""The measurement hook flce_probe_mfma_rate: a register-only MFMA loop in
the GEMM kernels' wave tile. Zero operands run at least as fast as varying
ones (the matrix cores draw less power on them), and neither exceeds the
published dense bf16 peak by more than timing noise."""
import pytest
import torch

import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce

pytestmark = pytest.mark.gpu

PEAK = 2516.6


def test_probe_mfma_rate():
    ws = torch.empty(256 * 512 * 4, dtype=torch.uint8, device=G.dev())
    st = torch.cuda.current_stream().cuda_stream
    flce.flce_probe_mfma_rate(False, 20000, ws.data_ptr(), ws.numel(), st)  # clock warm-up
    rnd = flce.flce_probe_mfma_rate(False, 20000, ws.data_ptr(), ws.numel(), st)
    zero = flce.flce_probe_mfma_rate(True, 20000, ws.data_ptr(), ws.numel(), st)
    print(f"[probe] random {rnd:.0f} TFLOP/s, zeros {zero:.0f} TFLOP/s", flush=True)
    assert 0.0 < rnd <= 1.05 * PEAK and 0.0 < zero <= 1.05 * PEAK
    assert zero >= 0.95 * rnd


def test_probe_data_movement_modes():
    """Modes 2 and 3 add the wave tile's LDS fragment reads and its L2 -> LDS
    DMA; each rate is positive and below the published peak, a workspace
    without the DMA window is rejected for mode 3, an unknown mode too."""
    st = torch.cuda.current_stream().cuda_stream
    small = torch.empty(256 * 512 * 4, dtype=torch.uint8, device=G.dev())
    big = torch.empty(256 * 512 * 4 + (2 << 20), dtype=torch.uint8, device=G.dev())
    rates = {}
    for mode in (flce.PROBE_REGISTERS, flce.PROBE_LDS, flce.PROBE_LDS_DMA):
        rates[mode] = flce.flce_probe_mfma_rate(mode, 20000, big.data_ptr(), big.numel(), st)
    print(f"[probe] registers {rates[0]:.0f}, lds {rates[2]:.0f}, lds+dma {rates[3]:.0f} TFLOP/s",
          flush=True)
    for r in rates.values():
        assert 0.0 < r <= 1.05 * PEAK
    with pytest.raises(flce.FlceError):
        flce.flce_probe_mfma_rate(flce.PROBE_LDS_DMA, 20000, small.data_ptr(), small.numel(), st)
    with pytest.raises(flce.FlceError):
        flce.flce_probe_mfma_rate(4, 20000, big.data_ptr(), big.numel(), st)
