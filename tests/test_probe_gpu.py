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
