"""GPU check of the measurement kernels behind the mainloop choice
(libnvfp4_mainloop_probe.so): what the scaled FP4 conversion does with a
scale that is not a power of two. The inner-loop rates are measurements, not
correctness properties: ``bench.py --mainloop-probe`` reports them."""
import sys

import pytest
import torch

from moe_matmul_amd import probe

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def test_scaled_fp4_conversion_applies_only_the_scale_exponent():
    """v_cvt_scalef32_pk_f16_fp4 of FP4 1.0 under an f32 scale gives 2^floor(log2 scale):
    the mantissa of an E4M3 scale needs a multiply of its own."""
    announce("nvfp4_probe_cvt_scale")
    scales = [1.0, 1.5, 1.875, 3.0, 0.75, 448.0, 0.125, 15.0]
    sc = torch.tensor(scales, dtype=torch.float32, device="cuda")
    out = torch.full((len(scales),), -1, dtype=torch.int16, device="cuda")
    probe.nvfp4_probe_cvt_scale(sc.data_ptr(), len(scales), out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.float16).float().tolist()
    assert got == [1.0, 1.0, 1.0, 2.0, 0.5, 256.0, 0.125, 8.0]
