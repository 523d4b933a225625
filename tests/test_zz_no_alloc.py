"""nvfp4_grouped_gemm_scratch (no allocation: the stream-K partials live in
the library's fixed device array) against nvfp4_grouped_gemm_ex with a caller
workspace, on two calls in a row, the second smaller. Same plan, same kernels:
the outputs must be bitwise equal, and within the oracle's tolerance."""
import sys

import numpy as np
import pytest
import torch

import moe_matmul_amd as mm
import oracle.nvfp4_oracle as O
from moe_matmul_amd import device as dev
from moe_matmul_amd import synth

pytestmark = pytest.mark.gpu

GUARD = 64


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_both(shapes, groups, cfg, split):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    geo = mm.nvfp4_launch_geometry(shapes, cus, cfg, split)
    announce(f"scratch vs ex shapes={shapes} cfg={cfg} split={split} plan={geo}")
    d_ex = dev.upload(shapes, groups, c_guard=GUARD)
    d_sc = dev.upload(shapes, groups, c_guard=GUARD)
    ws = dev.workspace_for(shapes)
    st = torch.cuda.current_stream()
    abc, sf = dev.pointer_tables(d_ex)
    mm.nvfp4_grouped_gemm_ex(shapes, abc, sf, len(shapes), ws.data_ptr(), ws.numel(), cfg, split, st)
    abc, sf = dev.pointer_tables(d_sc)
    mm.nvfp4_grouped_gemm_scratch(shapes, abc, sf, len(shapes), cfg, split, st)
    torch.cuda.synchronize()
    assert dev.guards_intact(d_ex) and dev.guards_intact(d_sc)
    ref = O.grouped_gemm(shapes, groups)
    for (m, n, k, l), a, b, r in zip(shapes, dev.c_as_numpy(shapes, d_ex), dev.c_as_numpy(shapes, d_sc), ref):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (m, n, k, l)
        assert not O.tolerance_violations(b, r["c16"], r["s"]).any(), (m, n, k, l)
    return geo


def test_scratch_matches_ex_on_two_calls_the_second_smaller():
    first = [(256, 256, 16384, 1), (40, 136, 64, 1), (129, 264, 2048 + 32, 1)]
    second = [(100, 136, 1024, 1), (33, 72, 512, 1)]
    for shapes, seed in ((first, 71), (second, 72)):
        groups = synth.make_custom(shapes, seed=seed)
        geo = run_both(shapes, groups, 3, 1)  # stream-K, 128x128 tiles: partials within the scratch array
        assert geo["split"] == 1 and 0 < geo["workspace_bytes"] <= mm.NVFP4_SCRATCH_BYTES
        run_both(shapes, groups, -1, -1)  # the heuristic, whatever it picks within the array


def test_scratch_refuses_a_plan_beyond_its_size():
    """Forced stream-K with 256x256 tiles on one long-K tile spreads over every
    compute unit: two 256 KiB partial slots per workgroup, beyond the array."""
    shapes = [(256, 256, 1 << 16, 1)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = mm.nvfp4_launch_geometry(shapes, cus, 0, 1)["workspace_bytes"]
    if need <= mm.NVFP4_SCRATCH_BYTES:
        pytest.skip("too few compute units for a plan beyond the scratch array")
    announce(f"scratch entry point, forced stream-K needing {need} bytes")
    groups = synth.make_custom(shapes, seed=73)
    d = dev.upload(shapes, groups)
    abc, sf = dev.pointer_tables(d)
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_scratch(shapes, abc, sf, 1, 0, 1, torch.cuda.current_stream())
    assert e.value.code == mm.NVFP4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert np.all(d[0]["c"].cpu().numpy().view(np.uint16) == dev.FP16_NAN_BITS)  # nothing was launched
