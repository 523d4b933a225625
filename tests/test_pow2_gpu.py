"""GPU parity of nvfp4_grouped_gemm_pow2 (every scale zero or a positive power
of two, computed with the FP4 MFMA and E8M0 scales) against the CPU oracle,
and its status word.

Tolerance as in test_parity_gpu: |C_gpu - C_ref| <= 2 ulp16(C_ref) + 1e-5 * S
(the oracle is the same exact definition; only the fp32 summation order of
the kernel differs). C is pre-filled with an fp16 NaN pattern inside guard
canaries.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import moe_matmul_amd as mm
import oracle.nvfp4_oracle as O
from moe_matmul_amd import device as dev
from moe_matmul_amd import synth

pytestmark = pytest.mark.gpu

GUARD = 64
# every scale the entry point takes: 0, the subnormal powers 2^-9 .. 2^-7 and
# the normal ones 2^-6 .. 2^8
POW2_ALL = np.array([0x00, 0x01, 0x02, 0x04] + [e << 3 for e in range(1, 16)], dtype=np.uint8)


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_pow2(shapes, groups, tile_config=-1, split_mode=-1, label=""):
    announce(f"pow2 {label} shapes={shapes} tile_config={tile_config} split_mode={split_mode}")
    d = dev.upload(shapes, groups, c_guard=GUARD)
    ws = dev.workspace_for(shapes) if split_mode != 0 else None
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev.run_pow2(shapes, d, status, tile_config=tile_config, split_mode=split_mode, workspace=ws)
    torch.cuda.synchronize()
    assert dev.guards_intact(d), "store outside C"
    return dev.c_as_numpy(shapes, d), int(status.item())


def check_rows(shapes, groups, got, rows=None):
    ref = O.grouped_gemm(shapes, groups, rows=rows)
    for g, ((m, n, k, l), c, r) in enumerate(zip(shapes, got, ref)):
        if m == 0 or n == 0:
            continue
        if rows is not None:
            c = c[:, rows[g], :]
        bad = O.tolerance_violations(c, r["c16"], r["s"])
        if bad.any():
            idx = np.argwhere(bad)[:5]
            detail = [(tuple(i), float(c[tuple(i)]), float(r["c16"][tuple(i)])) for i in idx]
            pytest.fail(f"group {g} {shapes[g]}: {int(bad.sum())} of {bad.size} elements out of tolerance, "
                        f"e.g. {detail}")


EDGE = {
    "g8_ragged": [(40, 4096, 256, 1), (401, 256, 128, 1), (7, 8, 64, 1), (128, 128, 128, 1),
                  (255, 520, 448, 1), (300, 200, 64, 1), (1, 1024, 512, 1), (96, 96, 960, 1)],
    "empty_groups_in_middle": [(64, 64, 128, 1), (0, 64, 128, 1), (100, 128, 256, 1), (64, 0, 128, 1),
                               (33, 72, 64, 1)],
    "k_zero": [(40, 48, 0, 1), (16, 16, 64, 1)],
    "batch_l2": [(100, 136, 192, 2)],
}


@pytest.mark.parametrize("cfg", [-1, 0, 1, 2, 3, 4])
def test_pow2_small_workloads_and_edges(cfg):
    """The two small workloads with power-of-two scales, and ragged, empty,
    k = 0 and l = 2 groups whose scales span every accepted code (zero,
    subnormal, 2^8) in every tile configuration."""
    for idx in (0, 1):
        shapes, groups = synth.make_workload(idx, scale_codes=synth.POW2_SCALE_CODES)
        got, status = run_pow2(shapes, groups, tile_config=cfg, label=f"workload {idx}")
        assert status == 0
        check_rows(shapes, groups, got)
    for name, shapes in EDGE.items():
        groups = synth.make_custom(shapes, seed=zlib.crc32(name.encode()) % 100000, scale_codes=POW2_ALL)
        got, status = run_pow2(shapes, groups, tile_config=cfg, label=name)
        assert status == 0
        check_rows(shapes, groups, got)
        for (m, n, k, l), c in zip(shapes, got):
            if k == 0 and m and n:
                assert np.all(c == 0), "k = 0 must write zeros"


@pytest.mark.parametrize("split", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_pow2_k_tails(cfg, split):
    """k % 128 = 32, 64 and 96 (the last stage partly past k; for k % 64 == 32
    a half-used scale atom whose padding bytes are poisoned with the E4M3 NaN
    code, which must neither count nor be reported), whole tiles and stream-K."""
    shapes = [(97, 136, 32, 1), (129, 72, 96, 1), (33, 264, 160, 2), (256, 8, 224, 1), (40, 48, 192, 1),
              (200, 136, 4096 + 96, 1), (65, 64, 64, 1)]
    groups = synth.make_custom(shapes, seed=6464 + cfg, scale_codes=synth.POW2_SCALE_CODES)
    for (m, n, k, l), g in zip(shapes, groups):
        if k % 64 == 0:
            continue
        for key, rows in (("sfa", m), ("sfb", n)):
            all_rows = np.arange(-(-rows // 128) * 128)
            kb = np.array([k // 16, k // 16 + 1])
            for li in range(l):
                g[key][O.sf_offset(all_rows[:, None], kb[None, :], rows, k, li).reshape(-1)] = 0x7F
    got, status = run_pow2(shapes, groups, tile_config=cfg, split_mode=split, label="k tails")
    assert status == 0
    check_rows(shapes, groups, got)


@pytest.mark.parametrize("idx,split", [(2, -1), (3, -1), (4, -1), (2, 1), (4, 1)])
def test_pow2_full_workloads(idx, split):
    """The three large workloads at full size with power-of-two scales, in the
    plan the heuristic picks (and stream-K for workloads 2 and 4), checked on a
    sample of rows of every group (the first, the last and every 37th)."""
    shapes, groups = synth.make_workload(idx, scale_codes=synth.POW2_SCALE_CODES)
    got, status = run_pow2(shapes, groups, split_mode=split, label=f"workload {idx}")
    assert status == 0
    rows = [np.unique(np.r_[0, np.arange(5, m, 37), m - 1]) for (m, n, k, l) in shapes]
    check_rows(shapes, groups, got, rows=rows)


@pytest.mark.parametrize("code", [0x39, 0xB8, 0x7F, 0x80, 0x3F])
@pytest.mark.parametrize("side", ["sfa", "sfb"])
def test_pow2_status_reports_other_scales(code, side):
    """One scale outside the accepted set (1.125, -1, NaN, -0, 1.875) in a
    used position sets the status word; the same call without it leaves 0."""
    shapes = [(200, 264, 512, 1), (77, 136, 256, 1)]
    groups = synth.make_custom(shapes, seed=4242, scale_codes=synth.POW2_SCALE_CODES)
    _, status = run_pow2(shapes, groups, label="clean")
    assert status == 0
    m, n, k, _ = shapes[1]
    rows = m if side == "sfa" else n
    groups[1][side][O.sf_offset(np.array([rows - 1]), np.array([k // 16 - 1]), rows, k).reshape(-1)] = code
    _, status = run_pow2(shapes, groups, label=f"planted {code:#x} in {side}")
    assert status == 1


def test_pow2_matches_general_entry_point():
    """On power-of-two scales both entry points meet the oracle; their results
    differ by at most the fp32 summation order (compared to the same bound)."""
    shapes, groups = synth.make_workload(1, scale_codes=synth.POW2_SCALE_CODES)
    got, status = run_pow2(shapes, groups, label="workload 1")
    assert status == 0
    d = dev.upload(shapes, groups)
    dev.run(shapes, d)
    torch.cuda.synchronize()
    ref = O.grouped_gemm(shapes, groups)
    for a, b, r in zip(got, dev.c_as_numpy(shapes, d), ref):
        assert not O.tolerance_violations(a, b, r["s"]).any()


def test_pow2_graph_replay_matches_eager():
    """Captured calls of the power-of-two entry point (whole tiles, no
    workspace) write, replay after replay with eager work in between, exactly
    what the eager call wrote; the status word stays 0."""
    shapes, groups = synth.make_workload(1, scale_codes=synth.POW2_SCALE_CODES)
    announce("pow2 graph replay, workload 1")
    d = dev.upload(shapes, groups)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev.run_pow2(shapes, d, status)
    torch.cuda.synchronize()
    eager = [c.copy() for c in dev.c_as_numpy(shapes, d)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.run_pow2(shapes, d, status, stream=side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dev.run_pow2(shapes, d, status, stream=side)
    for _ in range(3):
        for dd in d:
            dd["c"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, dev.c_as_numpy(shapes, d)):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert int(status.item()) == 0


def test_pow2_status_and_scale_padding():
    """The status check sees the padding rows of the last scale atom only where
    they are converted: SFA padding in a 32-row block that also holds rows
    below m, and SFB padding (every block column of a tile is computed). A NaN
    code in SFA padding rows past m's last 32-row block is not read, so not
    reported, and the results stay correct either way."""
    shapes = [(33, 72, 256, 1)]
    base = synth.make_custom(shapes, seed=3333, scale_codes=synth.POW2_SCALE_CODES)
    m, n, k, _ = shapes[0]
    kb = np.arange(k // 16)
    cases = [("sfa", np.arange(64, 128), 0), ("sfa", np.array([40]), 1), ("sfb", np.array([100]), 1)]
    for key, pad_rows, expect in cases:
        groups = [dict(g, **{key: g[key].copy()}) for g in base]
        rows = m if key == "sfa" else n
        groups[0][key][O.sf_offset(pad_rows[:, None], kb[None, :], rows, k).reshape(-1)] = 0x7F
        got, status = run_pow2(shapes, groups, label=f"{key} padding rows {pad_rows[0]}..")
        assert status == expect, (key, pad_rows[0])
        check_rows(shapes, groups, got)
