"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every element must satisfy |C_gpu - C_ref| <= 2 ulp16(C_ref) + 1e-5 * S, with
S = sum_k |a*sfa*b*sfb| (infinities as +-65536, NaN never accepted). Padded
scale rows are poisoned with the E4M3 NaN code 0x7F, C is pre-filled with an
fp16 NaN pattern and surrounded by guard canaries, so unwritten, stray or
out-of-bounds stores show up.
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


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def poison_padding(shapes, groups):
    """Copy of ``groups`` with every padding scale byte set to 0x7F (E4M3 NaN):
    rows >= m (n) of the last 128-row atom, and, when k % 64 == 32, the two
    unused 16-blocks of every row's last 64-K atom."""
    out = []
    for (m, n, k, l), g in zip(shapes, groups):
        g = dict(g)
        for key, rows in (("sfa", m), ("sfb", n)):
            buf = np.array(g[key], dtype=np.uint8, copy=True)
            pad_rows = np.arange(rows, -(-rows // 128) * 128)
            all_rows = np.arange(-(-rows // 128) * 128)
            for li in range(l):
                if pad_rows.size and k:
                    kb = np.arange(k // 16)
                    buf[O.sf_offset(pad_rows[:, None], kb[None, :], rows, k, li).reshape(-1)] = 0x7F
                if k % 64 and all_rows.size:
                    kb = np.array([k // 16, k // 16 + 1])
                    buf[O.sf_offset(all_rows[:, None], kb[None, :], rows, k, li).reshape(-1)] = 0x7F
            g[key] = buf
        out.append(g)
    return out


def check(shapes, groups, tile_config=-1, label="", ref=None, split_mode=None):
    groups = poison_padding(shapes, groups)
    announce(f"{label} shapes={shapes} tile_config={tile_config} split_mode={split_mode}")
    d = dev.upload(shapes, groups, c_guard=GUARD)
    ws = None if split_mode is None else dev.workspace_for(shapes)
    dev.run(shapes, d, tile_config=tile_config, split_mode=split_mode, workspace=ws)
    torch.cuda.synchronize()
    got = dev.c_as_numpy(shapes, d)
    assert dev.guards_intact(d), "store outside C"
    if ref is None:
        ref = O.grouped_gemm(shapes, groups)
    for g, ((m, n, k, l), c, r) in enumerate(zip(shapes, got, ref)):
        if m == 0 or n == 0:
            continue
        bad = O.tolerance_violations(c, r["c16"], r["s"])
        if bad.any():
            idx = np.argwhere(bad)[:5]
            detail = [(tuple(i), float(c[tuple(i)]), float(r["c16"][tuple(i)]), float(r["s"][tuple(i)]))
                      for i in idx]
            pytest.fail(f"group {g} {shapes[g]}: {int(bad.sum())} of {bad.size} elements out of "
                        f"tolerance, e.g. {detail}")
    return got


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_workload_parity(idx):
    shapes, groups = synth.make_workload(idx)
    check(shapes, groups, label=f"workload {idx} ({synth.WORKLOADS[idx]['name']})")


EDGE_CASES = {
    "single_row": [(1, 8, 64, 1)],
    "ragged_m_n_k": [(127, 136, 192, 1), (129, 264, 320, 1)],
    "m257_n8": [(257, 8, 128, 1)],
    "empty_groups_in_middle": [(64, 64, 128, 1), (0, 64, 128, 1), (100, 128, 256, 1), (64, 0, 128, 1),
                               (33, 72, 64, 1)],
    "k_zero": [(40, 48, 0, 1), (16, 16, 64, 1)],
    "batch_l2": [(100, 136, 192, 2)],
    "g8_ragged": [(40, 4096, 256, 1), (401, 256, 128, 1), (7, 8, 64, 1), (128, 128, 128, 1),
                  (255, 520, 448, 1), (300, 200, 64, 1), (1, 1024, 512, 1), (96, 96, 960, 1)],
}


@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_edge_shapes(name):
    shapes = EDGE_CASES[name]
    groups = synth.make_custom(shapes, seed=zlib.crc32(name.encode()) % 100000)
    got = check(shapes, groups, label=f"edge {name}")
    for (m, n, k, l), c in zip(shapes, got):
        if k == 0 and m and n:
            assert np.all(c == 0), "k = 0 must write zeros"


@pytest.mark.parametrize("split", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_every_tile_config(cfg, split):
    """Each compiled tile configuration, with whole tiles and with stream-K."""
    if cfg >= mm.nvfp4_num_tile_configs():
        pytest.skip("config not compiled")
    for idx in (0, 1):
        shapes, groups = synth.make_workload(idx)
        check(shapes, groups, tile_config=cfg, split_mode=split, label=f"workload {idx}")
    for name in ("g8_ragged", "empty_groups_in_middle", "k_zero", "batch_l2"):
        shapes = EDGE_CASES[name]
        check(shapes, synth.make_custom(shapes, seed=77), tile_config=cfg, split_mode=split, label=name)


@pytest.mark.parametrize("split", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_half_atom_k(cfg, split):
    """k % 64 == 32: the last 64-K scale atom is half used and its other half
    (poisoned with NaN codes) must not count; the last stage holds 32 or 96
    valid K of 128, in the first or the second 64-K group; groups of one call
    mix k % 128 = 32, 96 and 0, and a long K splits over workgroups."""
    if cfg >= mm.nvfp4_num_tile_configs():
        pytest.skip("config not compiled")
    shapes = [(97, 136, 32, 1), (129, 72, 96, 1), (33, 264, 160, 2), (256, 8, 224, 1), (40, 48, 128, 1),
              (200, 136, 4096 + 96, 1)]
    check(shapes, synth.make_custom(shapes, seed=3232 + cfg), tile_config=cfg, split_mode=split,
          label="half-atom k")


@pytest.mark.parametrize("split", [0, 1])
@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_masked_row_blocks(cfg, split):
    """M tails that leave each wave 0 .. 4 active 32-row blocks in both wave rows
    (row blocks alternate between the wave rows; blocks wholly past m are
    skipped), and groups split into a full-row class and a lighter tail class."""
    if cfg >= mm.nvfp4_num_tile_configs():
        pytest.skip("config not compiled")
    shapes = [(m, 136, 384, 1) for m in (1, 33, 65, 97, 129, 161, 225)] + [(193, 72, 128, 2)]
    check(shapes, synth.make_custom(shapes, seed=31 + cfg), tile_config=cfg, split_mode=split,
          label="masked row blocks")


@pytest.mark.parametrize("idx", [2, 3, 4])
def test_streamk_full_workloads(idx):
    shapes, groups = synth.make_workload(idx)
    check(shapes, groups, split_mode=1, label=f"workload {idx} stream-K")


def test_default_entry_point_allocates_nothing_and_captures():
    """Few tiles with a long K: with a workspace the heuristic would split K
    over the grid, but the default entry point has none and allocates none, so
    it runs whole tiles, and a HIP graph captured around it replays to the
    oracle's result (eager work and synchronisation between the replays)."""
    shapes = [(256, 256, 16384, 1), (40, 136, 64, 1)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mm.nvfp4_launch_geometry(shapes, cus)["split"] == 1  # the plan with a workspace
    groups = poison_padding(shapes, synth.make_custom(shapes, seed=12))
    ref = O.grouped_gemm(shapes, groups)
    announce(f"default entry point, graph capture, shapes={shapes}")
    d = dev.upload(shapes, groups, c_guard=GUARD)
    abc, sf = dev.pointer_tables(d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mm.nvfp4_grouped_gemm(shapes, abc, sf, len(shapes), side)
    torch.cuda.synchronize()
    eager = [c.copy() for c in dev.c_as_numpy(shapes, d)]
    for c, r in zip(eager, ref):
        assert not O.tolerance_violations(c, r["c16"], r["s"]).any()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        mm.nvfp4_grouped_gemm(shapes, abc, sf, len(shapes), side)
    for rep in range(3):
        for dd in d:
            dd["c"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert dev.guards_intact(d)
        for a, b in zip(eager, dev.c_as_numpy(shapes, d)):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"replay {rep} differs"


def test_streamk_plans_share_a_workspace():
    """Stream-K calls with different tile configurations (so different grids
    and slot sizes) in a row on one stream share one caller workspace: the
    slots of one call overlap those of the call before, and each call's
    fold must read only partials its own workgroups wrote."""
    shapes = [(256, 256, 16384, 1), (40, 136, 64, 1)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = synth.make_custom(shapes, seed=21)
    ref = O.grouped_gemm(shapes, poison_padding(shapes, groups))
    for cfg in (0, 3, 1, 0):
        assert mm.nvfp4_launch_geometry(shapes, cus, cfg)["split"] == 1
        check(shapes, groups, tile_config=cfg, split_mode=-1, ref=ref, label=f"stream-K cfg {cfg} after others")


@pytest.mark.parametrize("cfg", [0, 2])
def test_streamk_workspace_reuse_across_inputs(cfg):
    """One workspace, filled with 0xFF bytes first, serves stream-K calls on
    two different inputs in turn. The counters start from whatever the
    workspace held (the clear kernel zeroes them), and each call must fold
    only partials that its own workgroups stored in that call: a partial left
    by the call before carries the other input's values."""
    shapes = [(300, 1024, 2048, 1), (77, 512, 4096, 1), (512, 256, 1024, 2)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert mm.nvfp4_launch_geometry(shapes, cus, cfg, 1)["split"] == 1
    inputs = [poison_padding(shapes, synth.make_custom(shapes, seed=s)) for s in (901, 902)]
    refs = [O.grouped_gemm(shapes, g) for g in inputs]
    devs = [dev.upload(shapes, g) for g in inputs]
    ws = dev.workspace_for(shapes)
    ws.fill_(0xFF)
    for rep, x in enumerate((0, 1, 0, 1, 1, 0)):
        announce(f"stream-K workspace reuse cfg {cfg} call {rep} input {x}")
        for dd in devs[x]:
            dd["c"].fill_(-1)
        dev.run(shapes, devs[x], tile_config=cfg, split_mode=1, workspace=ws)
        torch.cuda.synchronize()
        for c, r in zip(dev.c_as_numpy(shapes, devs[x]), refs[x]):
            assert not O.tolerance_violations(c, r["c16"], r["s"]).any(), f"call {rep} (input {x})"


def test_streamk_random_shapes_every_config():
    """Random group shapes (empty groups, ragged m, n and k, k % 64 = 32,
    batches) on every tile configuration with stream-K forced, through one
    workspace filled with 0xFF first: every result within the oracle's
    tolerance, and a repeat bitwise identical (the fold tree fixes the order
    of every addition)."""
    rng = np.random.default_rng(2024)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for case in range(30):
        shapes = [(int(rng.choice([0, 1, 7, 33, 64, 100, 128, 200, 255, 256, 300, 400])),
                   int(rng.choice([8, 64, 136, 256, 264, 512])),
                   int(rng.choice([32, 64, 96, 128, 256, 512, 1024, 2048, 4096])),
                   int(rng.choice([1, 1, 1, 2]))) for _ in range(int(rng.integers(1, 9)))]
        groups = synth.make_custom(shapes, seed=int(rng.integers(1 << 30)))
        ref = O.grouped_gemm(shapes, groups)
        for cfg in range(mm.nvfp4_num_tile_configs()):
            if mm.nvfp4_launch_geometry(shapes, cus, cfg, 1)["workspace_bytes"] > ws.numel():
                continue
            announce(f"stream-K random case {case} cfg {cfg} shapes={shapes}")
            d = dev.upload(shapes, groups)
            outs = []
            for _ in range(2):
                for dd in d:
                    dd["c"].fill_(-1)
                dev.run(shapes, d, tile_config=cfg, split_mode=1, workspace=ws)
                torch.cuda.synchronize()
                outs.append([c.copy() for c in dev.c_as_numpy(shapes, d)])
            for (m, n, k, l), a, b, r in zip(shapes, outs[0], outs[1], ref):
                if m and n:
                    assert not O.tolerance_violations(a, r["c16"], r["s"]).any(), (case, cfg, (m, n, k, l))
                    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (case, cfg, (m, n, k, l))


@pytest.mark.parametrize("split", [-1, 0])
def test_max_k(split):
    """The largest K the library accepts (2^22): fp32 accumulation over 4M
    products; with the heuristic and a workspace every workgroup contributes a
    range of stages to the one tile (stream-K), forced whole tiles run all
    32768 stages in one workgroup."""
    shapes = [(33, 24, 1 << 22, 1)]
    assert mm.nvfp4_grouped_gemm_validate(shapes, [(16, 16, 16)], [(16, 16)]) == mm.NVFP4_OK
    check(shapes, synth.make_custom(shapes, seed=4242), split_mode=split, label="k = 2^22")


def test_streamk_is_deterministic_and_workspace_rules():
    shapes, groups = synth.make_workload(1)
    announce("stream-K determinism workload 1")
    d = dev.upload(shapes, groups)
    ws = dev.workspace_for(shapes)
    outs = []
    for _ in range(3):
        for dd in d:
            dd["c"].fill_(0)
        dev.run(shapes, d, split_mode=1, workspace=ws)
        torch.cuda.synchronize()
        outs.append([c.copy() for c in dev.c_as_numpy(shapes, d)])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    tiny = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(mm.Nvfp4Error) as e:
        dev.run(shapes, d, split_mode=1, workspace=tiny)
    assert e.value.code == mm.NVFP4_ERR_WORKSPACE
    for dd in d:
        dd["c"].fill_(-1)
    dev.run(shapes, d, workspace=tiny)  # the heuristic falls back to whole tiles
    torch.cuda.synchronize()
    ref = O.grouped_gemm(shapes, groups)
    for c, r in zip(dev.c_as_numpy(shapes, d), ref):
        assert not O.tolerance_violations(c, r["c16"], r["s"]).any()


def test_full_e4m3_range_scales():
    """Subnormal, negative and large scales (every finite E4M3 code)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    shapes = [(70, 72, 256, 1), (130, 8, 64, 1)]
    groups = synth.make_custom(shapes, seed=5, scale_codes=finite)
    check(shapes, groups, label="full E4M3 range")


def test_repeat_is_bitwise_deterministic_and_streams():
    shapes, groups = synth.make_workload(1)
    announce("determinism workload 1")
    d = dev.upload(shapes, groups)
    dev.run(shapes, d)
    torch.cuda.synchronize()
    first = [c.copy() for c in dev.c_as_numpy(shapes, d)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for dd in d:
            dd["c"].fill_(0)
        dev.run(shapes, d, stream=side)
    side.synchronize()
    second = dev.c_as_numpy(shapes, d)
    for a, b in zip(first, second):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("idx,split", [(1, 0), (2, 0), (3, 0), (1, 1), (2, 1)])
def test_graph_replay_matches_eager(idx, split):
    """A call captured in a HIP graph and replayed several times, with eager
    work and synchronisation between the replays, writes exactly what the
    eager call writes. Whole tiles, and stream-K with a caller workspace (each
    replay's fold reads the partials of the same replay)."""
    shapes, groups = synth.make_workload(idx)
    announce(f"graph replay workload {idx} split {split}")
    d = dev.upload(shapes, groups)
    ws = dev.workspace_for(shapes) if split else None
    dev.run(shapes, d, split_mode=split, workspace=ws)
    torch.cuda.synchronize()
    eager = [c.copy() for c in dev.c_as_numpy(shapes, d)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.run(shapes, d, stream=side, split_mode=split, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dev.run(shapes, d, stream=side, split_mode=split, workspace=ws)
    for rep in range(3):
        for dd in d:
            dd["c"].fill_(-1)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, dev.c_as_numpy(shapes, d)):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"replay {rep} differs"


def test_empty_call_launches_nothing():
    announce("all-empty groups")
    shapes = [(0, 64, 64, 1), (64, 0, 64, 1)]
    groups = synth.make_custom(shapes, seed=1)
    d = dev.upload(shapes, groups)
    dev.run(shapes, d)
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(6))
def test_random_problems(seed):
    """Random calls (seeded): 1..8 groups, m in [0, 300], n a multiple of 8 up to
    320, k a multiple of 32 up to 640 (k % 64 == 32 and k = 0 included), l in
    {1, 2}; every tile configuration and split mode in turn, through the
    by-value and the device-table entry points."""
    rng = np.random.default_rng(9000 + seed)
    for call in range(4):
        g = int(rng.integers(1, 9))
        shapes = [(int(rng.integers(0, 301)), 8 * int(rng.integers(0, 41)), 32 * int(rng.integers(0, 21)),
                   int(rng.choice([1, 1, 1, 2]))) for _ in range(g)]
        cfg = int(rng.integers(0, mm.nvfp4_num_tile_configs()))
        split = [None, 0, 1][call % 3]
        groups = synth.make_custom(shapes, seed=int(rng.integers(1 << 30)))
        check(shapes, groups, tile_config=cfg, split_mode=split, label=f"random seed {seed} call {call}")
        groups = poison_padding(shapes, groups)
        d = dev.upload(shapes, groups, c_guard=GUARD)
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        dev.run_device(dev.device_tables(shapes, d), len(shapes), tile_config=cfg, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0 and dev.guards_intact(d)
        ref = O.grouped_gemm(shapes, groups)
        for (m, n, k, l), c, r in zip(shapes, dev.c_as_numpy(shapes, d), ref):
            if m and n:
                assert not O.tolerance_violations(c, r["c16"], r["s"]).any(), (m, n, k, l)


STAGE_CASES = [("workload", 1), ("workload", 2), ("workload", 3), ("workload", 4),
               ("edge", "g8_ragged"), ("edge", "ragged_m_n_k"), ("edge", "batch_l2"),
               ("edge", "empty_groups_in_middle")]


@pytest.mark.parametrize("split", [0, 1])
@pytest.mark.parametrize("kind,which", STAGE_CASES)
def test_three_stage_pipeline_is_bitwise_identical(kind, which, split):
    """The kernels with a three-stage LDS pipeline (each buffer reloaded one
    stage sooner after its last reads) write exactly what the four-stage ones
    write, for every tile configuration, whole tiles and stream-K: an LDS
    buffer overwritten before all its readers are done would differ."""
    if kind == "workload":
        shapes, groups = synth.make_workload(which)
    else:
        shapes = EDGE_CASES[which]
        groups = synth.make_custom(shapes, seed=zlib.crc32(which.encode()) % 100000)
    groups = poison_padding(shapes, groups)
    d = dev.upload(shapes, groups, c_guard=GUARD)
    abc, sf = dev.pointer_tables(d)
    ws = dev.workspace_for(shapes)
    for cfg in range(mm.nvfp4_num_tile_configs()):
        outs = []
        for stages in (4, 3):
            announce(f"{kind} {which} cfg {cfg} split {split} stages {stages}")
            for dd in d:
                dd["c"].fill_(-1)
            mm.nvfp4_grouped_gemm_stages(shapes, abc, sf, len(shapes), ws.data_ptr(), ws.numel(), cfg, split,
                                         stages, torch.cuda.current_stream())
            torch.cuda.synchronize()
            assert dev.guards_intact(d)
            outs.append([c.copy() for c in dev.c_as_numpy(shapes, d)])
        for (m, n, k, l), a, b in zip(shapes, *outs):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (cfg, (m, n, k, l))


def test_three_stage_pipeline_half_atom_k():
    """The same check on k % 64 == 32 groups (the padding 16-blocks zeroed in
    LDS between the loads of a stage and its readers)."""
    shapes = [(97, 136, 32, 1), (129, 72, 96, 1), (33, 264, 160, 2), (256, 8, 224, 1), (200, 136, 4096 + 96, 1)]
    groups = poison_padding(shapes, synth.make_custom(shapes, seed=3737))
    d = dev.upload(shapes, groups, c_guard=GUARD)
    abc, sf = dev.pointer_tables(d)
    ws = dev.workspace_for(shapes)
    ref = O.grouped_gemm(shapes, groups)
    for cfg in range(mm.nvfp4_num_tile_configs()):
        for split in (0, 1):
            outs = []
            for stages in (4, 3):
                announce(f"half-atom k cfg {cfg} split {split} stages {stages}")
                for dd in d:
                    dd["c"].fill_(-1)
                mm.nvfp4_grouped_gemm_stages(shapes, abc, sf, len(shapes), ws.data_ptr(), ws.numel(), cfg, split,
                                             stages, torch.cuda.current_stream())
                torch.cuda.synchronize()
                outs.append([c.copy() for c in dev.c_as_numpy(shapes, d)])
            for a, b, r in zip(*outs, ref):
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (cfg, split)
                assert not O.tolerance_violations(b, r["c16"], r["s"]).any()


def test_one_row_block_tiles_every_config():
    """Tiles with at most 32 rows below m (the whole-tile kernels then put
    the four waves side by side along n on that one row block): against the
    oracle, and bitwise against the three-stage kernels, which keep the
    two-by-two wave layout for every tile. m tails of 1 .. 32 rows on every
    tile height, n tails that leave some waves' columns wholly past n, and a
    half-used last scale atom."""
    shapes = [(1, 136, 384, 1), (17, 264, 256, 1), (32, 512, 384, 1), (133, 40, 384, 1), (160, 328, 256, 2),
              (280, 264, 384, 1), (288, 72, 96, 1), (257, 520, 160, 1)]
    groups = poison_padding(shapes, synth.make_custom(shapes, seed=4141))
    d = dev.upload(shapes, groups, c_guard=GUARD)
    abc, sf = dev.pointer_tables(d)
    ws = dev.workspace_for(shapes)
    ref = O.grouped_gemm(shapes, groups)
    for cfg in range(mm.nvfp4_num_tile_configs()):
        outs = []
        for stages in (4, 3):
            announce(f"one-row-block tiles cfg {cfg} stages {stages}")
            for dd in d:
                dd["c"].fill_(-1)
            mm.nvfp4_grouped_gemm_stages(shapes, abc, sf, len(shapes), ws.data_ptr(), ws.numel(), cfg, 0,
                                         stages, torch.cuda.current_stream())
            torch.cuda.synchronize()
            assert dev.guards_intact(d), "store outside C"
            outs.append([c.copy() for c in dev.c_as_numpy(shapes, d)])
        for shape, a, b, r in zip(shapes, *outs, ref):
            assert not O.tolerance_violations(a, r["c16"], r["s"]).any(), (cfg, shape)
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (cfg, shape)


def config_of(bm, bn):
    return next(c for c in range(mm.nvfp4_num_tile_configs())
                if (mm.nvfp4_tile_config_info(c)["bm"], mm.nvfp4_tile_config_info(c)["bn"]) == (bm, bn))


@pytest.mark.parametrize("tile", [(256, 128), (128, 256), (128, 128)])
def test_long_k_split_over_waves(tile):
    """Calls whose groups all have at least 32 stages run the 256x128,
    128x256 and 128x128 kernels that split K over the waves in every tile:
    against the oracle, and bitwise against their three-stage counterpart.
    Row counts give every number of row blocks below m (1-8) and several tile
    rows; two groups have k % 64 == 32, one of them k = 4000 (32 stages, the
    shortest K that selects these kernels)."""
    cfg = config_of(*tile)
    shapes = [(300, 264, 4096, 1), (129, 136, 4160, 1), (33, 72, 4128, 1), (256, 128, 4096, 2), (511, 8, 4000, 1),
              (200, 392, 4096, 1), (1, 128, 4096, 1), (97, 520, 4096, 1)]
    assert mm.nvfp4_splits_k_over_waves(shapes, torch.cuda.get_device_properties(0).multi_processor_count, cfg, 0)
    groups = poison_padding(shapes, synth.make_custom(shapes, seed=4242))
    d = dev.upload(shapes, groups, c_guard=GUARD)
    abc, sf = dev.pointer_tables(d)
    ws = dev.workspace_for(shapes)
    ref = O.grouped_gemm(shapes, groups)
    outs = []
    for stages in (4, 3):
        announce(f"long-k split over waves cfg {cfg} stages {stages}")
        for dd in d:
            dd["c"].fill_(-1)
        mm.nvfp4_grouped_gemm_stages(shapes, abc, sf, len(shapes), ws.data_ptr(), ws.numel(), cfg, 0, stages,
                                     torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert dev.guards_intact(d), "store outside C"
        outs.append([c.copy() for c in dev.c_as_numpy(shapes, d)])
    for shape, a, b, r in zip(shapes, *outs, ref):
        assert not O.tolerance_violations(a, r["c16"], r["s"]).any(), shape
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), shape


@pytest.mark.parametrize("tile", [(256, 128), (128, 256), (128, 128)])
@pytest.mark.parametrize("seed", range(3))
def test_random_long_k_split_over_waves(seed, tile):
    """Random long-K calls on the 256x128, 128x256 and 128x128 tiles (seeded):
    every group with work has at least 32 stages, so whole tiles run the
    kernels that split K over the waves in every tile; m in [0, 600] (several
    tile rows, any row blocks below m), n a multiple of 8 up to 264, k in
    {4000, 4096, 4128, 4160, 4224}, l in {1, 2} (k = 0 groups included, which
    do not count against the choice). Against the oracle, and stream-K on the
    same call for comparison."""
    cfg = config_of(*tile)
    rng = np.random.default_rng(7700 + seed)
    g = int(rng.integers(2, 9))
    shapes = [(int(rng.integers(0, 601)), 8 * int(rng.integers(1, 34)), int(rng.choice([4000, 4096, 4128, 4160, 4224])),
               int(rng.choice([1, 1, 2]))) for _ in range(g)]
    shapes[-1] = (shapes[-1][0], shapes[-1][1], 0, 1) if seed == 2 else shapes[-1]
    assert mm.nvfp4_splits_k_over_waves(shapes, torch.cuda.get_device_properties(0).multi_processor_count, cfg, 0)
    groups = synth.make_custom(shapes, seed=int(rng.integers(1 << 30)))
    ref = O.grouped_gemm(shapes, poison_padding(shapes, groups))
    for split in (0, 1):
        check(shapes, groups, tile_config=cfg, split_mode=split, ref=ref, label=f"random long k seed {seed}")
