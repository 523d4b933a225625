"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and its host-side logic (argument validation, tile geometry, sizes) behaves as
the header states. No compute call is made (no GPU needed)."""
import ctypes
import os
import re

import pytest

import moe_matmul_amd as mm
from moe_matmul_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_grouped_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mm.load_library()
    names = declared_functions()
    assert "nvfp4_grouped_gemm" in names and len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    # every exported nvfp4_ symbol of the binary is declared (nothing undocumented)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mm.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r"\bT (nvfp4_\w+)", out)))
    assert exported == names


def _ptrs(g, base=0x10000):
    abc = [(base + 0x1000 * i, base + 0x2000 * i + 0x100000, base + 0x3000 * i + 0x200000) for i in range(g)]
    sf = [(base + 0x4000 * i + 0x300000, base + 0x5000 * i + 0x400000) for i in range(g)]
    return abc, sf


def test_validate_accepts_workloads():
    for idx in range(5):
        shapes = synth.workload_shapes(idx)
        abc, sf = _ptrs(len(shapes))
        assert mm.nvfp4_grouped_gemm_validate(shapes, abc, sf) == mm.NVFP4_OK


@pytest.mark.parametrize("shapes,code", [
    ([(128, 128, 48, 1)], mm.NVFP4_ERR_INVALID),        # k % 32
    ([(128, 100, 128, 1)], mm.NVFP4_ERR_INVALID),       # n % 8
    ([(-1, 128, 128, 1)], mm.NVFP4_ERR_INVALID),
    ([(128, -8, 128, 1)], mm.NVFP4_ERR_INVALID),
    ([(128, 128, -64, 1)], mm.NVFP4_ERR_INVALID),
    ([(128, 128, 128, 0)], mm.NVFP4_ERR_INVALID),       # l >= 1
    ([(128, 128, 1 << 23, 1)], mm.NVFP4_ERR_INVALID),   # k <= 2^22
    ([(1 << 20, 128, 4096, 1)], mm.NVFP4_ERR_INVALID),  # A bytes >= 2^31
])
def test_validate_rejects_bad_sizes(shapes, code):
    abc, sf = _ptrs(len(shapes))
    assert mm.nvfp4_grouped_gemm_validate(shapes, abc, sf) == code


def test_validate_group_count_and_nulls():
    lib = mm.load_library()
    shapes = [(64, 64, 64, 1)] * 9
    abc, sf = _ptrs(9)
    assert mm.nvfp4_grouped_gemm_validate(shapes, abc, sf, 9) == mm.NVFP4_ERR_INVALID
    assert mm.nvfp4_grouped_gemm_validate(shapes[:1], abc[:1], sf[:1], 0) == mm.NVFP4_ERR_INVALID
    null = ctypes.POINTER(ctypes.c_int32)()
    assert lib.nvfp4_grouped_gemm_validate(null, None, None, 1) == mm.NVFP4_ERR_INVALID
    for col in range(3):
        abc2 = [list(r) for r in abc[:1]]
        abc2[0][col] = 0
        assert mm.nvfp4_grouped_gemm_validate(shapes[:1], abc2, sf[:1]) == mm.NVFP4_ERR_INVALID
    for col in range(2):
        sf2 = [list(r) for r in sf[:1]]
        sf2[0][col] = 0
        assert mm.nvfp4_grouped_gemm_validate(shapes[:1], abc[:1], sf2) == mm.NVFP4_ERR_INVALID


def test_validate_alignment():
    shapes = [(64, 64, 64, 1)]
    abc, sf = _ptrs(1)
    for col in range(3):
        abc2 = [list(abc[0])]
        abc2[0][col] += 8
        assert mm.nvfp4_grouped_gemm_validate(shapes, abc2, sf) == mm.NVFP4_ERR_MISALIGNED
    for col in range(2):
        sf2 = [list(sf[0])]
        sf2[0][col] += 4
        assert mm.nvfp4_grouped_gemm_validate(shapes, abc, sf2) == mm.NVFP4_ERR_MISALIGNED


def test_validate_accepts_half_atom_k():
    """k % 64 == 32 (the last 64-K scale atom half used) is accepted, k % 32 != 0 is not."""
    abc, sf = _ptrs(1)
    for k in (32, 96, 160, 7168 + 32):
        assert mm.nvfp4_grouped_gemm_validate([(64, 64, k, 1)], abc, sf) == mm.NVFP4_OK, k
        assert mm.nvfp4_device_group_tiles((64, 64, k, 1), _group_ptrs()) == 1, k
    for k in (16, 48, 80, 112):
        assert mm.nvfp4_grouped_gemm_validate([(64, 64, k, 1)], abc, sf) == mm.NVFP4_ERR_INVALID, k
        assert mm.nvfp4_device_group_tiles((64, 64, k, 1), _group_ptrs()) == -1, k


def test_validate_edge_semantics():
    abc, sf = _ptrs(3)
    # empty groups may carry null pointers; k = 0 needs only C
    assert mm.nvfp4_grouped_gemm_validate([(0, 64, 64, 1), (64, 0, 64, 1), (8, 8, 64, 1)],
                                          [(0, 0, 0), (0, 0, 0), abc[2]], [(0, 0), (0, 0), sf[2]]) == mm.NVFP4_OK
    assert mm.nvfp4_grouped_gemm_validate([(8, 8, 0, 1)], [(0, 0, abc[0][2])], [(0, 0)]) == mm.NVFP4_OK
    assert mm.nvfp4_grouped_gemm_validate([(8, 8, 0, 1)], [(0, 0, 0)], [(0, 0)]) == mm.NVFP4_ERR_INVALID


def test_compute_call_validates_before_any_hip_call():
    # an invalid call must fail in validation (no device needed)
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm([(128, 100, 128, 1)], *_ptrs(1))
    assert e.value.code == mm.NVFP4_ERR_INVALID
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_config([(128, 128, 128, 1)], *_ptrs(1), tile_config=99)
    assert e.value.code in (mm.NVFP4_ERR_CONFIG,)


def test_num_groups_beyond_the_tables_is_refused():
    """A group count larger than the rows of any argument table would make the
    library read host memory past the marshalled arrays: the binding refuses
    it before calling C, for pre-marshalled arrays too."""
    shapes = [(64, 64, 64, 1)] * 2
    abc, sf = _ptrs(2)
    ps, pabc, psf = mm.prepare(problem_sizes=shapes, ptrs_abc=abc, ptrs_sfa_sfb=sf)
    calls = [
        lambda g: mm.nvfp4_grouped_gemm_validate(shapes, abc, sf, g),
        lambda g: mm.nvfp4_grouped_gemm_validate(ps, pabc, psf, g),
        lambda g: mm.nvfp4_grouped_gemm_validate(shapes, abc[:1], sf, g),
        lambda g: mm.nvfp4_grouped_gemm_validate(shapes, abc, sf[:1], g),
        lambda g: mm.nvfp4_grouped_gemm(shapes, abc, sf, g),
        lambda g: mm.nvfp4_grouped_gemm_config(ps, pabc, psf, g, None, 0),
        lambda g: mm.nvfp4_grouped_gemm_ex(shapes, abc, sf, g),
        lambda g: mm.nvfp4_grouped_gemm_stages(shapes, abc, sf, g, stages=3),
        lambda g: mm.nvfp4_grouped_gemm_pow2(shapes, abc, sf, 0x10000, g),
        lambda g: mm.nvfp4_launch_geometry(shapes, 256, num_groups=g),
        lambda g: mm.nvfp4_select_tile_config(shapes, 256, num_groups=g),
        lambda g: mm.nvfp4_workspace_bytes(shapes, 256, num_groups=g),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError):
            call(3 if i not in (2, 3) else 2)
    # fewer groups than rows is fine (only the first rows are read)
    assert mm.nvfp4_grouped_gemm_validate(ps, pabc, psf, 1) == mm.NVFP4_OK


def test_stages_entry_point_checks_before_any_hip_call():
    shapes = [(128, 128, 128, 1)]
    for stages in (0, 2, 5):
        with pytest.raises(mm.Nvfp4Error) as e:
            mm.nvfp4_grouped_gemm_stages(shapes, *_ptrs(1), stages=stages)
        assert e.value.code == mm.NVFP4_ERR_CONFIG
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_stages([(128, 100, 128, 1)], *_ptrs(1), stages=3)
    assert e.value.code == mm.NVFP4_ERR_INVALID
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_stages(shapes, *_ptrs(1), workspace=0x1010, workspace_bytes=1 << 20, stages=3)
    assert e.value.code == mm.NVFP4_ERR_MISALIGNED


def test_sf_bytes_matches_atom_padding():
    for rows, k, l in [(1, 64, 1), (128, 256, 1), (129, 64, 2), (300, 7168, 1), (0, 64, 1), (5, 0, 1)]:
        assert mm.nvfp4_sf_bytes(rows, k, l) == synth.sf_buffer_bytes(rows, k, l)
    assert mm.nvfp4_sf_bytes(-1, 64, 1) == 0


def test_tile_configs_and_geometry():
    n = mm.nvfp4_num_tile_configs()
    assert n >= 1
    for c in range(n):
        info = mm.nvfp4_tile_config_info(c)
        # whole 128-row scale atoms, or 64 rows (half of one)
        assert info["bm"] in (64, 128, 256) and info["bn"] in (64, 128, 256) and info["threads"] == 256
    with pytest.raises(mm.Nvfp4Error):
        mm.nvfp4_tile_config_info(n)
    shapes = synth.workload_shapes(2)
    for c in range(n):
        info = mm.nvfp4_tile_config_info(c)
        expect = sum(-(-m // info["bm"]) * -(-nn // info["bn"]) * l for (m, nn, k, l) in shapes)
        units = sum(-(-m // info["bm"]) * -(-nn // info["bn"]) * l * -(-k // 128) for (m, nn, k, l) in shapes)
        geo = mm.nvfp4_launch_geometry(shapes, 256, c, 0)
        assert geo["config"] == c and geo["total_tiles"] == expect and geo["grid"] == min(expect, 256)
        assert geo["split"] == 0 and geo["workspace_bytes"] == 0
        geo = mm.nvfp4_launch_geometry(shapes, 256, c, 1)
        assert geo["split"] == 1 and geo["grid"] == min(units, 256)
        # two fp32 tile slots and 10 int32 fold-tree counters per slot per workgroup (padded to 256 bytes)
        counters = -(-geo["grid"] * 2 * 10 * 4 // 256) * 256
        assert geo["workspace_bytes"] == geo["grid"] * 2 * info["bm"] * info["bn"] * 4 + counters
        assert mm.nvfp4_workspace_bytes(shapes, 256) >= geo["workspace_bytes"]
    # empty groups own no tiles, wherever they sit
    geo = mm.nvfp4_launch_geometry([(0, 128, 64, 1), (128, 128, 64, 1), (128, 0, 64, 1)], 256, 0, 0)
    assert geo["total_tiles"] == 1
    with pytest.raises(mm.Nvfp4Error):
        mm.nvfp4_launch_geometry(shapes, 256, 0, 2)
    sel = mm.nvfp4_select_tile_config(synth.workload_shapes(4), 256)
    assert 0 <= sel < n
    # the two small workloads fill more compute units with 64x64 tiles
    small = next(c for c in range(n) if (mm.nvfp4_tile_config_info(c)["bm"], mm.nvfp4_tile_config_info(c)["bn"]) == (64, 64))
    for idx in (0, 1):
        assert mm.nvfp4_select_tile_config(synth.workload_shapes(idx), 256) == small


def test_k_split_over_waves_choice():
    """Calls run the kernels that split K over the waves in every tile when
    they take whole tiles of a 256x128, 128x256 or 128x128 configuration and
    every group with work has at least 32 stages of 128 K (k > 3968); groups
    with m, n or k = 0 do not count, stream-K plans and the other
    configurations never do."""
    n = mm.nvfp4_num_tile_configs()
    shape_of = {(mm.nvfp4_tile_config_info(c)["bm"], mm.nvfp4_tile_config_info(c)["bn"]): c for c in range(n)}
    split_cfgs = [shape_of[s] for s in ((256, 128), (128, 256), (128, 128))]
    other_cfgs = [c for c in range(n) if c not in split_cfgs]
    long_k = [(300, 264, 4096, 1), (129, 136, 4000, 1), (33, 72, 7168, 2)]
    for c in split_cfgs:
        assert mm.nvfp4_splits_k_over_waves(long_k, 256, c, 0)
        assert not mm.nvfp4_splits_k_over_waves(long_k, 256, c, 1)
        # 31 stages in one group: no
        assert not mm.nvfp4_splits_k_over_waves(long_k + [(8, 8, 3968, 1)], 256, c, 0)
        # the shortest K that counts: 32 stages (k = 3969 is not a valid k; 4000 is)
        assert mm.nvfp4_splits_k_over_waves([(64, 64, 4000, 1)], 256, c, 0)
        # empty groups of short K do not count
        for empty in ((0, 64, 64, 1), (64, 0, 64, 1), (64, 64, 0, 1)):
            assert mm.nvfp4_splits_k_over_waves(long_k + [empty], 256, c, 0), empty
    for c in other_cfgs:
        assert not mm.nvfp4_splits_k_over_waves(long_k, 256, c, 0)
    # the heuristic's plan for the benchmark workloads: only the long-K MoE workload
    assert [mm.nvfp4_splits_k_over_waves(synth.workload_shapes(i), 256) for i in range(5)] == [
        False, False, True, False, False]
    with pytest.raises(mm.Nvfp4Error):
        mm.nvfp4_splits_k_over_waves(long_k, 256, n, 0)
    with pytest.raises(mm.Nvfp4Error):
        mm.nvfp4_splits_k_over_waves([(64, 64, 48, 1)], 256)  # k not a multiple of 32


def test_split_plan_covers_every_unit_once():
    """Stream-K plans: whole rounds of one tile per workgroup, then contiguous
    (possibly empty) unit ranges in workgroup order that cover exactly the
    units of the remaining tiles."""
    for idx in (1, 2, 3, 4):
        shapes = synth.workload_shapes(idx)
        for cfg in range(mm.nvfp4_num_tile_configs()):
            info = mm.nvfp4_tile_config_info(cfg)
            tiles = sum(-(-m // info["bm"]) * -(-n // info["bn"]) * l for (m, n, k, l) in shapes)
            units = sum(-(-m // info["bm"]) * -(-n // info["bn"]) * l * -(-k // 128) for (m, n, k, l) in shapes)
            whole, r = mm.nvfp4_split_plan(shapes, 256, cfg)
            grid = len(r) - 1
            assert grid == mm.nvfp4_launch_geometry(shapes, 256, cfg, 1)["grid"] == min(units, 256)
            assert whole % grid == 0 and 0 <= whole <= tiles
            # the whole tiles hold r[0] units: whole * nk when every group has the same k
            nks = [-(-k // 128) for (m, n, k, l) in shapes]
            assert min(nks) * whole <= r[0] <= max(nks) * whole and r[-1] == units
            if len(set(nks)) == 1:
                assert r[0] == whole * nks[0]
            assert all(a <= b for a, b in zip(r, r[1:]))
            if whole == 0:
                assert all(a < b for a, b in zip(r, r[1:]))  # without whole rounds no range is empty
    # a long K on few tiles: no whole round, one unit (128-K stage) per workgroup
    whole, r = mm.nvfp4_split_plan([(256, 256, 16384, 1), (40, 136, 64, 1)], 256, 0)
    assert whole == 0 and r == list(range(130))  # 128 + 1 units on 129 workgroups
    with pytest.raises(mm.Nvfp4Error):
        mm.nvfp4_split_plan([(0, 128, 256, 1)], 256, 0)  # no units to split


def test_ex_entry_point_checks_before_any_hip_call():
    shapes = [(128, 128, 128, 1)]
    abc, sf = _ptrs(1)
    with pytest.raises(mm.Nvfp4Error) as e:  # workspace not 256-byte aligned
        mm.nvfp4_grouped_gemm_ex(shapes, abc, sf, workspace=0x10010, workspace_bytes=1 << 20)
    assert e.value.code == mm.NVFP4_ERR_MISALIGNED
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_ex(shapes, abc, sf, split_mode=3)
    assert e.value.code == mm.NVFP4_ERR_CONFIG
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_ex([(128, 100, 128, 1)], abc, sf)
    assert e.value.code == mm.NVFP4_ERR_INVALID


def test_pow2_entry_point_checks_before_any_hip_call():
    """nvfp4_grouped_gemm_pow2: a status word is required (non-null, 4-byte
    aligned); then the checks of nvfp4_grouped_gemm_ex apply."""
    shapes = [(128, 128, 128, 1)]
    abc, sf = _ptrs(1)
    cases = [(dict(d_status=0), mm.NVFP4_ERR_INVALID),
             (dict(d_status=0x10002), mm.NVFP4_ERR_MISALIGNED),
             (dict(d_status=0x10000, workspace=0x10010, workspace_bytes=1 << 20), mm.NVFP4_ERR_MISALIGNED),
             (dict(d_status=0x10000, split_mode=3), mm.NVFP4_ERR_CONFIG),
             (dict(d_status=0x10000, tile_config=9), mm.NVFP4_ERR_CONFIG)]
    for kw, code in cases:
        with pytest.raises(mm.Nvfp4Error) as e:
            mm.nvfp4_grouped_gemm_pow2(shapes, abc, sf, **kw)
        assert e.value.code == code, kw
    with pytest.raises(mm.Nvfp4Error) as e:
        mm.nvfp4_grouped_gemm_pow2([(128, 100, 128, 1)], abc, sf, d_status=0x10000)
    assert e.value.code == mm.NVFP4_ERR_INVALID


def test_error_strings():
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(mm.nvfp4_error_string(code), str)


@pytest.mark.parametrize("shapes", [
    [(1 << 30, 1 << 10, 64, 1 << 30)],      # m*(k/2)*l would overflow int64
    [(1 << 20, 1 << 20, 64, 1 << 25)],      # m*n*l would overflow int64
    [(64, 64, 1 << 22, (1 << 31) - 1)],     # huge l
])
def test_validate_rejects_overflowing_products(shapes):
    abc, sf = _ptrs(len(shapes))
    assert mm.nvfp4_grouped_gemm_validate(shapes, abc, sf) == mm.NVFP4_ERR_INVALID


def _group_ptrs(base=0x100000):
    return [base, base + 0x1000, base + 0x2000, base + 0x3000, base + 0x4000]  # A, B, C, SFA, SFB


def test_device_group_check_matches_host_rules():
    """The per-group check the device-table kernel runs (host copy): the tiles
    it gives a valid group, and -1 for every size or pointer rule the host
    validation enforces."""
    p = _group_ptrs()
    for cfg in range(mm.nvfp4_num_tile_configs()):
        info = mm.nvfp4_tile_config_info(cfg)
        for (m, n, k, l) in [(300, 4096, 7168, 1), (1, 8, 64, 1), (129, 136, 0, 2), (0, 64, 64, 1), (64, 0, 64, 1)]:
            want = 0 if m == 0 or n == 0 else -(-m // info["bm"]) * -(-n // info["bn"]) * l
            assert mm.nvfp4_device_group_tiles((m, n, k, l), p, cfg) == want
    default = mm.nvfp4_tile_config_info(0)  # the device-table entry point's default: 256x256
    assert mm.nvfp4_device_group_tiles((300, 512, 64, 1), p) == -(-300 // default["bm"]) * -(-512 // default["bn"])
    bad_sizes = [(128, 128, 80, 1), (128, 100, 128, 1), (-1, 128, 128, 1), (128, -8, 128, 1), (128, 128, -64, 1),
                 (128, 128, 128, 0), (128, 128, 1 << 23, 1), (1 << 20, 128, 4096, 1), (64, 64, 1 << 22, (1 << 31) - 1),
                 (1 << 20, 1 << 20, 64, 1 << 25), ((1 << 30) + 1, 8, 64, 1),
                 ((1 << 17) + 128, 1 << 17, 64, 1)]  # more than 2^20 tiles of 128x128
    for sz in bad_sizes:
        abc = [(p[0], p[1], p[2])]
        host = mm.nvfp4_grouped_gemm_validate([sz], abc, [(p[3], p[4])])
        assert mm.nvfp4_device_group_tiles(sz, p) == -1, sz
        if sz != ((1 << 17) + 128, 1 << 17, 64, 1):
            assert host == mm.NVFP4_ERR_INVALID, sz
    assert mm.nvfp4_device_group_tiles((1 << 17, 1 << 17, 64, 1), p) > 0  # exactly 2^20 tiles of 128x128
    for i in range(5):  # null or misaligned A, B, C, SFA, SFB
        for v in (0, p[i] + 8):
            q = list(p)
            q[i] = v
            assert mm.nvfp4_device_group_tiles((64, 64, 64, 1), q) == -1
            # k = 0 needs only C; empty groups need nothing
            assert mm.nvfp4_device_group_tiles((64, 64, 0, 1), q) == (-1 if i == 2 else 1)
            assert mm.nvfp4_device_group_tiles((0, 64, 64, 1), q) == 0
    assert mm.nvfp4_device_group_tiles((64, 64, 64, 1), p, 99) == -1


def test_device_entry_point_checks_before_any_hip_call():
    lib = mm.load_library()
    ok = 0x100000
    cases = [
        ((ok, ok, ok, 0, -1, 0), mm.NVFP4_ERR_INVALID),                      # no groups
        ((ok, ok, ok, mm.NVFP4_MAX_DEVICE_GROUPS + 1, -1, 0), mm.NVFP4_ERR_INVALID),
        ((0, ok, ok, 8, -1, 0), mm.NVFP4_ERR_INVALID),                       # null tables
        ((ok, 0, ok, 8, -1, 0), mm.NVFP4_ERR_INVALID),
        ((ok, ok, 0, 8, -1, 0), mm.NVFP4_ERR_INVALID),
        ((ok + 8, ok, ok, 8, -1, 0), mm.NVFP4_ERR_MISALIGNED),               # tables 16-byte aligned
        ((ok, ok + 8, ok, 8, -1, 0), mm.NVFP4_ERR_MISALIGNED),
        ((ok, ok, ok + 8, 8, -1, 0), mm.NVFP4_ERR_MISALIGNED),
        ((ok, ok, ok, 8, -1, ok + 2), mm.NVFP4_ERR_MISALIGNED),              # status 4-byte aligned
        ((ok, ok, ok, 8, mm.nvfp4_num_tile_configs(), 0), mm.NVFP4_ERR_CONFIG),
        ((ok, ok, ok, 8, -2, 0), mm.NVFP4_ERR_CONFIG),
    ]
    for (ps, abc, sf, g, cfg, status), code in cases:
        rc = lib.nvfp4_grouped_gemm_device(ps, abc, sf, g, cfg, status, None)
        assert rc == code, (ps, abc, sf, g, cfg, status, rc)


def test_plan_cache_returns_the_plan_of_the_sizes_asked_for():
    """Plans are cached per thread by sizes (and compute units and forced
    choices): interleaving many different size sets (more than the cache holds)
    must return the same geometry as each set's first answer."""
    sets = [synth.workload_shapes(i) for i in range(5)]
    sets += [[(m, 136, 256, 1)] for m in (1, 33, 129, 300, 1000)]
    sets += [[(64, 64, 64, l)] for l in (1, 2, 3)]
    first = {}
    for rep in range(3):
        for i, shapes in enumerate(sets):
            for cus in (256, 80):
                for cfg, split in ((-1, -1), (0, 1), (3, 0)):
                    geo = mm.nvfp4_launch_geometry(shapes, cus, cfg, split)
                    key = (i, cus, cfg, split)
                    if rep == 0:
                        first[key] = geo
                    assert geo == first[key], key
    # the two group counts sharing a prefix of sizes are different problems
    a = mm.nvfp4_launch_geometry([(256, 256, 1024, 1)], 256, 0, 0)
    b = mm.nvfp4_launch_geometry([(256, 256, 1024, 1), (256, 256, 1024, 1)], 256, 0, 0)
    assert a["total_tiles"] == 1 and b["total_tiles"] == 2


def test_probe_library_exports_every_declared_symbol():
    """The measurement library (libnvfp4_mainloop_probe.so) exports exactly what
    include/nvfp4_mainloop_probe.h declares."""
    import subprocess

    from moe_matmul_amd import probe
    text = open(os.path.join(ROOT, "include", "nvfp4_mainloop_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))
    assert "nvfp4_probe_mainloop" in names
    lib = probe.load_probe_library()
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", probe.PROBE_LIB_PATH], capture_output=True, text=True).stdout
    assert sorted(set(re.findall(r"\bT (nvfp4_\w+)", out))) == names
    # argument checks run before any HIP call
    assert lib.nvfp4_probe_mainloop(11, 1, 1, 0x1000, None) == -1
    assert lib.nvfp4_probe_mainloop(0, 0, 1, 0x1000, None) == -1
    assert lib.nvfp4_probe_mainloop(0, 1, 1, None, None) == -1
    assert lib.nvfp4_probe_cvt_scale(None, 1, None, None) == -1
    assert lib.nvfp4_probe_cvt_scale(None, 0, None, None) == 0
    assert probe.nvfp4_probe_flops_per_iteration(0) == 2 * probe.nvfp4_probe_flops_per_iteration(1)
