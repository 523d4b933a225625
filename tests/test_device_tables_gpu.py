"""GPU parity of nvfp4_grouped_gemm_device (group tables in device memory, up
to 512 groups) against the CPU oracle, and against the by-value entry point.

Tolerance as in test_parity_gpu: |C_gpu - C_ref| <= 2 ulp16(C_ref) + 1e-5 * S.
The by-value entry point with whole tiles of the same configuration computes
every tile with the same code and the same K order, so the two agree bit for
bit. Rejected groups must leave C (pre-filled with an fp16 NaN pattern)
untouched; every C sits between guard canaries.
"""
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


def check_against_oracle(shapes, groups, got, skip=()):
    ref = O.grouped_gemm(shapes, groups)
    for g, ((m, n, k, l), c, r) in enumerate(zip(shapes, got, ref)):
        if m == 0 or n == 0 or g in skip:
            continue
        bad = O.tolerance_violations(c, r["c16"], r["s"])
        assert not bad.any(), f"group {g} {shapes[g]}: {int(bad.sum())} elements out of tolerance"


def run_device(shapes, d, tile_config=-1, tables=None):
    tables = dev.device_tables(shapes, d) if tables is None else tables
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    dev.run_device(tables, len(shapes), tile_config=tile_config, status=status)
    torch.cuda.synchronize()
    return int(status.item())


def super_batch_shapes(seed, batches=15, per_batch=8):
    """The super-batch of the pages: the groups of several benchmark calls in
    one launch. Each call here is a MoE-like set of 8 groups with m drawn
    uniformly from [40, 400] (as in the MoE workloads), at sizes the oracle
    finishes quickly: n and k drawn per call."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(batches):
        n = int(rng.choice([128, 256, 520]))
        k = int(rng.choice([128, 256, 512]))
        shapes += [(int(m), n, k, 1) for m in rng.integers(40, 401, size=per_batch)]
    return shapes


@pytest.mark.parametrize("cfg", [-1, 0, 1, 2, 3, 4])
def test_device_tables_match_oracle_and_host_path(cfg):
    """Small workloads, ragged edge cases and a long-K call: oracle parity, and
    bitwise equality with the by-value entry point (whole tiles, same
    configuration) except where that runs the kernels that split K over the
    waves in every tile (long K on 256x128, 128x256 or 128x128 tiles): there
    both are checked against the oracle."""
    cases = [synth.make_workload(0), synth.make_workload(1)]
    edge = [(127, 136, 192, 1), (0, 64, 128, 1), (129, 264, 320, 1), (40, 48, 0, 1), (64, 0, 128, 1),
            (100, 136, 192, 2), (1, 8, 64, 1), (257, 8, 128, 1)]  # at most 8: the by-value limit
    cases.append((edge, synth.make_custom(edge, seed=515)))
    long_k = [(300, 264, 4096, 1), (129, 136, 4160, 1), (33, 72, 4000, 1)]
    cases.append((long_k, synth.make_custom(long_k, seed=516)))
    host_cfg = 0 if cfg < 0 else cfg  # -1: the entry point's default, 256x256 tiles
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for shapes, groups in cases:
        announce(f"device tables cfg={cfg} shapes={shapes}")
        d = dev.upload(shapes, groups, c_guard=GUARD)
        assert run_device(shapes, d, cfg) == 0
        got = [c.copy() for c in dev.c_as_numpy(shapes, d)]
        assert dev.guards_intact(d)
        check_against_oracle(shapes, groups, got)
        h = dev.upload(shapes, groups, c_guard=GUARD)
        dev.run(shapes, h, tile_config=host_cfg, split_mode=0, workspace=None)
        torch.cuda.synchronize()
        host = dev.c_as_numpy(shapes, h)
        if mm.nvfp4_splits_k_over_waves(shapes, cus, host_cfg, 0):
            check_against_oracle(shapes, groups, host)
            continue
        for (m, n, k, l), a, b in zip(shapes, got, host):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (m, n, k, l)


@pytest.mark.parametrize("cfg", [-1, 0])
def test_device_super_batch_120_groups(cfg):
    shapes = super_batch_shapes(seed=120)
    assert len(shapes) == 120
    groups = synth.make_custom(shapes, seed=1201)
    announce(f"super-batch 120 groups cfg={cfg}")
    d = dev.upload(shapes, groups, c_guard=GUARD)
    assert run_device(shapes, d, cfg) == 0
    got = dev.c_as_numpy(shapes, d)
    assert dev.guards_intact(d)
    check_against_oracle(shapes, groups, got)


@pytest.mark.parametrize("cfg", [0, 3])
def test_device_max_groups(cfg):
    """512 groups (the most the entry point takes): small and empty groups,
    k = 0 among them, every row count of a last tile row."""
    G = mm.NVFP4_MAX_DEVICE_GROUPS
    rng = np.random.default_rng(G)
    shapes = [(int(m), int(n), int(k), 1) for m, n, k in zip(rng.integers(0, 300, G),
                                                           rng.choice([8, 16, 24, 136], G),
                                                           rng.choice([0, 64, 128], G))]
    groups = synth.make_custom(shapes, seed=10240)
    announce(f"device tables, {G} groups, cfg {cfg}")
    d = dev.upload(shapes, groups, c_guard=8)
    assert run_device(shapes, d, cfg) == 0
    got = dev.c_as_numpy(shapes, d)
    assert dev.guards_intact(d)
    check_against_oracle(shapes, groups, got)
    for (m, n, k, l), c in zip(shapes, got):
        if k == 0 and m and n:
            assert np.all(c == 0)


def test_device_rejects_bad_groups_and_leaves_their_c():
    """Groups that break a size rule or carry a misaligned address are
    rejected by the kernel: counted in the status word, C untouched. Every bad
    entry here still points into buffers large enough for what it claims, so
    nothing can reach outside them."""
    shapes = [(96, 136, 256, 1)] * 8
    groups = synth.make_custom(shapes, seed=808)
    announce("device tables with rejected groups")
    d = dev.upload(shapes, groups, c_guard=GUARD)
    sizes, abc, sf = dev.device_tables(shapes, d)
    bad = {1: ("size", (96, 136, 240, 1)),        # k % 32
           2: ("size", (96, 132, 256, 1)),        # n % 8
           3: ("size", (96, 136, 256, 0)),        # l = 0
           5: ("abc", 2),                         # C misaligned by 2 bytes (inside its guard band)
           6: ("abc", 0)}                         # A misaligned
    for g, (what, v) in bad.items():
        if what == "size":
            sizes[g] = torch.tensor(v, dtype=torch.int32)
        else:
            abc[g, v] += 2
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev.run_device((sizes, abc, sf), len(shapes), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == len(bad)
    got = dev.c_as_numpy(shapes, d)
    assert dev.guards_intact(d)
    for g in bad:
        assert np.all(got[g].view(np.uint16) == dev.FP16_NAN_BITS), f"rejected group {g} was written"
    check_against_oracle(shapes, groups, got, skip=set(bad))


def test_device_graph_replay_follows_tables():
    """A captured call reads the tables at replay time: replays after the
    tables were rewritten (other sizes, other buffers) compute the new groups."""
    sets = []
    for seed, shapes in ((1, [(200, 264, 320, 1), (64, 136, 128, 1), (0, 64, 64, 1)]),
                         (2, [(33, 520, 192, 1), (300, 72, 256, 1), (129, 8, 64, 1)])):
        groups = synth.make_custom(shapes, seed=seed)
        sets.append((shapes, groups, dev.upload(shapes, groups, c_guard=GUARD)))
    announce("device tables graph replay")
    tables = [dev.device_tables(s, d) for s, _, d in sets]
    live = tuple(t.clone() for t in tables[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.run_device(live, 3, stream=side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dev.run_device(live, 3, stream=side)
    for rep in range(4):
        shapes, groups, d = sets[rep % 2]
        for dst, src in zip(live, tables[rep % 2]):
            dst.copy_(src)
        for dd in d:
            dd["c"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dev.c_as_numpy(shapes, d)
        assert dev.guards_intact(d)
        check_against_oracle(shapes, groups, got)
